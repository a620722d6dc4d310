"""Build the gfx950 HIP library in-tree: ``python -m block_scaled_fp4_sigmoid_amd.build``.

Produces ``block_scaled_fp4_sigmoid_amd/libbsmoe.so`` (hipcc, --offload-arch=gfx950).
Flags: -ffp-contract=off (every expression rounds where written), IEEE
denormals kept, packed FP32 instructions disabled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["bsm_abi.hip", "bsm_quant.hip", "bsm_route.hip", "bsm_moe.hip", "bsm_ceil.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build_library(verbose=False):
    out = os.path.join(HERE, "libbsmoe.so")
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + [os.path.join(HERE, "csrc", s) for s in SOURCES] + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libbsmoe.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
