"""Build the oracle's C quantizers: ``python -m oracle.build_c``.

TEST INFRASTRUCTURE ONLY.  Produces ``oracle/liboracle_quant.so`` from
``oracle/quant_c.c`` with gcc: binary32 arithmetic on SSE (no x87 excess
precision), no fast-math, no floating-point contraction, OpenMP over rows.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_quant.so")
CMD = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-mfpmath=sse", "-msse2", "-fopenmp",
       "-shared", "-fPIC", os.path.join(HERE, "quant_c.c"), "-o"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    r = subprocess.run(CMD + [tmp, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed building liboracle_quant.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
