"""Compile tests/native/host_checks.cpp with g++ into tests/native/libbsm_host_checks.so."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    out = os.path.join(HERE, "libbsm_host_checks.so")
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(HERE, "host_checks.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
