"""Builds the oracle's shared library (plain C, gcc) in place.

Test infrastructure only: the oracle is the CPU reference the GPU library is
checked against."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    out = os.path.join(_HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", out + ".tmp",
           os.path.join(_HERE, "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build()
