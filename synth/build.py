"""Builds the two fillers of the synthetic-input generator, in place."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_host() -> str:
    out = os.path.join(_HERE, "libsynth_host.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wno-unknown-pragmas", "-o", out + ".tmp", os.path.join(_HERE, "synth_host.c")]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_dev() -> str:
    out = os.path.join(_HERE, "libsynth_dev.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", out + ".tmp", os.path.join(_HERE, "synth_dev.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for synth_dev.hip:\n" + r.stderr)
    os.replace(out + ".tmp", out)
    return out


def build() -> None:
    build_host()
    build_dev()


if __name__ == "__main__":
    build()
