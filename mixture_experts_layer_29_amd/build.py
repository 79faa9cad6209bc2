"""Builds libmoe.so in place: every HIP source compiled for gfx950 with hipcc,
then linked into one shared library next to this file.

Every kernel's register and scratch use is read from the compiler's
resource-usage remarks and written to _build/resource_usage.json; the build
fails if any kernel keeps values in scratch memory (register spills), which
would put per-lane memory traffic into the hot loops."""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
BUILD = os.path.join(_HERE, "_build")
LIB = os.path.join(_HERE, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "route.hip", "permute.hip", "gemm_bf16.hip", "gemm_dense.hip",
           "gemm_f32.hip", "combine.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(_HERE), "include")]


REPORT = os.path.join(BUILD, "resource_usage.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
         "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_usage(text: str) -> dict:
    """{kernel symbol: {vgprs, agprs, scratch_bytes, waves_per_simd, lds_bytes}} from
    hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for key, val in _REMARK.findall(text):
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, parse_resource_usage(r.stderr)


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    usage = {k: v for _, u in done for k, v in u.items()}
    with open(REPORT, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    spills = {k: v["scratch_bytes"] for k, v in usage.items() if v.get("scratch_bytes", 0)}
    if spills:
        raise RuntimeError("kernels using scratch memory (register spills), bytes per lane: "
                           + ", ".join(f"{k}: {v}" for k, v in sorted(spills.items())))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
