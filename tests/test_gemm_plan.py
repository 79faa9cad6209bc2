"""Host check of the grouped GEMM's streaming plan (csrc/gemm_plan.h).

gemm_plan_sim.cpp replays one wave's loads, vmcnt waits, barriers and LDS reads
in the kernel's program order, for every tile height (1..8 row blocks), both
wave layouts, the whole-CU and the half-CU LDS plans (two work-groups per CU,
up to 4 row blocks) and K lengths from 1 to 112 blocks, and checks that every wait
lets through only loads younger than the ones its sub-iteration reads, that
no stage is refilled before its last read (or, for stages several waves
read, before a barrier after it), and that the counts are tight.  A plan
whose wait ignores the activation loads must fail the same check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_29_amd", "csrc")
SIM = os.path.join(ROOT, "tests", "gemm_plan_sim.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build_and_run(include_dir, out):
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", include_dir, SIM, "-o", out],
                   check=True, capture_output=True, text=True)
    return subprocess.run([out], capture_output=True, text=True)


def test_wait_counts_and_stage_reuse(tmp_path):
    r = _build_and_run(CSRC, str(tmp_path / "sim"))
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:]


def test_simulation_rejects_a_wait_that_ignores_the_activations(tmp_path):
    src = open(os.path.join(CSRC, "gemm_plan.h")).read()
    line = "    if (ka > newest) newest = ka;"
    assert line in src
    (tmp_path / "gemm_plan.h").write_text(src.replace(line, "    (void)ka;"))
    r = _build_and_run(str(tmp_path), str(tmp_path / "sim_bad"))
    assert r.returncode != 0 and "activations not landed" in r.stdout
