"""The seeded input generator: known answers, transform accuracy, determinism.

The generator holds none of the method; these tests pin it to its published
definitions (Philox4x32-10 known-answer vectors; Box-Muller pieces against
the mathematics) so that the workloads' inputs are what the recipes say."""
import math

import numpy as np
import pytest

import synth


# Known-answer vectors for Philox4x32 with 10 rounds, as published with the
# Random123 library of Salmon et al. (kat_vectors).
@pytest.mark.parametrize("ctr,key,expect", [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, expect):
    assert synth.philox4x32_10(ctr, key) == expect


def test_log_sqrt_pieces_match_math():
    lib = synth._load_host()
    rng = np.random.default_rng(1)
    for a in list(rng.integers(0, 2**32, 2000)) + [0, 1, 2**31, 2**32 - 2, 2**32 - 1]:
        a = int(a)
        got = lib.synth_log_u1_host(a)
        want = math.log((a + 1) / 2.0**32)
        assert abs(got - want) <= 4e-16 * max(1.0, abs(want))
    for v in list(rng.uniform(0, 50, 2000)) + [1e-10, 1.0, 4.0, 44.3614]:
        assert abs(lib.synth_sqrt_host(float(v)) - math.sqrt(v)) <= 2.3e-16 * math.sqrt(v)


def test_box_muller_pairs_match_math():
    import ctypes

    lib = synth._load_host()
    rng = np.random.default_rng(2)
    z0, z1 = ctypes.c_double(), ctypes.c_double()
    for a, b in rng.integers(0, 2**32, (2000, 2)):
        lib.synth_box_muller_host(int(a), int(b), ctypes.byref(z0), ctypes.byref(z1))
        rho = math.sqrt(-2.0 * math.log((int(a) + 1) / 2.0**32))
        th = 2.0 * math.pi * int(b) / 2.0**32
        assert abs(z0.value - rho * math.cos(th)) <= 1e-14 * max(1.0, rho)
        assert abs(z1.value - rho * math.sin(th)) <= 1e-14 * max(1.0, rho)


def test_normal_moments_and_subranges():
    n = 1 << 22
    a = synth.fill_normal_host(n, 0, 0, 1, 1.0, synth.F32)
    assert abs(a.mean()) < 3e-3 and abs(a.std() - 1.0) < 3e-3
    assert abs((a.astype(np.float64) ** 4).mean() - 3.0) < 0.03
    # any sub-range regenerates the same elements (counter-based)
    for first, cnt in [(0, 5), (3, 17), (12345, 1000), (n - 7, 7)]:
        b = synth.fill_normal_host(cnt, first, 0, 1, 1.0, synth.F32)
        assert np.array_equal(b, a[first:first + cnt])
    # other seeds / tensor ids give other streams
    c = synth.fill_normal_host(1000, 0, 1, 1, 1.0, synth.F32)
    d = synth.fill_normal_host(1000, 0, 0, 2, 1.0, synth.F32)
    assert not np.array_equal(c, a[:1000]) and not np.array_equal(d, a[:1000])


def test_bf16_is_rounded_f32():
    f = synth.fill_normal_host(4096, 100, 0, 4, 0.05, synth.F32)
    h = synth.fill_normal_host(4096, 100, 0, 4, 0.05, synth.BF16)
    assert np.array_equal(h, synth.f32_to_bf16_bits(f))
    back = synth.bf16_bits_to_f32(h)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2.0**-8)


def test_expert_slices_are_rows_of_the_stacked_tensor():
    w = synth.WORKLOADS["tiny"]
    full = synth.host_tensor(w, "w1")
    for e in (0, 7, w.E - 1):
        assert np.array_equal(synth.host_tensor(w, "w1", expert=e), full[e])


def test_recipe_stdevs():
    w = synth.WORKLOADS["dsv3_prefill"]
    wr = synth.host_tensor(w, "w_router").astype(np.float64)
    assert abs(wr.var() * w.d - 1.0) < 0.01  # variance 1/d: logits ~ N(0, 1)
    b = synth.host_tensor(w, "bias")
    assert b.dtype == np.float32 and abs(b.std() - 0.01) < 0.002
    w1 = synth.bf16_bits_to_f32(synth.host_tensor(w, "w1", expert=3)).astype(np.float64)
    assert abs(w1.var() * w.d_in - 1.0) < 0.01


def test_zipf_profile():
    E = 896
    b = synth.zipf_bias(E, 0)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    want = np.sort((0.25 * ranks ** -1.1).astype(np.float32))
    assert np.array_equal(np.sort(b), want)
    assert not np.array_equal(b, (0.25 * ranks ** -1.1).astype(np.float32))  # shuffled
    assert np.array_equal(b, synth.zipf_bias(E, 0))


def test_workload_sizes_match_page_shapes():
    """Every size the pages print (tests/golden/page_shapes.json, each with its
    citation) is the size of the workloads built on it."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")
    facts = json.load(open(path))["facts"]
    assert facts
    for f in facts:
        for name in f["workloads"]:
            assert getattr(synth.WORKLOADS[name], f["field"]) == f["value"], (name, f["what"])
