"""The routed-expert GEMMs at every tile height, with many tiles per CU.

moe_expert_gate_up, moe_expert_gate_up_gather and moe_expert_down on widths
of 576..1152 (K from 9 blocks of 64), sized to select each tile height (32,
64, 128 and 256 rows; 4 and 8 waves) with thousands of tiles, so every CU runs
several tiles of different heights; with empty experts, experts spread over
several m-tiles (whose weights are loaded through the cache, while single-tile
experts load theirs non-temporal), and both forms of the gate/up input
(gathered through the permutation, and already in expert order, which must
give the same bits).  Every row is compared with the oracle's per-row expert
halves."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, cfg_of, moe, needs_gpu, oracle_cfg,
                         to_device, to_host, torch)

pytestmark = [pytest.mark.gpu, needs_gpu]


def routing(rng, N, E, k, hot=(), empty=()):
    """k distinct experts per token, the `hot` ones chosen by every token."""
    allowed = [e for e in range(E) if e not in empty and e not in hot]
    rows = [np.concatenate([list(hot), rng.choice(allowed, k - len(hot), replace=False)])
            for _ in range(N)]
    return np.sort(np.array(rows, np.int32), axis=1)


CASES = [
    # name, N, E, k, d_in, d_ff, act, hot, empty
    # ~8 rows per expert: 32-row tiles, 8 gate/up tiles per expert, ~8 tiles per work-group
    ("rb1_many_tiles", 512, 256, 4, 1024, 1024, "silu", (), (3, 200)),
    # ~16 rows: 64-row tiles
    ("rb2", 256, 64, 4, 768, 1152, "situ", (), (7,)),
    # ~16 rows, down with K = 576 (9 blocks, the shortest streamed K)
    ("rb2_k9_down", 256, 64, 4, 1024, 576, "silu", (), ()),
    # ~40 rows: 128-row tiles; one hot expert spans 5 m-tiles; gate/up K = 576
    ("rb4_hot", 640, 64, 4, 576, 1152, "silu", (5,), (9,)),
    ("rb4_situ", 640, 64, 4, 768, 1152, "situ", (), ()),
    # ~100 rows: 256-row tiles, 8 waves for gate/up, 4 for down
    ("rb8", 800, 32, 4, 1024, 1152, "silu", (), (1,)),
    # ~180 rows: 256-row tiles, 8 waves for both
    ("rb8_w8_down", 720, 16, 4, 1024, 640, "silu", (0,), ()),
]


def _workload(N, E, k, d_in, d_ff, act):
    return synth.Workload(name="tiles", N=N, d=d_in, E=E, G=1, TG=1, k=k, d_ff=d_ff,
                          route_scale=1.0, act=act, situ_beta=4.0 if act == "situ" else 1.0,
                          situ_linear_beta=8.0 if act == "situ" else 0.0, dtype=synth.BF16,
                          seed=E + d_ff)


@pytest.mark.parametrize("name,N,E,k,d_in,d_ff,act,hot,empty", CASES)
def test_gate_up_and_down_tile_heights(name, N, E, k, d_in, d_ff, act, hot, empty):
    print(f"expert tile heights parity: {name}", flush=True)
    rng = np.random.default_rng(len(name) * 7 + N)
    m = moe()
    w = _workload(N, E, k, d_in, d_ff, act)
    cfg = cfg_of(w)
    idx = routing(rng, N, E, k, hot, empty)
    counts, offsets, perm, _ = oracle.counts_perm(idx, E)
    erow = np.repeat(np.arange(E, dtype=np.int32), counts)
    S = N * k
    x = synth.fill_normal_host(N * d_in, 0, 21, 1, 1.0, synth.BF16).reshape(N, d_in)
    W = {n: synth.host_tensor(w, n) for n in ("w1", "w3", "w2")}
    dW = {n: to_device(a, True) for n, a in W.items()}
    doffs = torch.from_numpy(offsets).cuda()
    ocfg = oracle_cfg(w)
    x_rows = x[perm // k]
    h_ref = oracle.gate_up_rows(ocfg, W["w1"], W["w3"], x_rows, erow)

    # gathered rows (the block's form) and rows already in expert order
    h = torch.empty((S, d_ff), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gate_up_gather(cfg, N, to_device(x, True), torch.from_numpy(perm).cuda(), doffs,
                                dW["w1"], dW["w3"], h, m.workspace(cfg, N, m.CALL_GATE_UP))
    h2 = torch.empty_like(h)
    m.moe_expert_gate_up(cfg, N, to_device(x_rows, True), doffs, dW["w1"], dW["w3"], h2,
                         m.workspace(cfg, N, m.CALL_GATE_UP))
    torch.cuda.synchronize()
    got = to_host(h)
    assert np.array_equal(got, to_host(h2)), "gathered and sorted inputs give different h"
    assert_close_bf16(as_f64(got), h_ref, f"{name} gate/up", output_rounding_slack=True)

    hin = synth.fill_normal_host(S * d_ff, 0, 22, 1, 0.5, synth.BF16).reshape(S, d_ff)
    out = torch.empty((S, d_in), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_down(cfg, N, to_device(hin, True), doffs, dW["w2"], out,
                      m.workspace(cfg, N, m.CALL_DOWN))
    torch.cuda.synchronize()
    o_ref = oracle.down_rows(ocfg, W["w2"], hin, erow)
    assert_close_bf16(as_f64(to_host(out)), o_ref, f"{name} down")


def test_output_rows_outside_segments_untouched():
    """Rows past expert_offsets[E] (a caller may pass a shorter table) are not written."""
    m = moe()
    N, E, k, d_in, d_ff = 256, 64, 4, 768, 640
    w = _workload(N, E, k, d_in, d_ff, "silu")
    cfg = cfg_of(w)
    rng = np.random.default_rng(5)
    idx = routing(rng, N, E, k)
    counts, offsets, perm, _ = oracle.counts_perm(idx, E)
    # the last expert's rows are dropped from the table
    offsets = offsets.copy()
    offsets[E] = offsets[E - 1]
    S = N * k
    W = {n: synth.host_tensor(w, n) for n in ("w1", "w3")}
    x = synth.fill_normal_host(S * d_in, 0, 23, 1, 1.0, synth.BF16).reshape(S, d_in)
    h = torch.full((S, d_ff), 7.0, dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gate_up(cfg, N, to_device(x, True), torch.from_numpy(offsets).cuda(),
                         to_device(W["w1"], True), to_device(W["w3"], True), h,
                         m.workspace(cfg, N, m.CALL_GATE_UP))
    torch.cuda.synchronize()
    tail = as_f64(to_host(h[int(offsets[E]):]))
    assert np.all(tail == 7.0)
