"""Decode-sized blocks (every expert in one 32-row m-tile or a few, the tiles
two to a CU): moe_block_forward against the same steps called one by one
through the C ABI (route, permute, gathered gate/up, slot-order down, combine)
-- the same kernels on the same tiles, so the same bits -- and against the
oracle.  The hot-expert cases give one expert two or three m-tiles; three
calls in a row on one workspace give the same bits."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, cfg_of, device_inputs, moe, needs_gpu,
                         oracle_cfg, resolve_routing, to_host, torch, weights_of)

pytestmark = [pytest.mark.gpu, needs_gpu]

CASES = {
    # name: workload, hot expert (bias raised so that it takes every token) or None
    "spread": (synth.Workload(name="spread", N=48, d=1024, E=128, G=1, TG=1, k=8, d_ff=512,
                              route_scale=2.827, seed=21), None),
    "hot_two_mtiles": (synth.Workload(name="hot2", N=64, d=512, E=64, G=1, TG=1, k=8, d_ff=256,
                                      route_scale=2.0, seed=22), 9),
    "hot_three_mtiles_situ": (synth.Workload(name="hot3", N=80, d=768, E=96, G=4, TG=2, k=6,
                                             d_ff=320, act="situ", situ_beta=4.0,
                                             situ_linear_beta=8.0, route_scale=2.5, seed=23), 40),
    "one_token": (synth.Workload(name="one", N=1, d=256, E=16, G=1, TG=1, k=4, d_ff=128,
                                 route_scale=1.0, seed=24), None),
}


def separate_calls(w, dev, cfg):
    """The block's steps one call at a time (no shared expert, no latent)."""
    m = moe()
    N, k, E = w.N, w.k, w.E
    idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((N, k), dtype=torch.float32, device="cuda")
    bias = dev["bias"] if w.use_bias else None
    m.moe_route(cfg, N, dev["hidden"], dev["w_router"], bias, idx, wts,
                m.workspace(cfg, N, m.CALL_ROUTE))
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    offsets = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    perm = torch.empty((N * k,), dtype=torch.int32, device="cuda")
    inv = torch.empty((N * k,), dtype=torch.int32, device="cuda")
    m.moe_permute(cfg, N, idx, None, counts, offsets, perm, inv, None,
                  m.workspace(cfg, N, m.CALL_PERMUTE))
    h = torch.empty((N * k, w.d_ff), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gate_up_gather(cfg, N, dev["hidden"], perm, offsets, dev["w1"], dev["w3"], h,
                                m.workspace(cfg, N, m.CALL_GATE_UP))
    out = torch.empty((N * k, w.d), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_down_scatter(cfg, N, h, offsets, perm, dev["w2"], out,
                              m.workspace(cfg, N, m.CALL_DOWN))
    y = torch.empty((N, w.d), dtype=torch.bfloat16, device="cuda")
    m.moe_combine(cfg, N, out, None, wts, None, y)
    torch.cuda.synchronize()
    return y, idx, wts, counts


@pytest.mark.parametrize("name", list(CASES))
def test_decode_block(name):
    w, hot = CASES[name]
    print(f"decode block parity: {name} N={w.N} d={w.d} E={w.E} k={w.k} d_ff={w.d_ff}",
          flush=True)
    m = moe()
    cfg = cfg_of(w)
    dev = device_inputs(w, on_device_gen=False)
    if hot is not None:
        dev["bias"][hot] = 5.0
    y = torch.full((w.N, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
    cnt = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    m.moe_block_forward(cfg, w.N, weights_of(dev, w), dev["hidden"], y,
                        m.workspace(cfg, w.N, m.CALL_BLOCK), idx, wt, cnt)
    torch.cuda.synchronize()
    if hot is not None:
        assert cnt.cpu().numpy()[hot] == w.N  # w.N / 32 m-tiles for one expert
    y2, idx2, wt2, cnt2 = separate_calls(w, dev, cfg)
    assert torch.equal(idx, idx2) and torch.equal(wt, wt2) and torch.equal(cnt, cnt2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "block != steps one by one"
    x = to_host(dev["hidden"])
    r_idx, r_w, _, _ = resolve_routing(x, to_host(dev["w_router"]), to_host(dev["bias"]), w,
                                       idx.cpu().numpy(), wt.cpu().numpy())
    W = {n: to_host(t) for n, t in dev.items() if n not in ("hidden", "w_router", "bias")}
    y_ref = oracle.block_tokens(oracle_cfg(w), W, x, np.arange(w.N), r_idx, r_w)
    assert_close_bf16(as_f64(to_host(y)), y_ref, name)


def test_repeated_calls_reuse_the_workspace():
    """Three calls in a row on one workspace give the same bits (the tile
    tables and intermediates are rewritten by every call)."""
    w, hot = CASES["hot_two_mtiles"]
    m = moe()
    cfg = cfg_of(w)
    dev = device_inputs(w, on_device_gen=False)
    dev["bias"][hot] = 5.0
    ws = m.workspace(cfg, w.N, m.CALL_BLOCK)
    ys = []
    for _ in range(3):
        y = torch.empty((w.N, w.d), dtype=torch.bfloat16, device="cuda")
        m.moe_block_forward(cfg, w.N, weights_of(dev, w), dev["hidden"], y, ws)
        ys.append(y)
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0].view(torch.int16), t.view(torch.int16)) for t in ys[1:])
