"""moe_block_forward against the oracle on every token of small blocks: the tiny
fp32 workload, bf16 twins with a shared expert, groups, the latent projection
with its norm and SiTU experts, a hot expert, N = 1; determinism; N = 0."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, assert_close_f32, cfg_of, device_inputs, moe,
                         needs_gpu, oracle_cfg, resolve_routing, to_host, torch, weights_of)

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_block(w, dev, with_outputs=True):
    m = moe()
    cfg = cfg_of(w)
    ydt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float32
    y = torch.full((w.N, w.d), float("nan"), dtype=ydt, device="cuda")
    idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda") if with_outputs else None
    wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda") if with_outputs else None
    cnt = torch.empty((w.E,), dtype=torch.int32, device="cuda") if with_outputs else None
    ws = m.workspace(cfg, w.N, m.CALL_BLOCK)
    m.moe_block_forward(cfg, w.N, weights_of(dev, w), dev["hidden"], y, ws, idx, wt, cnt)
    torch.cuda.synchronize()
    return y, idx, wt, cnt


def host_weights(dev):
    return {n: to_host(t) for n, t in dev.items() if n not in ("hidden", "w_router", "bias")}


def check_block(w):
    print(f"block parity: {w.name} N={w.N} d={w.d} E={w.E} k={w.k} L={w.L} d_sh={w.d_sh} "
          f"act={w.act} dtype={w.dtype}", flush=True)
    dev = device_inputs(w, on_device_gen=False)
    y, idx, wt, cnt = run_block(w, dev)
    x = to_host(dev["hidden"])
    r_idx, r_w, flags, _ = resolve_routing(x, to_host(dev["w_router"]), to_host(dev["bias"]), w,
                                           idx.cpu().numpy(), wt.cpu().numpy())
    counts, _, _, _ = oracle.counts_perm(r_idx, w.E)
    assert np.array_equal(cnt.cpu().numpy(), counts)
    y_ref = oracle.block_tokens(oracle_cfg(w), host_weights(dev), x, np.arange(w.N), r_idx, r_w)
    got = as_f64(to_host(y))
    assert np.all(np.isfinite(got))
    if w.dtype == synth.BF16:
        # softmax routing without renormalisation: |y| reaches ~14 rms, where
        # bf16 storage of y alone exceeds the max-error bar (see the helper)
        return assert_close_bf16(got, y_ref, w.name,
                                 output_rounding_slack=(w.score_func == "softmax"
                                                        and not w.norm_topk_prob))
    return assert_close_f32(got, y_ref, w.name)


TINY = synth.WORKLOADS["tiny"]
VARIANTS = {
    "tiny": TINY,
    "tiny_bf16": TINY.scaled(dtype=synth.BF16),
    "tiny_shared": TINY.scaled(d_sh=64),
    "groups_bf16": synth.Workload(name="groups_bf16", N=300, d=512, E=64, G=8, TG=3, k=6,
                                  d_ff=128, route_scale=2.5, seed=4),
    "k2_like_shared": synth.Workload(name="k2_like_shared", N=513, d=1024, E=48, G=1, TG=1, k=8,
                                     d_ff=256, d_sh=256, route_scale=2.827, seed=5),
    "k3_like_latent": synth.Workload(name="k3_like_latent", N=200, d=1024, E=96, G=1, TG=1, k=8,
                                     d_ff=384, d_sh=384, L=512, act="situ", situ_beta=4.0,
                                     situ_linear_beta=8.0, bias_kind="zipf",
                                     route_scale=2.827, seed=6),
    "latent_no_norm_fp32": synth.Workload(name="latent_no_norm_fp32", N=50, d=128, E=16, G=2,
                                          TG=1, k=3, d_ff=64, L=64, latent_norm=False,
                                          route_scale=1.5, dtype=synth.F32, seed=7),
    "ragged_bf16": synth.Workload(name="ragged_bf16", N=77, d=200, E=24, G=3, TG=2, k=5,
                                  d_ff=72, d_sh=40, route_scale=1.0, seed=8),
    "one_token": TINY.scaled(N=1, dtype=synth.BF16),
    "decode_like": synth.Workload(name="decode_like", N=32, d=2048, E=384, G=1, TG=1, k=8,
                                  d_ff=256, d_sh=256, route_scale=2.827, seed=9),
    # DeepSeek-V3.2-Exp gate forms: softmax scoring (no renormalisation) and a
    # router without a bias (groups scored by their largest choice)
    "softmax_groups_bf16": synth.Workload(name="softmax_groups_bf16", N=300, d=512, E=64, G=8,
                                          TG=3, k=6, d_ff=128, route_scale=2.5, seed=11,
                                          score_func="softmax", norm_topk_prob=False),
    "nobias_groups_bf16": synth.Workload(name="nobias_groups_bf16", N=300, d=512, E=64, G=8,
                                         TG=3, k=6, d_ff=128, route_scale=2.5, seed=12,
                                         use_bias=False),
    "softmax_nobias_fp32": TINY.scaled(name="softmax_nobias_fp32", score_func="softmax",
                                       use_bias=False, seed=13),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_block(name):
    check_block(VARIANTS[name])


def test_hot_expert_takes_every_token():
    w = synth.Workload(name="hot", N=400, d=256, E=32, G=1, TG=1, k=4, d_ff=128,
                       route_scale=2.0, seed=10)
    dev = device_inputs(w, on_device_gen=False)
    dev["bias"][9] = 5.0
    y, idx, wt, cnt = run_block(w, dev)
    assert cnt.cpu().numpy()[9] == w.N
    x = to_host(dev["hidden"])
    b = to_host(dev["bias"])
    r_idx, r_w, _, _ = resolve_routing(x, to_host(dev["w_router"]), b, w, idx.cpu().numpy(),
                                       wt.cpu().numpy())
    y_ref = oracle.block_tokens(oracle_cfg(w), host_weights(dev), x, np.arange(w.N), r_idx, r_w)
    assert_close_bf16(as_f64(to_host(y)), y_ref, "hot")


def test_deterministic():
    w = VARIANTS["k2_like_shared"]
    dev = device_inputs(w, on_device_gen=False)
    y1, i1, w1, c1 = run_block(w, dev)
    y2, i2, w2, c2 = run_block(w, dev, with_outputs=False)
    y3, i3, w3, c3 = run_block(w, dev)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert torch.equal(i1, i3) and torch.equal(w1, w3) and torch.equal(c1, c3)


def test_zero_tokens():
    m = moe()
    w = TINY
    m.moe_block_forward(cfg_of(w), 0, m.Weights(None, None, None, None, None), None, None, None)
