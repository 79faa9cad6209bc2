"""moe_route against the oracle: indices identical (near ties re-checked with the
GPU's indices), weights within 1e-5 relative, over the tiny workload, its bf16
twin and a sweep of expert counts, group shapes, top-k and token counts."""
import numpy as np
import pytest

import synth
from moe_testlib import cfg_of, device_inputs, moe, needs_gpu, resolve_routing, to_host, torch

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_route(w, dev):
    m = moe()
    cfg = cfg_of(w)
    idx = torch.full((w.N, w.k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((w.N, w.k), -7.0, dtype=torch.float32, device="cuda")
    ws = m.workspace(cfg, w.N, m.CALL_ROUTE)
    m.moe_route(cfg, w.N, dev["hidden"], dev["w_router"], dev["bias"] if w.use_bias else None,
                idx, wt, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), wt.cpu().numpy()


def check(w):
    print(f"route parity: {w.name} N={w.N} E={w.E} G={w.G} TG={w.TG} k={w.k} dtype={w.dtype} "
          f"score={w.score_func} bias={w.use_bias}", flush=True)
    dev = device_inputs(w, on_device_gen=False)
    gi, gw = run_route(w, dev)
    x = to_host(dev["hidden"])
    wr = to_host(dev["w_router"])
    b = to_host(dev["bias"])
    _, _, flags, n_res = resolve_routing(x, wr, b, w, gi, gw)
    assert np.all(np.diff(gi, axis=1) > 0)  # ascending, distinct
    return n_res


def test_tiny_fp32():
    check(synth.WORKLOADS["tiny"])


def test_tiny_bf16():
    check(synth.WORKLOADS["tiny"].scaled(dtype=synth.BF16))


SWEEP = [
    # N, d, E, G, TG, k, bias_std
    (1, 64, 8, 1, 1, 1, 0.01),
    (3, 128, 8, 2, 1, 2, 0.01),
    (64, 256, 16, 4, 2, 4, 0.1),
    (1000, 512, 64, 8, 3, 8, 0.01),
    (257, 520, 256, 8, 4, 8, 0.01),
    (200, 1024, 384, 1, 1, 8, 0.01),
    (130, 1024, 896, 1, 1, 8, 0.01),
    (77, 256, 1024, 16, 4, 16, 0.05),
    (50, 256, 96, 48, 7, 5, 0.01),
]


@pytest.mark.parametrize("N,d,E,G,TG,k,bstd", SWEEP)
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_sweep(N, d, E, G, TG, k, bstd, dtype):
    w = synth.Workload(name="sweep", N=N, d=d, E=E, G=G, TG=TG, k=k, d_ff=64,
                       route_scale=1.7, dtype=dtype, bias_std=bstd, seed=N + E)
    check(w)


def test_dominant_bias_and_no_renorm():
    w = synth.Workload(name="bias", N=300, d=256, E=64, G=4, TG=2, k=6, d_ff=64,
                       route_scale=2.0, dtype=synth.BF16, seed=3)
    dev = device_inputs(w, on_device_gen=False)
    dev["bias"][17] = 10.0
    gi, gw = run_route(w, dev)
    assert np.all(np.any(gi == 17, axis=1))
    w1 = w.scaled(norm_topk_prob=False)
    m = moe()
    cfg = cfg_of(w1)
    idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
    m.moe_route(cfg, w.N, dev["hidden"], dev["w_router"], dev["bias"], idx, wt,
                m.workspace(cfg, w.N, m.CALL_ROUTE))
    torch.cuda.synchronize()
    resolve_routing(to_host(dev["hidden"]), to_host(dev["w_router"]), to_host(dev["bias"]), w1,
                    idx.cpu().numpy(), wt.cpu().numpy())


def test_zero_tokens_is_noop():
    w = synth.WORKLOADS["tiny"]
    m = moe()
    cfg = cfg_of(w)
    m.moe_route(cfg, 0, None, None, None, None, None, None)


# Router forms of the DeepSeek-V3.2-Exp gate: softmax scoring, and routers
# without a bias (groups scored by their largest choice).
FORMS = [("softmax", True), ("sigmoid", False), ("softmax", False)]


@pytest.mark.parametrize("score_func,use_bias", FORMS)
@pytest.mark.parametrize("N,d,E,G,TG,k,bstd", [SWEEP[0], SWEEP[2], SWEEP[3], SWEEP[4], SWEEP[6],
                                                SWEEP[7], SWEEP[8]])
def test_router_forms(N, d, E, G, TG, k, bstd, score_func, use_bias):
    w = synth.Workload(name="form", N=N, d=d, E=E, G=G, TG=TG, k=k, d_ff=64, route_scale=1.7,
                       dtype=synth.BF16, bias_std=bstd, seed=N + E + 1, score_func=score_func,
                       use_bias=use_bias, norm_topk_prob=(score_func == "sigmoid"))
    check(w)
