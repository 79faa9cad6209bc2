"""The four full-size workloads, in the launch configuration the benchmark times.

Routing is checked on every token (indices identical up to near ties, weights
to 1e-5), the per-expert counts and the dispatch permutation bit-exactly, and
the block output on a seeded sample of tokens that the oracle computes one by
one from regenerated host copies of exactly the weights those tokens touch."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, cfg_of, device_inputs, moe, needs_gpu,
                         oracle_cfg, resolve_routing, to_host, torch, weights_of)

pytestmark = [pytest.mark.gpu, needs_gpu]

SAMPLE_TOKENS = 6


def sampled_tokens(w, n):
    rng = np.random.default_rng(1234)
    mid = rng.choice(np.arange(1, w.N - 1), n - 2, replace=False)
    return np.sort(np.concatenate([[0, w.N - 1], mid])).astype(np.int64)


@pytest.mark.parametrize("name", ["dsv3_prefill", "k2_prefill", "k2_decode", "k3_latent_prefill"])
def test_full_workload(name):
    w = synth.WORKLOADS[name]
    print(f"full workload parity: {name} N={w.N} E={w.E}", flush=True)
    m = moe()
    cfg = cfg_of(w)
    dev = device_inputs(w, on_device_gen=True)
    y = torch.empty((w.N, w.d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
    cnt = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    ws = m.workspace(cfg, w.N, m.CALL_BLOCK)
    m.moe_block_forward(cfg, w.N, weights_of(dev, w), dev["hidden"], y, ws, idx, wt, cnt)
    torch.cuda.synchronize()

    # routing on every token, against host copies from the host generator
    x = synth.host_tensor(w, "hidden")
    wr = synth.host_tensor(w, "w_router")
    bias = synth.host_tensor(w, "bias")
    g_idx = idx.cpu().numpy()
    r_idx, r_w, flags, n_res = resolve_routing(x, wr, bias, w, g_idx, wt.cpu().numpy())
    print(f"  near-tie tokens resolved with the GPU's choice: {n_res}", flush=True)
    counts, offsets, perm, inv = oracle.counts_perm(r_idx, w.E)
    assert np.array_equal(cnt.cpu().numpy(), counts)

    # the dispatch permutation on the GPU's routing
    perm_d = torch.empty(w.N * w.k, dtype=torch.int32, device="cuda")
    inv_d = torch.empty_like(perm_d)
    offs_d = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    cnt_d = torch.empty(w.E, dtype=torch.int32, device="cuda")
    m.moe_permute(cfg, w.N, idx, None, cnt_d, offs_d, perm_d, inv_d, None,
                  m.workspace(cfg, w.N, m.CALL_PERMUTE))
    torch.cuda.synchronize()
    assert np.array_equal(perm_d.cpu().numpy(), perm)
    assert np.array_equal(inv_d.cpu().numpy(), inv)
    assert np.array_equal(offs_d.cpu().numpy(), offsets)

    # block output on sampled tokens
    toks = sampled_tokens(w, SAMPLE_TOKENS)
    need = sorted({int(e) for t in toks for e in r_idx[t]})
    W = {n: {e: synth.host_tensor(w, n, expert=e) for e in need} for n in ("w1", "w3", "w2")}
    for n in ("sh_w1", "sh_w3", "sh_w2", "w_down", "w_up", "gamma"):
        if n in w.shapes():
            W[n] = synth.host_tensor(w, n)
    y_ref = oracle.block_tokens(oracle_cfg(w), W, x, toks, r_idx[toks], r_w[toks])
    got = as_f64(to_host(y)[toks])
    r, m_rel = assert_close_bf16(got, y_ref, name)
    print(f"  sampled y: rel L2 {r:.2e}, max err / rms {m_rel:.2e}", flush=True)
    assert np.all(np.isfinite(as_f64(to_host(y))))
