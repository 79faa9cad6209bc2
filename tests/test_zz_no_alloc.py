"""moe_permute_static, the dispatch entry point that allocates nothing, against
moe_permute (the same call with a caller workspace): bit-identical counts,
offsets, permutation, inverse and sorted rows, on two calls in a row, the
second with a smaller input (the static scratch keeps the first call's
contents), through the C ABI; and the size limit, refused on the host."""
import ctypes

import numpy as np
import pytest

import mixture_experts_layer_29_amd as m
from mixture_experts_layer_29_amd import binding
from moe_testlib import needs_gpu, to_host, torch


def routing(rng, N, E, k):
    return np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(N)]), axis=1).astype(
        np.int32)


def permute_both(cfg, N, idx, x):
    E, k = cfg.n_experts, cfg.top_k
    outs = []
    for static in (False, True):
        o = dict(cnt=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                 off=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                 perm=torch.full((N * k,), -7, dtype=torch.int32, device="cuda"),
                 inv=torch.full((N * k,), -7, dtype=torch.int32, device="cuda"),
                 xs=torch.zeros((N * k, x.shape[1]), dtype=x.dtype, device="cuda"))
        if static:
            m.moe_permute_static(cfg, N, idx, x, o["cnt"], o["off"], o["perm"], o["inv"], o["xs"])
        else:
            m.moe_permute(cfg, N, idx, x, o["cnt"], o["off"], o["perm"], o["inv"], o["xs"],
                          m.workspace(cfg, N, m.CALL_PERMUTE))
        torch.cuda.synchronize()
        outs.append({n: to_host(t) for n, t in o.items()})
    return outs


@pytest.mark.gpu
@needs_gpu
def test_static_scratch_permute_matches_workspace_permute():
    rng = np.random.default_rng(29)
    E, k, d = 384, 8, 256
    cfg = m.make_config(d=d, n_experts=E, n_group=1, topk_group=1, top_k=k, d_ff=128,
                        route_scale=1.0, dtype=m.DTYPE_BF16)
    for N in (8192, 1000):  # the second call is smaller than the first
        print(f"static-scratch permute: N={N} E={E} k={k}", flush=True)
        idx = torch.from_numpy(routing(rng, N, E, k)).cuda()
        x = torch.randn((N, d), generator=torch.Generator().manual_seed(N)).to(
            torch.bfloat16).cuda()
        ref, got = permute_both(cfg, N, idx, x)
        for name in ref:
            assert np.array_equal(ref[name], got[name]), name
        assert ref["off"][-1] == N * k
        assert np.array_equal(np.sort(got["perm"]), np.arange(N * k))


def test_static_scratch_size_limit_refused_on_host():
    c = m.make_config(d=256, n_experts=1024, n_group=1, topk_group=1, top_k=8, d_ff=128,
                      route_scale=1.0, dtype=m.DTYPE_BF16)
    fake = 1 << 20
    N = 65536  # ceil(N/64) * E * 12 bytes = 12 MiB > the static scratch
    st = binding.lib().moe_permute_static(ctypes.byref(c), N, fake, None, fake, fake, fake, fake,
                                         None, None)
    assert st == binding.MOE_ERR_UNSUPPORTED
    assert "static scratch" in binding.last_error()
