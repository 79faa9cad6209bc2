"""moe_permute against the oracle: counts, offsets, permutation and its inverse
bit-exact, gathered rows bit-exact; ragged token counts, empty experts and one
expert holding every token."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import cfg_of, moe, needs_gpu, to_device, to_host, torch

pytestmark = [pytest.mark.gpu, needs_gpu]


def routing(rng, N, E, k, hot=None):
    rows = []
    for _ in range(N):
        if hot is not None:
            rest = rng.choice([e for e in range(E) if e != hot], k - 1, replace=False)
            rows.append(np.sort(np.concatenate([[hot], rest])))
        else:
            rows.append(np.sort(rng.choice(E, k, replace=False)))
    return np.array(rows, np.int32).reshape(N, k)


CASES = [(1, 8, 2, None), (63, 16, 4, None), (64, 16, 4, None), (65, 16, 4, None),
         (1000, 64, 8, None), (4097, 384, 8, None), (300, 1024, 16, None), (500, 32, 4, 5),
         (129, 896, 8, None)]


@pytest.mark.parametrize("N,E,k,hot", CASES)
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_permute(N, E, k, hot, dtype):
    print(f"permute parity: N={N} E={E} k={k} hot={hot} dtype={dtype}", flush=True)
    rng = np.random.default_rng(N * 7 + E)
    m = moe()
    d = 40
    w = synth.Workload(name="perm", N=N, d=d, E=E, G=1, TG=1, k=k, d_ff=8, route_scale=1.0,
                       dtype=dtype)
    cfg = cfg_of(w)
    idx = routing(rng, N, E, k, hot)
    x = synth.fill_normal_host(N * d, 0, 1, 1, 1.0, dtype).reshape(N, d)
    dx = to_device(x, dtype == synth.BF16)
    didx = torch.from_numpy(idx).cuda()
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    offs = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    perm = torch.full((N * k,), -1, dtype=torch.int32, device="cuda")
    inv = torch.full((N * k,), -1, dtype=torch.int32, device="cuda")
    xs = torch.empty((N * k, d), dtype=dx.dtype, device="cuda")
    ws = m.workspace(cfg, N, m.CALL_PERMUTE)
    m.moe_permute(cfg, N, didx, dx, counts, offs, perm, inv, xs, ws)
    torch.cuda.synchronize()
    c, o, p, ip = oracle.counts_perm(idx, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offs.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p)
    assert np.array_equal(inv.cpu().numpy(), ip)
    assert np.array_equal(to_host(xs), x[p // k])
    if hot is not None:
        assert c[hot] == N


def test_permute_without_gather_and_zero_tokens():
    m = moe()
    w = synth.Workload(name="perm", N=10, d=16, E=8, G=1, TG=1, k=2, d_ff=8, route_scale=1.0)
    cfg = cfg_of(w)
    counts = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    offs = torch.full((9,), -1, dtype=torch.int32, device="cuda")
    m.moe_permute(cfg, 0, None, None, counts, offs, None, None, None,
                  m.workspace(cfg, 0, m.CALL_PERMUTE))
    torch.cuda.synchronize()
    assert counts.cpu().numpy().tolist() == [0] * 8
    assert offs.cpu().numpy().tolist() == [0] * 9
