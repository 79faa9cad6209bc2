"""The block's dense products through moe_shared_expert and moe_latent_project,
against the oracle's per-row expert halves (the shared expert is the same gated
MLP as a routed expert, on the full-width input; a latent projection is a
down-row product x . W^T), plus an fp32 residual added in fp64.

From 512 rows on these run the MFMA tile kernel (256 x 256 tiles on 8 waves);
the sizes here span several tiles in both directions, with a ragged last row
tile and widths that do not fill a column tile.  The full-size cases are the
shapes of the prefill workloads (shared expert of the Kimi-K2-style prefill,
latent projections of the Kimi-K3-style prefill), compared on 64 sampled rows
spread over every row tile (each sampled row covers every column tile)."""
import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, moe, needs_gpu, to_device, to_host, torch)

pytestmark = [pytest.mark.gpu, needs_gpu]


def cfg_for(m, d, d_sh=0, L=0, act="silu"):
    return m.make_config(d=d, n_experts=4, n_group=1, topk_group=1, top_k=2, d_ff=64,
                         route_scale=1.0, act=act, situ_beta=4.0 if act == "situ" else 0.0,
                         situ_linear_beta=8.0 if act == "situ" else 0.0, d_latent=L,
                         d_ff_shared=d_sh, dtype=m.DTYPE_BF16)


def ocfg(d, width, act="silu", K=None):
    """Oracle config for one weight set used as expert 0: d_in = d, d_ff = width."""
    return dict(d=d, E=1, k=1, d_ff=width, act=act, situ_beta=4.0 if act == "situ" else 1.0,
                situ_linear_beta=8.0 if act == "situ" else 0.0)


def normal(shape, seed, std):
    return synth.fill_normal_host(int(np.prod(shape)), 0, seed, 1, std, synth.BF16).reshape(shape)


def sample_rows(M, n=64):
    """n rows spread over every 256-row tile (first, last and random ones)."""
    rng = np.random.default_rng(M)
    rows = set(range(0, M, 256)) | set(range(255, M, 256)) | {M - 1}
    rows |= set(rng.choice(M, max(0, n - len(rows)), replace=False).tolist())
    return np.array(sorted(rows))


def check_shared(M, d, d_sh, act, rows=None):
    m = moe()
    c = cfg_for(m, d, d_sh=d_sh, act=act)
    x = normal((M, d), 31, 1.0)
    w1 = normal((d_sh, d), 32, d ** -0.5)
    w3 = normal((d_sh, d), 33, d ** -0.5)
    w2 = normal((d, d_sh), 34, d_sh ** -0.5)
    out = torch.empty((M, d), dtype=torch.float32, device="cuda")
    m.moe_shared_expert(c, M, to_device(x, True), to_device(w1, True), to_device(w3, True),
                        to_device(w2, True), out, m.workspace(c, M, m.CALL_SHARED))
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    e0 = np.zeros(len(rows), np.int32)
    h = oracle.gate_up_rows(ocfg(d, d_sh, act), {0: w1}, {0: w3}, x[rows], e0)
    # the GPU rounds h to bf16 before the down product: so does the reference
    h16 = synth.f32_to_bf16_bits(h.astype(np.float32))
    ref = oracle.down_rows(ocfg(d, d_sh, act), {0: w2}, h16, e0)
    got = to_host(out)[rows].astype(np.float64)
    return assert_close_bf16(got, ref, f"shared expert M={M} d={d} d_sh={d_sh} {act}")


def check_latent(M, d, L, up, residual, rows=None):
    m = moe()
    c = cfg_for(m, d, L=L)
    K, n_out = (L, d) if up else (d, L)
    x = normal((M, K), 41 + up, 1.0)
    w = normal((n_out, K), 43 + up, K ** -0.5)
    res = (synth.fill_normal_host(M * n_out, 0, 45, 1, 1.0, synth.F32).reshape(M, n_out)
           if residual else None)
    out = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")
    m.moe_latent_project(c, M, up, to_device(x, True), to_device(w, True),
                         None if res is None else to_device(res, False), out)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    ref = oracle.down_rows(ocfg(n_out, K), {0: w}, x[rows], np.zeros(len(rows), np.int32))
    if res is not None:
        ref = ref + res[rows].astype(np.float64)
    got = as_f64(to_host(out)[rows])
    return assert_close_bf16(got, ref, f"latent {'up' if up else 'down'} M={M} K={K} n={n_out}")


@pytest.mark.parametrize("M,d,d_sh,act", [
    (512, 1024, 1024, "silu"),     # 2 x 8 gate/up tiles, 2 x 4 down tiles
    (1000, 768, 384, "situ"),      # ragged last row tile, 3 gate/up column tiles
    (768, 1536, 640, "silu"),      # down K = 640 (10 blocks); gate/up ends in half a tile
])
def test_shared_expert(M, d, d_sh, act):
    print(f"dense parity: shared expert M={M} d={d} d_sh={d_sh} {act}", flush=True)
    check_shared(M, d, d_sh, act)


@pytest.mark.parametrize("M,d,L,up,residual", [
    (512, 1024, 512, 0, False),
    (1000, 1024, 768, 0, False),
    (1000, 1024, 768, 1, True),
    (600, 768, 1280, 1, False),
])
def test_latent_projection(M, d, L, up, residual):
    print(f"dense parity: latent up={up} M={M} d={d} L={L} residual={residual}", flush=True)
    check_latent(M, d, L, up, residual)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 160])
def test_short_k(d):
    """K of 1 to 5 blocks of 32: fewer blocks than the copy pipeline runs ahead,
    so its waits take their shortened forms from the first block on."""
    print(f"dense parity: short K latent down M=520 d={d} L=264", flush=True)
    check_latent(520, d, 264, 0, False)


def test_short_k_shared_and_up():
    print("dense parity: short K shared expert M=600 d=96 d_sh=64, latent up L=96", flush=True)
    check_shared(600, 96, 64, "silu")
    check_latent(600, 520, 96, 1, True)


def test_full_size_shared_expert():
    """Kimi-K2-style prefill: 8192 tokens, d 7168, shared d_ff 2048."""
    print("dense parity: full-size shared expert 8192 x 7168 x 2048", flush=True)
    r, mx = check_shared(8192, 7168, 2048, "silu", rows=sample_rows(8192))
    print(f"  rel L2 {r:.2e}, max err / rms {mx:.2e}", flush=True)


@pytest.mark.parametrize("up", [0, 1])
def test_full_size_latent_projections(up):
    """Kimi-K3-style prefill: 4096 tokens, d 7168, latent 3584 (up with a residual)."""
    print(f"dense parity: full-size latent up={up} 4096 x 7168 x 3584", flush=True)
    r, mx = check_latent(4096, 7168, 3584, up, bool(up), rows=sample_rows(4096))
    print(f"  rel L2 {r:.2e}, max err / rms {mx:.2e}", flush=True)
