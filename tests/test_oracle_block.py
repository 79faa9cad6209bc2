"""Pins for the oracle's expert, combine, latent and shared-expert arithmetic.

- a second formulation in torch (CPU, float64): every expert runs on every
  token and the outputs are masked by the routing (no dispatch at all), with
  torch's own silu / rms_norm / linear;
- the sorted dispatch (gather by the oracle's permutation, per-expert slices,
  un-permute, weighted sum) gives the same rows as the per-token oracle;
- closed forms: SiLU and SiTU identities through identity weights, the SiTU
  bound beta * linear_beta and its SiLU limit, RMS 1 after the latent norm,
  a zero token, identical experts, a removed expert, the shared expert.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _cfg(d, E, k, d_ff, d_sh=0, L=0, act="silu", beta=1.0, lbeta=0.0, norm=True, eps=1e-6):
    return dict(d=d, E=E, k=k, d_ff=d_ff, d_sh=d_sh, L=L, act=act, situ_beta=beta,
                situ_linear_beta=lbeta, latent_norm=norm, norm_eps=eps)


def _make(rng, N, cfg, bf16=False):
    d, E, d_ff, d_sh, L = cfg["d"], cfg["E"], cfg["d_ff"], cfg["d_sh"], cfg["L"]
    d_in = L or d

    def mat(*shape, fan):
        a = rng.normal(0, 1.0 / math.sqrt(fan), shape).astype(np.float32)
        return synth.f32_to_bf16_bits(a).reshape(shape) if bf16 else a

    W = {"w1": mat(E, d_ff, d_in, fan=d_in), "w3": mat(E, d_ff, d_in, fan=d_in),
         "w2": mat(E, d_in, d_ff, fan=d_ff)}
    if d_sh:
        W.update(sh_w1=mat(d_sh, d, fan=d), sh_w3=mat(d_sh, d, fan=d), sh_w2=mat(d, d_sh, fan=d_sh))
    if L:
        W.update(w_down=mat(L, d, fan=d), w_up=mat(d, L, fan=L),
                 gamma=rng.uniform(0.5, 1.5, L).astype(np.float32))
    x = mat(N, d, fan=1)
    idx = np.stack([np.sort(rng.choice(E, cfg["k"], replace=False)) for _ in range(N)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (N, cfg["k"]))
    return x, W, idx, w


def _t(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = synth.bf16_bits_to_f32(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)


def dense_forward(cfg, W, x, idx, w):
    """Masked dense formulation: all experts on all tokens, weighted by the routing."""
    X = _t(x)
    N = X.shape[0]

    def act(g, u):
        if cfg["act"] == "silu":
            return F.silu(g) * u
        b, lb = cfg["situ_beta"], cfg["situ_linear_beta"]
        a = b * torch.tanh(g / b) * torch.sigmoid(g)
        return a * (lb * torch.tanh(u / lb) if lb > 0 else u)

    def mlp(v, w1, w3, w2):
        return F.linear(act(F.linear(v, _t(w1)), F.linear(v, _t(w3))), _t(w2))

    Xin = F.linear(X, _t(W["w_down"])) if cfg["L"] else X
    coef = torch.zeros(N, cfg["E"], dtype=torch.float64)
    coef.scatter_add_(1, torch.from_numpy(idx.astype(np.int64)), torch.from_numpy(w))
    Y = torch.zeros_like(Xin)
    for e in range(cfg["E"]):
        Y += coef[:, e:e + 1] * mlp(Xin, W["w1"][e], W["w3"][e], W["w2"][e])
    if cfg["L"]:
        if cfg["latent_norm"]:
            Y = F.rms_norm(Y, (cfg["L"],), weight=_t(W["gamma"]), eps=cfg["norm_eps"])
        Y = F.linear(Y, _t(W["w_up"]))
    if cfg["d_sh"]:
        Y = Y + mlp(X, W["sh_w1"], W["sh_w3"], W["sh_w2"])
    return Y.numpy()


CASES = {
    "silu": _cfg(16, 8, 3, 8),
    "silu_shared": _cfg(16, 8, 2, 12, d_sh=8),
    "situ": _cfg(16, 6, 2, 8, act="situ", beta=4.0, lbeta=8.0),
    "situ_no_linear_beta": _cfg(16, 6, 2, 8, act="situ", beta=2.0, lbeta=0.0),
    "latent_norm_shared_situ": _cfg(24, 8, 3, 8, d_sh=8, L=12, act="situ", beta=4.0, lbeta=8.0),
    "latent_no_norm": _cfg(16, 8, 2, 8, L=8, norm=False),
    "k1": _cfg(8, 4, 1, 8),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("bf16", [False, True])
def test_dense_formulation(name, bf16):
    cfg = CASES[name]
    rng = np.random.default_rng(len(name) + 7 * bf16)
    x, W, idx, w = _make(rng, 20, cfg, bf16)
    y = oracle.block_tokens(cfg, W, x, np.arange(20), idx, w)
    ref = dense_forward(cfg, W, x, idx, w)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_sorted_dispatch_equals_per_token():
    cfg = CASES["silu"]
    rng = np.random.default_rng(11)
    N = 30
    x, W, idx, w = _make(rng, N, cfg)
    counts, offsets, perm, inv = oracle.counts_perm(idx, cfg["E"])
    k = cfg["k"]
    xs = x[perm // k].astype(np.float64)
    outs = np.zeros_like(xs)
    for e in range(cfg["E"]):
        s = slice(offsets[e], offsets[e + 1])
        g = xs[s] @ W["w1"][e].T.astype(np.float64)
        u = xs[s] @ W["w3"][e].T.astype(np.float64)
        outs[s] = (g / (1.0 + np.exp(-g)) * u) @ W["w2"][e].T.astype(np.float64)
    y_sorted = (outs[inv].reshape(N, k, -1) * w[:, :, None]).sum(axis=1)
    y = oracle.block_tokens(cfg, W, x, np.arange(N), idx, w)
    np.testing.assert_allclose(y, y_sorted, rtol=1e-12, atol=1e-13)


# ---- closed forms through identity weights --------------------------------
# One expert, W1 = I, W3 = c*I, W2 = I and routing weight 1: y_i = h(x_i, c*x_i).

def _identity_block(x_vals, act, c, beta=1.0, lbeta=0.0):
    m = len(x_vals)
    cfg = _cfg(m, 2, 1, m, act=act, beta=beta, lbeta=lbeta)
    eye = np.eye(m, dtype=np.float32)
    W = {"w1": np.stack([eye, eye]), "w3": np.stack([c * eye, c * eye]),
         "w2": np.stack([eye, eye])}
    x = np.asarray(x_vals, np.float32)[None, :]
    return oracle.block_tokens(cfg, W, x, [0], np.array([[0]], np.int32), np.array([[1.0]]))[0]


G_VALS = [0.0, 0.25, 0.5, 1.0, 1.5, 2.0, 3.0, 5.0, 8.0]


def test_silu_identities():
    g = np.array(G_VALS + [-v for v in G_VALS])
    h = _identity_block(g, "silu", 1.0).astype(np.float64)
    g = g.astype(np.float32).astype(np.float64)
    m = len(G_VALS)
    hp, hm = h[:m], h[m:]
    gp = g[:m]
    # silu(g)*g + silu(-g)*(-g) = g^2 (sigma(g) + sigma(-g)) = g^2
    np.testing.assert_allclose(hp + hm, gp ** 2, rtol=1e-13, atol=1e-15)
    assert h[0] == 0.0  # silu(0) = 0


def test_situ_identities():
    beta = 4.0
    g = np.array(G_VALS + [-v for v in G_VALS])
    h = _identity_block(g, "situ", 1.0, beta=beta)
    g = g.astype(np.float32).astype(np.float64)
    m = len(G_VALS)
    hp, hm, gp = h[:m], h[m:], g[:m]
    # a(g) = beta tanh(g/beta) sigma(g):  a(g) - a(-g) = beta tanh(g/beta),
    # a(g) + a(-g) = beta tanh(g/beta) tanh(g/2); with u = g: h = a(g) g.
    t = np.array([math.tanh(v / beta) for v in gp])
    np.testing.assert_allclose(hp + hm, gp * beta * t, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(hp - hm, gp * beta * t * np.tanh(gp / 2), rtol=1e-12, atol=1e-15)


def test_situ_large_beta_is_silu():
    g = [0.3, -1.2, 2.5, -4.0, 6.0]
    a = _identity_block(g, "situ", 1.0, beta=1e4)
    b = _identity_block(g, "silu", 1.0)
    np.testing.assert_allclose(a, b, rtol=1e-6)


def test_situ_bound_and_gate_up_order():
    beta, lbeta = 4.0, 8.0
    g = np.linspace(-30, 30, 61)
    h = _identity_block(g, "situ", 1000.0, beta=beta, lbeta=lbeta)
    assert np.all(np.abs(h) <= beta * lbeta + 1e-12)
    # up branch saturates at linear_beta: h -> linear_beta * a(g) for |g| >= 1
    g32 = g.astype(np.float32).astype(np.float64)
    a = beta * np.tanh(g32 / beta) / (1 + np.exp(-g32))
    sel = np.abs(g32) >= 1.0
    np.testing.assert_allclose(h[sel], (lbeta * np.sign(g32) * a)[sel], rtol=1e-6, atol=1e-9)


def test_latent_norm_gives_unit_rms():
    cfg = _cfg(16, 4, 2, 8, L=16, norm=True, eps=1e-300)
    rng = np.random.default_rng(3)
    x, W, idx, w = _make(rng, 6, cfg)
    W["w_up"] = np.eye(16, dtype=np.float32)
    W["gamma"] = np.ones(16, np.float32)
    y = oracle.block_tokens(cfg, W, x, np.arange(6), idx, w)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    gamma = rng.uniform(0.5, 2.0, 16).astype(np.float32)
    W["gamma"] = gamma
    y2 = oracle.block_tokens(cfg, W, x, np.arange(6), idx, w)
    np.testing.assert_allclose(y2, y * gamma[None, :].astype(np.float64), rtol=1e-13)


def test_zero_token_identical_and_removed_experts():
    cfg = CASES["silu_shared"]
    rng = np.random.default_rng(4)
    N = 10
    x, W, idx, w = _make(rng, N, cfg)
    x[3] = 0.0
    y = oracle.block_tokens(cfg, W, x, np.arange(N), idx, w)
    assert np.all(y[3] == 0.0)
    # identical experts: y = (sum of weights) * MLP(x) + shared
    W_same = dict(W)
    for n in ("w1", "w3", "w2"):
        W_same[n] = np.stack([W[n][0]] * cfg["E"])
    y_same = oracle.block_tokens(cfg, W_same, x, np.arange(N), idx, w)
    cfg1 = dict(cfg, k=1)
    y1 = oracle.block_tokens(cfg1, W_same, x, np.arange(N), idx[:, :1], w.sum(axis=1, keepdims=True))
    np.testing.assert_allclose(y_same, y1, rtol=1e-12, atol=1e-14)
    # removing expert e (w2 = 0) changes exactly the tokens routed to it
    e = int(idx[0, 0])
    W_rm = dict(W)
    W_rm["w2"] = W["w2"].copy()
    W_rm["w2"][e] = 0.0
    y_rm = oracle.block_tokens(cfg, W_rm, x, np.arange(N), idx, w)
    hit = np.any(idx == e, axis=1)
    assert np.all(y_rm[~hit] == y[~hit])
    assert np.all(np.any(y_rm[hit] != y[hit], axis=1))


def test_shared_expert_adds_on_full_input():
    cfg = _cfg(12, 4, 1, 8, d_sh=8)
    rng = np.random.default_rng(9)
    x, W, _, _ = _make(rng, 5, cfg)
    # shared expert = expert 2, routing weight 1 on expert 2: output doubles
    W["sh_w1"], W["sh_w3"], W["sh_w2"] = W["w1"][2], W["w3"][2], W["w2"][2]
    idx = np.full((5, 1), 2, np.int32)
    y = oracle.block_tokens(cfg, W, x, np.arange(5), idx, np.ones((5, 1)))
    y_routed = oracle.block_tokens(dict(cfg, d_sh=0), W, x, np.arange(5), idx, np.ones((5, 1)))
    np.testing.assert_allclose(y, 2.0 * y_routed, rtol=1e-13)


# ---- the row stages the GPU parity tests use ------------------------------

@pytest.mark.parametrize("name", ["silu", "situ", "situ_no_linear_beta", "k1"])
@pytest.mark.parametrize("bf16", [False, True])
def test_row_stages_compose_to_the_block(name, bf16):
    """gate_up_rows, down_rows and combine over the sorted dispatch give the
    per-token oracle's y (itself pinned to the masked dense formulation above),
    with a residual added once; gate_up_rows alone equals torch's float64
    linear + activation on each row's own expert."""
    cfg = CASES[name]
    rng = np.random.default_rng(31 + len(name) + bf16)
    N, k = 25, cfg["k"]
    x, W, idx, w = _make(rng, N, cfg, bf16)
    w32 = w.astype(np.float32).astype(np.float64)  # combine takes fp32 weights
    counts, offsets, perm, inv = oracle.counts_perm(idx, cfg["E"])
    xs = x[perm // k]
    expert = np.repeat(np.arange(cfg["E"]), counts).astype(np.int32)
    h = oracle.gate_up_rows(cfg, W["w1"], W["w3"], xs, expert)
    # the stages store h and the expert outputs in the weights' type (fp32 or
    # bf16, as the GPU path does), so the composition carries those roundings
    def store(a):
        a = a.astype(np.float32)
        return synth.f32_to_bf16_bits(a).reshape(a.shape) if bf16 else a

    h32 = store(h)
    out = oracle.down_rows(cfg, W["w2"], h32, expert)
    res = store(rng.normal(0, 1, (N, cfg["d"])))
    y = oracle.combine(store(out), inv, w32.astype(np.float32), res)
    ref = oracle.block_tokens(cfg, W, x, np.arange(N), idx, w32) + _t(res).numpy()
    if bf16:
        assert np.linalg.norm(y - ref) <= 1e-2 * np.linalg.norm(ref)
    else:
        np.testing.assert_allclose(y, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())

    X = _t(xs)
    for r in range(0, xs.shape[0], 7):
        e = expert[r]
        g = F.linear(X[r], _t(W["w1"][e]))
        u = F.linear(X[r], _t(W["w3"][e]))
        if cfg["act"] == "silu":
            hr = F.silu(g) * u
        else:
            b, lb = cfg["situ_beta"], cfg["situ_linear_beta"]
            hr = b * torch.tanh(g / b) * torch.sigmoid(g) * (lb * torch.tanh(u / lb) if lb > 0 else u)
        np.testing.assert_allclose(h[r], hr.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out[r], F.linear(_t(h32[r]), _t(W["w2"][e])).numpy(),
                                   rtol=1e-12, atol=1e-14)
