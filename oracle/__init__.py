"""CPU oracle for the routed MoE block forward (Python side of liboracle.so).

TEST INFRASTRUCTURE ONLY.  The arithmetic lives in ``oracle.c`` (plain C, fp64,
token by token; page citations there).  This wrapper marshals numpy arrays and
adds one acceptance rule the pages' near-tie exception needs:
``valid_choice`` decides whether another implementation's expert choice for a
token is a legitimate resolution of a near tie.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

F32, BF16 = 0, 1
ACT = {"silu": 0, "situ": 1}
FLAG_NEAR_TIE_EXPERT = 1
FLAG_NEAR_TIE_GROUP = 2
FLAG_FILL_MATTERS = 4
NEAR_TIE_REL = 1e-6

_lib = None


class _BlockCfg(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int64),
        ("E", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("d_ff", ctypes.c_int64),
        ("d_sh", ctypes.c_int64),
        ("L", ctypes.c_int64),
        ("act", ctypes.c_int32),
        ("situ_beta", ctypes.c_double),
        ("situ_linear_beta", ctypes.c_double),
        ("latent_norm", ctypes.c_int32),
        ("norm_eps", ctypes.c_double),
        ("dtype", ctypes.c_int32),
    ]


class _BlockWeights(ctypes.Structure):
    _fields_ = [
        ("w1", ctypes.POINTER(ctypes.c_void_p)),
        ("w3", ctypes.POINTER(ctypes.c_void_p)),
        ("w2", ctypes.POINTER(ctypes.c_void_p)),
        ("sh_w1", ctypes.c_void_p),
        ("sh_w3", ctypes.c_void_p),
        ("sh_w2", ctypes.c_void_p),
        ("w_down", ctypes.c_void_p),
        ("w_up", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
    ]


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b

            _b.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_router_scores.argtypes = [i64, i64, i64, P, i32, P, P, i32, P, P, P]
        lib.oracle_router_scores.restype = i32
        lib.oracle_select.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P]
        lib.oracle_select.restype = i32
        lib.oracle_weights.argtypes = [i32, i32, f64, P, P, P]
        lib.oracle_weights.restype = None
        lib.oracle_route.argtypes = [i64, i64, i64, i32, i32, i32, i32, f64, i32, P, i32, P, P, P,
                                     P, P]
        lib.oracle_route.restype = i32
        lib.oracle_counts_perm.argtypes = [i64, i32, i64, P, P, P, P, P]
        lib.oracle_counts_perm.restype = i32
        lib.oracle_block_tokens.argtypes = [ctypes.POINTER(_BlockCfg),
                                            ctypes.POINTER(_BlockWeights), P, i64, P, P, P, P]
        lib.oracle_block_tokens.restype = i32
        lib.oracle_gate_up_rows.argtypes = [ctypes.POINTER(_BlockCfg), P, P, i64, P, P, P]
        lib.oracle_gate_up_rows.restype = i32
        lib.oracle_down_rows.argtypes = [ctypes.POINTER(_BlockCfg), P, i64, P, P, P]
        lib.oracle_down_rows.restype = i32
        lib.oracle_combine.argtypes = [i64, i32, i64, i32, P, P, P, P, P]
        lib.oracle_combine.restype = i32
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bits
        return BF16
    raise TypeError(f"unsupported array dtype {a.dtype} (float32 or bf16 bits as uint16)")


def _c(a: np.ndarray, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


SCORE_FUNCS = {"sigmoid": 0, "softmax": 1}


def _bias_ptr(bias):
    """(array kept alive or None, pointer or None): a router may have no bias."""
    if bias is None:
        return None, None
    b = _c(bias, np.float32)
    return b, b.ctypes.data


def router_scores(x, w_router, bias, score_func: str = "sigmoid"):
    """fp32 logits, scores and choice scores [N, E] as the pages compute them
    (bias None: a router without a bias, choice = score)."""
    x = _c(x)
    w_router = _c(w_router, np.float32)
    keep, bptr = _bias_ptr(bias)
    N, d = x.shape
    E = w_router.shape[0]
    logit = np.empty((N, E), np.float32)
    score = np.empty((N, E), np.float32)
    choice = np.empty((N, E), np.float32)
    rc = _load().oracle_router_scores(N, d, E, x.ctypes.data, _dtype_code(x), w_router.ctypes.data,
                                      bptr, SCORE_FUNCS[score_func], logit.ctypes.data,
                                      score.ctypes.data, choice.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_router_scores failed ({rc})")
    return logit, score, choice


def select(choice_row, G: int, TG: int, k: int, group_by_max: bool = False):
    """Group pruning + top-k on one token's fp32 choice scores (group score:
    sum of the two largest, or the largest when group_by_max: no bias).

    Returns (idx ascending [k] int32, flags, gap_expert, gap_group, group_scores [G])."""
    choice_row = _c(choice_row, np.float32)
    E = choice_row.shape[0]
    idx = np.empty(k, np.int32)
    ge = ctypes.c_double()
    gg = ctypes.c_double()
    gs = np.empty(G, np.float32)
    f = _load().oracle_select(E, G, TG, k, int(bool(group_by_max)), choice_row.ctypes.data,
                              idx.ctypes.data,
                              ctypes.byref(ge), ctypes.byref(gg), gs.ctypes.data)
    if f < 0:
        raise ValueError("invalid routing configuration")
    return idx, int(f), ge.value, gg.value, gs


def weights(score_row, idx, norm_topk_prob: bool, route_scale: float):
    score_row = _c(score_row, np.float32)
    idx = _c(idx, np.int32)
    out = np.empty(idx.shape[0], np.float64)
    _load().oracle_weights(idx.shape[0], int(bool(norm_topk_prob)), float(route_scale),
                           score_row.ctypes.data, idx.ctypes.data, out.ctypes.data)
    return out


def route(x, w_router, bias, G: int, TG: int, k: int, norm_topk_prob: bool, route_scale: float,
          score_func: str = "sigmoid"):
    """Router for all tokens: (topk_idx [N,k] int32 ascending, topk_weight [N,k] f64, flags [N]).
    bias None: a router without a bias (groups scored by their largest choice)."""
    x = _c(x)
    w_router = _c(w_router, np.float32)
    keep, bptr = _bias_ptr(bias)
    N, d = x.shape
    E = w_router.shape[0]
    idx = np.empty((N, k), np.int32)
    w = np.empty((N, k), np.float64)
    flags = np.zeros(N, np.uint8)
    rc = _load().oracle_route(N, d, E, G, TG, k, int(bool(norm_topk_prob)), float(route_scale),
                              SCORE_FUNCS[score_func], x.ctypes.data, _dtype_code(x),
                              w_router.ctypes.data, bptr, idx.ctypes.data, w.ctypes.data,
                              flags.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_route failed ({rc})")
    return idx, w, flags


def counts_perm(topk_idx, E: int):
    """(counts [E], offsets [E+1], perm [N*k], inv_perm [N*k]) as int32."""
    topk_idx = _c(topk_idx, np.int32)
    N, k = topk_idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(N * k, np.int32)
    inv = np.empty(N * k, np.int32)
    rc = _load().oracle_counts_perm(N, k, E, topk_idx.ctypes.data, counts.ctypes.data,
                                    offsets.ctypes.data, perm.ctypes.data, inv.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_counts_perm failed ({rc})")
    return counts, offsets, perm, inv


def block_tokens(cfg: dict, weights_: dict, x, tokens, topk_idx, topk_weight):
    """Block output rows (fp64 [len(tokens), d]) for the given tokens.

    cfg keys: d, E, k, d_ff, d_sh, L, act ('silu'|'situ'), situ_beta,
    situ_linear_beta, latent_norm, norm_eps.  weights_: 'w1', 'w3', 'w2' map an
    expert id to its matrix (a stacked [E, ...] array also works); optional
    'sh_w1', 'sh_w3', 'sh_w2', 'w_down', 'w_up', 'gamma'.  Arrays are float32
    or bf16 bits (uint16), all of the same element type as x."""
    x = _c(x)
    dt = _dtype_code(x)
    tokens = _c(np.asarray(tokens), np.int64)
    n_tok = tokens.shape[0]
    k = int(cfg["k"])
    idx = _c(np.asarray(topk_idx).reshape(n_tok, k), np.int32)
    w = _c(np.asarray(topk_weight).reshape(n_tok, k), np.float64)
    E = int(cfg["E"])
    keep = []

    def ptr(a):
        if a is None:
            return None
        a = _c(a)
        if a.dtype != np.float32 and _dtype_code(a) != dt:
            raise TypeError("weights must share the element type of x")
        keep.append(a)
        return a.ctypes.data

    def table(name):
        src = weights_[name]
        arr = (ctypes.c_void_p * E)()
        for e in range(E):
            m = None
            if isinstance(src, dict):
                m = src.get(e)
            else:
                m = src[e]
            arr[e] = ptr(m) if m is not None else None
        keep.append(arr)
        return arr

    c = _BlockCfg(d=int(cfg["d"]), E=E, k=k, d_ff=int(cfg["d_ff"]), d_sh=int(cfg.get("d_sh", 0)),
                  L=int(cfg.get("L", 0)), act=ACT[cfg.get("act", "silu")],
                  situ_beta=float(cfg.get("situ_beta", 1.0)),
                  situ_linear_beta=float(cfg.get("situ_linear_beta", 0.0)),
                  latent_norm=int(bool(cfg.get("latent_norm", True))),
                  norm_eps=float(cfg.get("norm_eps", 1e-6)), dtype=dt)
    W = _BlockWeights(
        w1=ctypes.cast(table("w1"), ctypes.POINTER(ctypes.c_void_p)),
        w3=ctypes.cast(table("w3"), ctypes.POINTER(ctypes.c_void_p)),
        w2=ctypes.cast(table("w2"), ctypes.POINTER(ctypes.c_void_p)),
        sh_w1=ptr(weights_.get("sh_w1")), sh_w3=ptr(weights_.get("sh_w3")),
        sh_w2=ptr(weights_.get("sh_w2")), w_down=ptr(weights_.get("w_down")),
        w_up=ptr(weights_.get("w_up")),
        gamma=ptr(_c(weights_["gamma"], np.float32)) if weights_.get("gamma") is not None else None)
    if c.d_sh and not (W.sh_w1 and W.sh_w3 and W.sh_w2):
        raise ValueError("shared expert weights missing")
    if c.L and not (W.w_down and W.w_up and W.gamma):
        raise ValueError("latent projection weights missing")
    y = np.empty((n_tok, c.d), np.float64)
    rc = _load().oracle_block_tokens(ctypes.byref(c), ctypes.byref(W), x.ctypes.data, n_tok,
                                     tokens.ctypes.data, idx.ctypes.data, w.ctypes.data,
                                     y.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_block_tokens failed ({rc})")
    return y


def _cfg_struct(cfg: dict, dt: int) -> _BlockCfg:
    return _BlockCfg(d=int(cfg["d"]), E=int(cfg["E"]), k=int(cfg.get("k", 1)),
                     d_ff=int(cfg["d_ff"]), d_sh=int(cfg.get("d_sh", 0)), L=int(cfg.get("L", 0)),
                     act=ACT[cfg.get("act", "silu")], situ_beta=float(cfg.get("situ_beta", 1.0)),
                     situ_linear_beta=float(cfg.get("situ_linear_beta", 0.0)),
                     latent_norm=int(bool(cfg.get("latent_norm", True))),
                     norm_eps=float(cfg.get("norm_eps", 1e-6)), dtype=dt)


def _ptr_table(src, E, keep):
    arr = (ctypes.c_void_p * E)()
    for e in range(E):
        m = src.get(e) if isinstance(src, dict) else src[e]
        if m is not None:
            m = _c(m)
            keep.append(m)
            arr[e] = m.ctypes.data
    keep.append(arr)
    return arr


def gate_up_rows(cfg: dict, w1, w3, x_rows, expert):
    """h [R, d_ff] fp64: act(w1[e] x, w3[e] x) for each row x with its expert e."""
    x_rows = _c(x_rows)
    expert = _c(np.asarray(expert), np.int32)
    R = x_rows.shape[0]
    keep = []
    c = _cfg_struct(cfg, _dtype_code(x_rows))
    h = np.empty((R, c.d_ff), np.float64)
    rc = _load().oracle_gate_up_rows(ctypes.byref(c), _ptr_table(w1, c.E, keep),
                                     _ptr_table(w3, c.E, keep), R, x_rows.ctypes.data,
                                     expert.ctypes.data, h.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_gate_up_rows failed ({rc})")
    return h


def down_rows(cfg: dict, w2, h_rows, expert):
    """out [R, d_in] fp64: w2[e] h for each row h with its expert e."""
    h_rows = _c(h_rows)
    expert = _c(np.asarray(expert), np.int32)
    R = h_rows.shape[0]
    keep = []
    c = _cfg_struct(cfg, _dtype_code(h_rows))
    d_in = c.L or c.d
    out = np.empty((R, d_in), np.float64)
    rc = _load().oracle_down_rows(ctypes.byref(c), _ptr_table(w2, c.E, keep), R,
                                  h_rows.ctypes.data, expert.ctypes.data, out.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_down_rows failed ({rc})")
    return out


def combine(out_sorted, inv_perm, topk_weight, residual=None):
    """y [N, width] fp64 = residual + sum_j w[n, j] * out_sorted[inv_perm[n*k + j]]."""
    out_sorted = _c(out_sorted)
    w = _c(topk_weight, np.float32)
    N, k = w.shape
    inv = _c(np.asarray(inv_perm).reshape(-1), np.int32)
    width = out_sorted.shape[1]
    res = None if residual is None else _c(residual)
    y = np.empty((N, width), np.float64)
    _load().oracle_combine(N, k, width, _dtype_code(out_sorted), out_sorted.ctypes.data,
                           inv.ctypes.data, w.ctypes.data,
                           None if res is None else res.ctypes.data, y.ctypes.data)
    return y


def valid_choice(choice_row, G: int, TG: int, k: int, idx, tol: float = 2 * NEAR_TIE_REL,
                 group_by_max: bool = False) -> bool:
    """Is `idx` a legitimate expert choice for this token up to near ties?

    It is when some set K of TG groups containing the chosen experts' groups is
    a top-TG set of the group scores, and `idx` is a top-k set of the choice
    scores inside K, where "top" tolerates a shortfall of tol (relative to the
    boundary value) against any excluded competitor.  Used only for tokens the
    oracle flags as near ties."""
    choice_row = np.asarray(choice_row, np.float32)
    E = choice_row.shape[0]
    idx = [int(i) for i in np.asarray(idx).ravel()]
    if len(idx) != k or len(set(idx)) != k or min(idx) < 0 or max(idx) >= E:
        return False
    per = E // G
    _, _, _, _, gs = select(choice_row, G, TG, k, group_by_max)
    gs = gs.astype(np.float64)
    groups = sorted({i // per for i in idx})
    if len(groups) > TG:
        return False
    rest = [g for g in range(G) if g not in groups]
    rest.sort(key=lambda g: (-gs[g], g))
    kept = set(groups) | set(rest[: TG - len(groups)])
    out_g = [g for g in range(G) if g not in kept]
    if out_g:
        lo = min(gs[g] for g in kept)
        hi = max(gs[g] for g in out_g)
        if lo < hi - tol * abs(hi):
            return False
    cand = [e for e in range(E) if (e // per) in kept]
    chosen = set(idx)
    excl = [choice_row[e] for e in cand if e not in chosen]
    if excl:
        lo = float(min(choice_row[e] for e in chosen))
        hi = float(max(excl))
        if lo < hi - tol * abs(hi):
            return False
    return True
