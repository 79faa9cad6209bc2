"""Thin Python binding of libmoe's C ABI (include/moe.h).

Argument marshalling only: every step of the MoE block runs in libmoe's HIP
kernels.  Tensors are torch tensors on the GPU (bf16 or fp32 as the config's
dtype says; int32 indices; fp32 router weight, bias and routing weights);
``stream`` defaults to torch's current stream.  A non-OK status raises
``MoeError``; a missing ``libmoe.so`` raises at import of the first call."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1
ACT_SILU, ACT_SITU = 0, 1
SCORE_SIGMOID, SCORE_SOFTMAX = 0, 1
TOPK_NOAUX_TC = 0
CALL_ROUTE, CALL_PERMUTE, CALL_GATE_UP, CALL_DOWN, CALL_COMBINE, CALL_BLOCK, CALL_SHARED, \
    CALL_LATENT = range(8)


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int64),
        ("n_experts", ctypes.c_int64),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32),
        ("route_scale", ctypes.c_float),
        ("score_func", ctypes.c_int32),
        ("topk_method", ctypes.c_int32),
        ("training", ctypes.c_int32),
        ("d_ff", ctypes.c_int64),
        ("act", ctypes.c_int32),
        ("situ_beta", ctypes.c_float),
        ("situ_linear_beta", ctypes.c_float),
        ("d_latent", ctypes.c_int64),
        ("latent_norm", ctypes.c_int32),
        ("norm_eps", ctypes.c_float),
        ("d_ff_shared", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
    ]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "bias", "w1", "w3", "w2", "w_down", "gamma", "w_up", "sh_w1", "sh_w3",
        "sh_w2")]


def make_config(*, d, n_experts, n_group, topk_group, top_k, d_ff, route_scale,
                norm_topk_prob=True, act=ACT_SILU, situ_beta=0.0, situ_linear_beta=0.0,
                d_latent=0, latent_norm=True, norm_eps=1e-6, d_ff_shared=0, dtype=DTYPE_BF16,
                score_func=SCORE_SIGMOID, topk_method=TOPK_NOAUX_TC, training=False) -> moe_config:
    if isinstance(act, str):
        act = {"silu": ACT_SILU, "situ": ACT_SITU}[act]
    if isinstance(score_func, str):
        score_func = {"sigmoid": SCORE_SIGMOID, "softmax": SCORE_SOFTMAX}[score_func]
    return moe_config(d=d, n_experts=n_experts, n_group=n_group, topk_group=topk_group,
                      top_k=top_k, norm_topk_prob=int(bool(norm_topk_prob)),
                      route_scale=route_scale, score_func=score_func, topk_method=topk_method,
                      training=int(bool(training)), d_ff=d_ff, act=act, situ_beta=situ_beta,
                      situ_linear_beta=situ_linear_beta, d_latent=d_latent,
                      latent_norm=int(bool(latent_norm)), norm_eps=norm_eps,
                      d_ff_shared=d_ff_shared, dtype=dtype)


_lib = None


def lib():
    """The loaded libmoe.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        C = ctypes.POINTER(moe_config)
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_validate_config.argtypes = [C]
        L.moe_workspace_size.argtypes = [C, i64, i32, ctypes.POINTER(sz)]
        L.moe_route.argtypes = [C, i64, P, P, P, P, P, P, sz, P]
        L.moe_permute.argtypes = [C, i64, P, P, P, P, P, P, P, P, sz, P]
        L.moe_permute_static.argtypes = [C, i64, P, P, P, P, P, P, P, P]
        L.moe_expert_gate_up.argtypes = [C, i64, P, P, P, P, P, P, sz, P]
        L.moe_expert_gate_up_gather.argtypes = [C, i64, P, P, P, P, P, P, P, sz, P]
        L.moe_expert_down.argtypes = [C, i64, P, P, P, P, P, sz, P]
        L.moe_expert_down_scatter.argtypes = [C, i64, P, P, P, P, P, P, sz, P]
        L.moe_combine.argtypes = [C, i64, P, P, P, P, P, P]
        L.moe_block_forward.argtypes = [C, i64, ctypes.POINTER(moe_weights), P, P, P, P, P, P, sz, P]
        L.moe_shared_expert.argtypes = [C, i64, P, P, P, P, P, P, sz, P]
        L.moe_latent_project.argtypes = [C, i64, i32, P, P, P, P, P]
        for f in ("moe_validate_config", "moe_workspace_size", "moe_route", "moe_permute",
                  "moe_permute_static",
                  "moe_expert_gate_up", "moe_expert_gate_up_gather", "moe_expert_down",
                  "moe_expert_down_scatter", "moe_combine", "moe_block_forward", "moe_shared_expert", "moe_latent_project"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().moe_status_str(s).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, last_error())


def _p(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_validate_config(cfg: moe_config) -> None:
    _check(lib().moe_validate_config(ctypes.byref(cfg)))


def moe_workspace_size(cfg: moe_config, N: int, call: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), N, call, ctypes.byref(out)))
    return out.value


def workspace(cfg: moe_config, N: int, call: int, device="cuda"):
    """A device byte buffer large enough for `call` (torch allocations are 256-B aligned)."""
    import torch

    n = moe_workspace_size(cfg, N, call)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(cfg, N, hidden, w_router, bias, topk_idx, topk_weight, ws, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), N, _p(hidden), _p(w_router), _p(bias), _p(topk_idx),
                           _p(topk_weight), _p(ws), _nbytes(ws), _stream(stream)))


def moe_permute(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm, inv_perm,
                x_sorted, ws, stream=None):
    _check(lib().moe_permute(ctypes.byref(cfg), N, _p(topk_idx), _p(x_in), _p(tokens_per_expert),
                             _p(expert_offsets), _p(perm), _p(inv_perm), _p(x_sorted), _p(ws),
                             _nbytes(ws), _stream(stream)))


def moe_permute_static(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm,
                       inv_perm, x_sorted, stream=None):
    """moe_permute with its scratch in the library's static device array (no workspace)."""
    _check(lib().moe_permute_static(ctypes.byref(cfg), N, _p(topk_idx), _p(x_in),
                                    _p(tokens_per_expert), _p(expert_offsets), _p(perm),
                                    _p(inv_perm), _p(x_sorted), _stream(stream)))


def moe_expert_gate_up(cfg, N, x_sorted, expert_offsets, w1, w3, h_sorted, ws, stream=None):
    _check(lib().moe_expert_gate_up(ctypes.byref(cfg), N, _p(x_sorted), _p(expert_offsets), _p(w1),
                                    _p(w3), _p(h_sorted), _p(ws), _nbytes(ws), _stream(stream)))


def moe_expert_gate_up_gather(cfg, N, x_in, perm, expert_offsets, w1, w3, h_sorted, ws,
                              stream=None):
    _check(lib().moe_expert_gate_up_gather(ctypes.byref(cfg), N, _p(x_in), _p(perm),
                                           _p(expert_offsets), _p(w1), _p(w3), _p(h_sorted),
                                           _p(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down(cfg, N, h_sorted, expert_offsets, w2, out_sorted, ws, stream=None):
    _check(lib().moe_expert_down(ctypes.byref(cfg), N, _p(h_sorted), _p(expert_offsets), _p(w2),
                                 _p(out_sorted), _p(ws), _nbytes(ws), _stream(stream)))


def moe_expert_down_scatter(cfg, N, h_sorted, expert_offsets, perm, w2, out_slots, ws,
                            stream=None):
    """moe_expert_down writing row p to slot perm[p] (token order, k rows per token)."""
    _check(lib().moe_expert_down_scatter(ctypes.byref(cfg), N, _p(h_sorted), _p(expert_offsets),
                                         _p(perm), _p(w2), _p(out_slots), _p(ws), _nbytes(ws),
                                         _stream(stream)))


def moe_shared_expert(cfg, N, hidden, sh_w1, sh_w3, sh_w2, out, ws, stream=None):
    """out [N, d] fp32 = the shared expert's MLP on hidden."""
    _check(lib().moe_shared_expert(ctypes.byref(cfg), N, _p(hidden), _p(sh_w1), _p(sh_w3),
                                   _p(sh_w2), _p(out), _p(ws), _nbytes(ws), _stream(stream)))


def moe_latent_project(cfg, N, up, x, w, residual, out, stream=None):
    """The latent down (up=0) or up (up=1) projection, with an optional fp32 residual."""
    _check(lib().moe_latent_project(ctypes.byref(cfg), N, int(up), _p(x), _p(w), _p(residual),
                                    _p(out), _stream(stream)))


def moe_combine(cfg, N, out_sorted, inv_perm, topk_weight, residual, y, stream=None):
    """inv_perm None: out_sorted holds the rows in slot order (moe_expert_down_scatter)."""
    _check(lib().moe_combine(ctypes.byref(cfg), N, _p(out_sorted), _p(inv_perm), _p(topk_weight),
                             _p(residual), _p(y), _stream(stream)))


@dataclass
class Weights:
    """Device tensors of one block (None where the config has no such part)."""

    w_router: object
    bias: object
    w1: object
    w3: object
    w2: object
    w_down: object = None
    gamma: object = None
    w_up: object = None
    sh_w1: object = None
    sh_w3: object = None
    sh_w2: object = None

    def as_struct(self) -> moe_weights:
        return moe_weights(**{f: _p(getattr(self, f)) for f, _ in moe_weights._fields_})


def moe_block_forward(cfg, N, weights: Weights, hidden, y, ws, topk_idx_out=None,
                      topk_weight_out=None, tokens_per_expert_out=None, stream=None):
    w = weights.as_struct()
    _check(lib().moe_block_forward(ctypes.byref(cfg), N, ctypes.byref(w), _p(hidden), _p(y),
                                   _p(topk_idx_out), _p(topk_weight_out),
                                   _p(tokens_per_expert_out), _p(ws), _nbytes(ws),
                                   _stream(stream)))
