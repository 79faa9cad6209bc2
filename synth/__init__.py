"""Seeded synthetic inputs for the MoE block: workloads, tensor recipes, fillers.

This module holds no step of the method.  It names the five workloads (sizes,
activation, dtypes, input distributions), gives every input tensor a recipe
(tensor id, standard deviation, shape), and fills host arrays (``libsynth_host.so``)
or device memory (``libsynth_dev.so``) with the counter-based generator defined in
``synth_core.h``.  Both fillers produce the same bits for the same element, so the
oracle can regenerate on the host exactly the inputs the GPU was given.

Distributions (variances, the plainest reading of the pages' init): hidden ~ N(0,1); router
weight ~ N(0, 1/d); correction bias ~ N(0, 0.01^2), or for the skewed latent
workload a Zipf rank profile 0.25 * r^-1.1 over a seeded permutation of the
experts; gate/up weights ~ N(0, 1/d_in); down weights ~ N(0, 1/d_ff); shared and
latent projection weights likewise N(0, 1/fan_in); latent norm weight = 1.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

F32, BF16 = 0, 1

# Tensor ids: the third Philox counter word, one stream per tensor.
TID = {
    "hidden": 1,
    "w_router": 2,
    "bias": 3,
    "w1": 4,
    "w3": 5,
    "w2": 6,
    "sh_w1": 7,
    "sh_w3": 8,
    "sh_w2": 9,
    "w_down": 10,
    "w_up": 11,
    "bias_perm": 12,
}


@dataclass(frozen=True)
class Workload:
    """One MoE block configuration and its synthetic-input recipe."""

    name: str
    N: int  # tokens = B * T
    d: int  # model width
    E: int  # routed experts
    G: int  # expert groups
    TG: int  # groups kept per token
    k: int  # experts per token
    d_ff: int  # routed expert intermediate width
    route_scale: float
    act: str = "silu"  # "silu" | "situ"
    situ_beta: float = 1.0
    situ_linear_beta: float = 0.0  # <= 0: up branch left linear
    d_sh: int = 0  # shared expert intermediate width (0: none)
    L: int = 0  # latent width (0: no latent projection)
    latent_norm: bool = True
    norm_eps: float = 1e-6
    norm_topk_prob: bool = True
    dtype: int = BF16  # hidden, expert, shared and latent weights, outputs
    bias_kind: str = "normal"  # "normal" (std bias_std) | "zipf"
    bias_std: float = 0.01
    # router form (passed to the library and the oracle; the generator still
    # draws a bias tensor, which a router without one ignores)
    score_func: str = "sigmoid"  # "sigmoid" | "softmax"
    use_bias: bool = True
    B: int = 1
    T: int = 0
    seed: int = 0

    @property
    def d_in(self) -> int:
        return self.L if self.L else self.d

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)

    # ---- tensor recipes -------------------------------------------------
    def shapes(self) -> dict:
        s = {
            "hidden": (self.N, self.d),
            "w_router": (self.E, self.d),
            "bias": (self.E,),
            "w1": (self.E, self.d_ff, self.d_in),
            "w3": (self.E, self.d_ff, self.d_in),
            "w2": (self.E, self.d_in, self.d_ff),
        }
        if self.d_sh:
            s["sh_w1"] = (self.d_sh, self.d)
            s["sh_w3"] = (self.d_sh, self.d)
            s["sh_w2"] = (self.d, self.d_sh)
        if self.L:
            s["w_down"] = (self.L, self.d)
            s["w_up"] = (self.d, self.L)
            s["gamma"] = (self.L,)
        return s

    def stdev(self, name: str) -> float:
        return {
            "hidden": 1.0,
            "w_router": 1.0 / math.sqrt(self.d),
            "bias": self.bias_std,
            "w1": 1.0 / math.sqrt(self.d_in),
            "w3": 1.0 / math.sqrt(self.d_in),
            "w2": 1.0 / math.sqrt(self.d_ff),
            "sh_w1": 1.0 / math.sqrt(self.d),
            "sh_w3": 1.0 / math.sqrt(self.d),
            "sh_w2": 1.0 / math.sqrt(self.d_sh) if self.d_sh else 0.0,
            "w_down": 1.0 / math.sqrt(self.d),
            "w_up": 1.0 / math.sqrt(self.L) if self.L else 0.0,
        }[name]

    def dtype_of(self, name: str) -> int:
        if name in ("w_router", "bias", "gamma"):
            return F32
        return self.dtype


WORKLOADS = {
    "tiny": Workload(
        name="tiny", N=64, d=256, E=16, G=4, TG=2, k=4, d_ff=128, route_scale=2.5,
        dtype=F32, B=1, T=64),
    "dsv3_prefill": Workload(
        name="dsv3_prefill", N=4096, d=7168, E=256, G=8, TG=4, k=8, d_ff=2048,
        route_scale=2.5, B=1, T=4096),
    "k2_prefill": Workload(
        name="k2_prefill", N=8192, d=7168, E=384, G=1, TG=1, k=8, d_ff=2048,
        route_scale=2.827, d_sh=2048, B=2, T=4096),
    "k2_decode": Workload(
        name="k2_decode", N=256, d=7168, E=384, G=1, TG=1, k=8, d_ff=2048,
        route_scale=2.827, d_sh=2048, B=256, T=1),
    "k3_latent_prefill": Workload(
        name="k3_latent_prefill", N=4096, d=7168, E=896, G=1, TG=1, k=8, d_ff=3072,
        route_scale=2.827, act="situ", situ_beta=4.0, situ_linear_beta=8.0, d_sh=3072,
        L=3584, latent_norm=True, bias_kind="zipf", B=1, T=4096),
}
WORKLOAD_ORDER = ["tiny", "dsv3_prefill", "k2_prefill", "k2_decode", "k3_latent_prefill"]


# ---- native fillers -------------------------------------------------------
_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth_host.so")
        if not os.path.exists(path):
            from . import build as _b

            _b.build_host()
        lib = ctypes.CDLL(path)
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_double]
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_fill_u32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_uint32]
        lib.synth_fill_u32.restype = ctypes.c_int
        lib.synth_philox.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_log_u1_host.argtypes = [ctypes.c_uint32]
        lib.synth_log_u1_host.restype = ctypes.c_double
        lib.synth_sqrt_host.argtypes = [ctypes.c_double]
        lib.synth_sqrt_host.restype = ctypes.c_double
        lib.synth_box_muller_host.argtypes = [ctypes.c_uint32, ctypes.c_uint32,
                                              ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_double)]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_dev_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                              ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_double, ctypes.c_void_p]
        lib.synth_dev_fill_normal.restype = ctypes.c_int
        _dev = lib
    return _dev


def philox4x32_10(ctr, key):
    lib = _load_host()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox(c, k, o)
    return list(o)


def fill_normal_host(count: int, first: int, seed: int, tid: int, std: float, dtype: int):
    """Elements [first, first+count) of a normal tensor as float32 or bf16 bits (uint16)."""
    out = np.empty(count, dtype=np.float32 if dtype == F32 else np.uint16)
    rc = _load_host().synth_fill_normal(out.ctypes.data, dtype, count, first, seed, tid, std)
    if rc != 0:
        raise RuntimeError("synth_fill_normal failed")
    return out


def fill_u32_host(count: int, first: int, seed: int, tid: int):
    out = np.empty(count, dtype=np.uint32)
    rc = _load_host().synth_fill_u32(out.ctypes.data, count, first, seed, tid)
    if rc != 0:
        raise RuntimeError("synth_fill_u32 failed")
    return out


def zipf_bias(E: int, seed: int, s: float = 1.1, scale: float = 0.25) -> np.ndarray:
    """Skewed correction bias: expert pi(r) gets scale * r^-s for rank r = 1..E,
    pi a Fisher-Yates shuffle driven by the bias_perm stream."""
    words = fill_u32_host(E, 0, seed, TID["bias_perm"])
    perm = list(range(E))
    for i in range(E - 1, 0, -1):
        j = (int(words[i]) * (i + 1)) >> 32
        perm[i], perm[j] = perm[j], perm[i]
    out = np.empty(E, dtype=np.float32)
    for r in range(1, E + 1):
        out[perm[r - 1]] = np.float32(scale * float(r) ** (-s))
    return out


def host_tensor(w: Workload, name: str, expert: int | None = None) -> np.ndarray:
    """Host copy of one input tensor (or of one expert's slice of a stacked one).

    float32 tensors come back as float32; bf16 tensors as their uint16 bits."""
    shape = w.shapes()[name]
    if name == "gamma":
        return np.ones(shape, dtype=np.float32)
    if name == "bias" and w.bias_kind == "zipf":
        return zipf_bias(w.E, w.seed)
    dt = w.dtype_of(name)
    if expert is None:
        count, first = int(np.prod(shape)), 0
        out_shape = shape
    else:
        per = int(np.prod(shape[1:]))
        count, first = per, expert * per
        out_shape = shape[1:]
    flat = fill_normal_host(count, first, w.seed, TID[name], w.stdev(name), dt)
    return flat.reshape(out_shape)


def fill_device(w: Workload, name: str, ptr: int, stream: int = 0, expert: int | None = None):
    """Fill device memory at `ptr` with the tensor (or expert slice) `name`."""
    shape = w.shapes()[name]
    if name in ("gamma",) or (name == "bias" and w.bias_kind == "zipf"):
        raise ValueError(f"{name} is generated on the host only")
    if expert is None:
        count, first = int(np.prod(shape)), 0
    else:
        per = int(np.prod(shape[1:]))
        count, first = per, expert * per
    rc = _load_dev().synth_dev_fill_normal(ptr, w.dtype_of(name), count, first, w.seed,
                                           TID[name], w.stdev(name), stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_normal({name}) failed: {rc}")


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)
