"""Shared helpers of the GPU parity tests: device inputs from the seeded
recipes, the libmoe config of a workload, routing comparison with the
near-tie rule, and the floating-point acceptance measures."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def has_gpu() -> bool:
    return torch is not None and torch.cuda.is_available()


needs_gpu = pytest.mark.skipif(not has_gpu(), reason="needs an MI355X GPU")


def moe():
    import mixture_experts_layer_29_amd as m

    m.binding.lib()  # fails loudly when libmoe.so is missing
    return m


def cfg_of(w: synth.Workload):
    m = moe()
    return m.make_config(d=w.d, n_experts=w.E, n_group=w.G, topk_group=w.TG, top_k=w.k,
                         d_ff=w.d_ff, route_scale=w.route_scale,
                         norm_topk_prob=w.norm_topk_prob, act=w.act, situ_beta=w.situ_beta,
                         situ_linear_beta=w.situ_linear_beta, d_latent=w.L,
                         latent_norm=w.latent_norm, norm_eps=w.norm_eps, d_ff_shared=w.d_sh,
                         dtype=m.DTYPE_BF16 if w.dtype == synth.BF16 else m.DTYPE_F32,
                         score_func=w.score_func)


def torch_dtype(w: synth.Workload, name: str):
    return torch.float32 if w.dtype_of(name) == synth.F32 else torch.bfloat16


def to_device(a: np.ndarray, bf16: bool):
    """Host array (float32, or bf16 bits as uint16) -> device tensor."""
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    """Device tensor -> float32 array, or uint16 bits for bf16."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def device_inputs(w: synth.Workload, on_device_gen: bool = True) -> dict:
    """Every input tensor of the workload on the GPU.  Large tensors are filled
    in place by the device generator; the rest are generated on the host."""
    out = {}
    for name, shape in w.shapes().items():
        dt = torch_dtype(w, name)
        if name == "gamma" or (name == "bias" and w.bias_kind == "zipf") or not on_device_gen:
            a = synth.host_tensor(w, name)
            out[name] = to_device(a, dt == torch.bfloat16).reshape(shape)
        else:
            t = torch.empty(shape, dtype=dt, device="cuda")
            synth.fill_device(w, name, t.data_ptr())
            out[name] = t
    torch.cuda.synchronize()
    return out


def weights_of(dev: dict, w: synth.Workload = None):
    m = moe()
    bias = dev["bias"] if (w is None or w.use_bias) else None
    return m.Weights(w_router=dev["w_router"], bias=bias, w1=dev["w1"], w3=dev["w3"],
                     w2=dev["w2"], w_down=dev.get("w_down"), gamma=dev.get("gamma"),
                     w_up=dev.get("w_up"), sh_w1=dev.get("sh_w1"), sh_w3=dev.get("sh_w3"),
                     sh_w2=dev.get("sh_w2"))


def oracle_cfg(w: synth.Workload) -> dict:
    return dict(d=w.d, E=w.E, k=w.k, d_ff=w.d_ff, d_sh=w.d_sh, L=w.L, act=w.act,
                situ_beta=w.situ_beta, situ_linear_beta=w.situ_linear_beta,
                latent_norm=w.latent_norm, norm_eps=w.norm_eps)


def resolve_routing(x, w_router, bias, w: synth.Workload, gpu_idx, gpu_wt, wt_rtol=1e-5):
    """Compare the GPU's routing with the oracle's, token by token.

    Indices must be identical except on tokens the oracle flags as near ties,
    where the GPU's choice must pass oracle.valid_choice; the oracle then
    recomputes that token's weights from the GPU's indices.  Weights must match
    to wt_rtol.  Returns (indices, weights, flags, n_resolved) in the oracle's
    terms, to be used downstream (counts, permutation, outputs)."""
    if not w.use_bias:
        bias = None
    o_idx, o_w, flags = oracle.route(x, w_router, bias, w.G, w.TG, w.k, w.norm_topk_prob,
                                     w.route_scale, w.score_func)
    _, score, choice = oracle.router_scores(x, w_router, bias, w.score_func)
    gpu_idx = np.asarray(gpu_idx)
    diff = np.flatnonzero(np.any(o_idx != gpu_idx, axis=1))
    near = (flags & (oracle.FLAG_NEAR_TIE_EXPERT | oracle.FLAG_NEAR_TIE_GROUP)) != 0
    bad = [int(n) for n in diff if not near[n]]
    assert not bad, (f"{len(bad)} tokens route differently with no near tie, e.g. token {bad[0]}: "
                     f"gpu {gpu_idx[bad[0]].tolist()} oracle {o_idx[bad[0]].tolist()}")
    idx = o_idx.copy()
    wt = o_w.copy()
    for n in diff:
        assert oracle.valid_choice(choice[n], w.G, w.TG, w.k, gpu_idx[n],
                                   group_by_max=bias is None), (
            f"token {n}: near tie resolved to an invalid choice {gpu_idx[n].tolist()}")
        idx[n] = gpu_idx[n]
        wt[n] = oracle.weights(score[n], gpu_idx[n], w.norm_topk_prob, w.route_scale)
    np.testing.assert_allclose(np.asarray(gpu_wt, np.float64), wt, rtol=wt_rtol, atol=0)
    return idx, wt, flags, len(diff)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close_bf16(got, ref, what="", output_rounding_slack=False):
    """The bf16 acceptance bar: relative L2 <= 1e-2 and max |err| <= 5e-2 rms(ref).

    output_rounding_slack: widen each element's max-error bar by half a bf16
    ulp of that element.  Storing y in bf16 alone moves an element by up to
    2^-9 of its magnitude (relative), which exceeds 5e-2 rms wherever |y| >
    12.8 rms: only outputs with such heavy tails need it (softmax routing
    without renormalisation gives tokens very different weight totals)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(got, ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    m = float(np.max(err)) if got.size else 0.0
    assert r <= 1e-2, f"{what}: relative L2 {r:.3e} > 1e-2"
    if output_rounding_slack and got.size:
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
        worst = float(np.max(err - half_ulp))
        assert worst <= 5e-2 * rms, (f"{what}: max (abs err - half ulp) {worst:.3e} > "
                                     f"5e-2 * rms {rms:.3e}")
    else:
        assert m <= 5e-2 * rms, f"{what}: max abs err {m:.3e} > 5e-2 * rms {rms:.3e}"
    return r, m / max(rms, 1e-300)


def assert_close_f32(got, ref, what="", tol=1e-5):
    """fp32 blocks: relative L2 <= 1e-5 (derived in the design notes)."""
    r = rel_l2(got, ref)
    assert r <= tol, f"{what}: relative L2 {r:.3e} > {tol:.0e}"
    return r
