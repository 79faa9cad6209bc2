"""Benchmark of the MoE block forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one moe_block_forward over one batch of synthetic tokens whose
inputs are already resident in HBM (filled in place by the seeded device
generator).  W untimed steps, then exactly K timed steps between device
synchronisations; rank 0 prints one JSON line.  The default workload is the
largest one-GPU configuration, the Kimi-K3-style latent prefill (4096 tokens,
d 7168 projected to a 3584 latent, 896 experts, top-8, d_ff 3072, SiTU with
beta 4 and linear beta 8 in fp32, RMS-normed latent projected back up, one
shared expert of d_ff 3072, Zipf-skewed correction bias; bf16 experts, fp32
router).

Beside the block throughput the line carries:
  roofline      the dominant kernel (the routed gate/up grouped GEMM) timed with
                HIP events recorded by libmoe on its own stream around that one
                launch in every timed step; achieved = algorithmic bytes per
                launch (w1 and w3 of every expert that holds a row, plus the
                experts' input read once) / average launch time, against the
                8 TB/s HBM peak.  The gathered input rows and the h rows are
                implementation traffic: `traffic` is what the hardware counters
                measured for the launch (profiles/traffic.json), given only while
                the kernel sources still hash to what was measured;
  cpu_baseline  the oracle (plain C, fp64) on the host's cores: the router over
                all N tokens, and the experts, combine and projections over a
                bounded token sample, as tokens/s.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s (% bf16 MFMA peak); decode HBM GB/s (% peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
STAGES = ["route", "latent_down", "dispatch", "shared", "gate_up", "down", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources whose code the routed grouped-GEMM launches run
GEMM_SOURCES = ["common.h", "gemm_common.h", "gemm_plan.h", "gemm_lds.h", "gemm_bf16.hip"]


def gemm_source_digest() -> str:
    """sha256 over the grouped-GEMM sources: counters taken on other code do not apply."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_29_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="k3_latent_prefill")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="first run one plain device copy of this many MiB (a known-size "
                        "reference for hardware byte counters)")
    return p.parse_args()


class Hip:
    """hipEvent helpers straight from the HIP runtime (events for libmoe's stage hooks)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b) -> float:
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value


def algorithmic_work(w, counts):
    """Flops and minimum bytes of one block forward, and of the routed launches.

    Bytes count what the method must move once: the weights of every expert
    that holds a row, the shared and latent weights, the router weight and bias,
    the block input and output and the routing outputs.  The expert-sorted
    intermediates (gathered input rows, h, expert outputs) are implementation
    traffic and are reported apart."""
    active = int((counts > 0).sum())
    S = w.N * w.k
    d_in = w.d_in
    flops = 2.0 * S * 3 * d_in * w.d_ff + 6.0 * w.N * w.d * w.d_sh + 4.0 * w.N * w.d * w.L
    router_flops = 2.0 * w.N * w.d * w.E
    wbytes = active * 3 * d_in * w.d_ff * 2 + 3 * w.d * w.d_sh * 2 + 2 * w.d * w.L * 2
    io = w.N * w.d * 2 * 2 + w.E * w.d * 4 + w.E * 4 + S * 8
    # routed gate/up: w1 and w3 of the active experts + the experts' input once
    gate_up_bytes = active * 2 * d_in * w.d_ff * 2 + w.N * d_in * 2
    # routed down: w2 of the active experts
    down_bytes = active * d_in * w.d_ff * 2
    impl = {"gate_up_gathered_rows": S * d_in * 2, "gate_up_h_written": S * w.d_ff * 2,
            "down_h_read": S * w.d_ff * 2, "down_out_written": S * d_in * 2}
    return flops, router_flops, wbytes + io, gate_up_bytes, down_bytes, impl, active


def cpu_baseline(w, seconds):
    """The oracle on the host's cores: the router over all N tokens, timed once,
    and the experts + combine (+ projections) over a bounded token sample,
    repeated for about `seconds`.  The rate is N over the router time plus N
    times the sampled per-token time."""
    import numpy as np

    import oracle
    import synth

    x = synth.host_tensor(w, "hidden")
    wr = synth.host_tensor(w, "w_router")
    bias = synth.host_tensor(w, "bias")
    t0 = time.perf_counter()
    idx, wt, _ = oracle.route(x, wr, bias, w.G, w.TG, w.k, w.norm_topk_prob, w.route_scale)
    t_route = time.perf_counter() - t0
    n_tok = 8
    toks = np.arange(0, w.N, w.N // n_tok)[:n_tok]
    need = sorted({int(e) for e in idx[toks].ravel()})
    W = {n: {e: synth.host_tensor(w, n, expert=e) for e in need} for n in ("w1", "w3", "w2")}
    for n in ("sh_w1", "sh_w3", "sh_w2", "w_down", "w_up", "gamma"):
        if n in w.shapes():
            W[n] = synth.host_tensor(w, n)
    cfg = dict(d=w.d, E=w.E, k=w.k, d_ff=w.d_ff, d_sh=w.d_sh, L=w.L, act=w.act,
               situ_beta=w.situ_beta, situ_linear_beta=w.situ_linear_beta,
               latent_norm=w.latent_norm, norm_eps=w.norm_eps)
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.block_tokens(cfg, W, x, toks, idx[toks], wt[toks])
        done += n_tok
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_token = t_route / w.N + el / done
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"router on all {w.N} tokens ({t_route:.1f} s); experts, combine and "
                      f"projections on {n_tok} tokens (every {w.N // n_tok}th) repeated "
                      f"{done // n_tok}x ({el:.1f} s); rate = N / (router time + N x sampled "
                      f"per-token time)"}


def traffic_entry(workload, kernel):
    """Counter-measured bytes of one launch, if taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f).get(f"{workload}/{kernel}")
    if not tr or tr.get("gemm_source_digest") != gemm_source_digest():
        return None
    return tr


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(expert parallelism is a design, not an implementation)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_29_amd as m
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    m.binding.lib()
    w = synth.WORKLOADS[args.workload]
    cfg = m.make_config(d=w.d, n_experts=w.E, n_group=w.G, topk_group=w.TG, top_k=w.k,
                        d_ff=w.d_ff, route_scale=w.route_scale, norm_topk_prob=w.norm_topk_prob,
                        act=w.act, situ_beta=w.situ_beta, situ_linear_beta=w.situ_linear_beta,
                        d_latent=w.L, latent_norm=w.latent_norm, norm_eps=w.norm_eps,
                        d_ff_shared=w.d_sh,
                        dtype=m.DTYPE_BF16 if w.dtype == synth.BF16 else m.DTYPE_F32)
    dev = {}
    for name, shape in w.shapes().items():
        dt = torch.float32 if w.dtype_of(name) == synth.F32 else torch.bfloat16
        if name == "gamma" or (name == "bias" and w.bias_kind == "zipf"):
            dev[name] = torch.from_numpy(synth.host_tensor(w, name)).cuda()
        else:
            dev[name] = torch.empty(shape, dtype=dt, device="cuda")
            synth.fill_device(w, name, dev[name].data_ptr())
    weights = m.Weights(w_router=dev["w_router"], bias=dev["bias"], w1=dev["w1"], w3=dev["w3"],
                        w2=dev["w2"], w_down=dev.get("w_down"), gamma=dev.get("gamma"),
                        w_up=dev.get("w_up"), sh_w1=dev.get("sh_w1"), sh_w3=dev.get("sh_w3"),
                        sh_w2=dev.get("sh_w2"))
    ydt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float32
    y = torch.empty((w.N, w.d), dtype=ydt, device="cuda")
    counts = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    ws = m.workspace(cfg, w.N, m.CALL_BLOCK)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        m.moe_block_forward(cfg, w.N, weights, dev["hidden"], y, ws, tokens_per_expert_out=counts)
    torch.cuda.synchronize()

    hip = Hip()
    n_ev = len(STAGES) + 1
    events = [[hip.event() for _ in range(n_ev)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        arr = (ctypes.c_void_p * n_ev)(*[e.value for e in events[i]])
        m.binding.lib().moe_set_stage_events(arr, n_ev)
        m.moe_block_forward(cfg, w.N, weights, dev["hidden"], y, ws,
                            tokens_per_expert_out=counts, stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    m.binding.lib().moe_set_stage_events(None, 0)

    stage_ms = {s: 0.0 for s in STAGES}
    for i in range(args.steps):
        for j, s in enumerate(STAGES):
            stage_ms[s] += hip.elapsed_ms(events[i][j], events[i][j + 1]) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps
    cnt = counts.cpu().numpy()
    flops, router_flops, abytes, gu_bytes, dn_bytes, impl, active = algorithmic_work(w, cnt)
    sec = ms_per_step / 1e3
    gu_ms = stage_ms["gate_up"]
    dn_ms = stage_ms["down"]
    gu_gbs = gu_bytes / (gu_ms / 1e3) / 1e9
    traffic = traffic_entry(w.name, "gate_up")
    out = {
        "metric": METRIC,
        "value": w.N / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.BF16 else "f32",
        "data": "synthetic (seeded Philox normals; weights random, resident in HBM)",
        "config": {"workload": w.name, "tokens": w.N, "B": w.B, "T": w.T, "d": w.d,
                   "experts": w.E, "groups": w.G, "topk_group": w.TG, "top_k": w.k,
                   "d_ff": w.d_ff, "d_ff_shared": w.d_sh, "d_latent": w.L, "act": w.act,
                   "route_scale": w.route_scale, "parallelism": "single GPU"},
        "tflops": flops / sec / 1e12,
        "mfma_frac": flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "router_fp32_tflops": router_flops / sec / 1e12,
        "hbm_gbs": abytes / sec / 1e9,
        "hbm_frac": abytes / sec / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": abytes,
        "active_experts": active,
        "tokens_per_expert": {"min": int(cnt.min()), "max": int(cnt.max()),
                              "mean": float(cnt.mean())},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {"kernel": "moe_gemm_bf16 (routed gate/up, gathered rows, "
                               f"{w.act} epilogue)",
                     "bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gu_gbs / HBM_PEAK_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_ms": gu_ms,
                     "implementation_bytes_per_launch": {
                         "gathered_rows": impl["gate_up_gathered_rows"],
                         "h_written": impl["gate_up_h_written"]},
                     "traffic_source": traffic["source"] if traffic else None},
        "routed_down": {"achieved": dn_bytes / (dn_ms / 1e3) / 1e9, "unit": "GB/s",
                        "frac": dn_bytes / (dn_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                        "algorithmic_bytes_per_launch": dn_bytes, "avg_launch_ms": dn_ms},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
