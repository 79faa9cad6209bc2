"""The routed-expert GEMMs at full size, every row of selected experts.

For each full workload the expert calls run at full width on the workload's
real segment table (the oracle's routing of every token), in the launch
configuration the block uses: the gathered gate/up (rows read from the
experts' input through the permutation, as moe_block_forward runs it) and the
down product.  Every row of these experts is compared with the oracle:
  - the hottest expert (all of its m-tiles) and the coldest non-empty one;
  - the first and the last expert of each of the eight XCD runs the dispatch
    scan cuts the experts into (tiles at the run boundaries), and experts 0
    and E-1.
Inputs are seeded: the device fills whole tensors in place and the host
regenerates, counter by counter, only the rows and experts it compares.  The
down product takes an independent seeded input of h's shape.

The decode workload is also checked on its whole block output: y of all 256
tokens against the oracle."""
import time

import numpy as np
import pytest

import oracle
import synth
from moe_testlib import (as_f64, assert_close_bf16, cfg_of, device_inputs, moe, needs_gpu,
                         oracle_cfg, resolve_routing, to_device, to_host, torch, weights_of)

pytestmark = [pytest.mark.gpu, needs_gpu]

# seeded stand-ins for the experts' input in latent mode and for h (no tensor
# of the workload uses these seeds)
XIN_SEED, XIN_TID = 11, 1
H_SEED, H_TID, H_STD = 12, 1, 0.5


def tile_rows(w) -> int:
    """Rows per m-tile the library picks for the workload (tile height policy:
    256 rows from 64 routed rows per expert on average, 128 from 24, 64 from
    12, else 32)."""
    avg = w.N * w.k / w.E
    return 256 if avg >= 64 else 128 if avg >= 24 else 64 if avg >= 12 else 32


def xcd_run_starts(counts, rows_per_tile):
    """First expert of each of the 8 runs of about equal cost (4 per m-tile, 1
    per 32-row block), as the dispatch scan splits them."""
    mt = (counts + rows_per_tile - 1) // rows_per_tile
    cost = mt * 4 + (counts + 31) // 32
    start = np.cumsum(cost) - cost
    total = int(cost.sum())
    out = [0]
    for x in range(1, 8):
        mark = (total * x + 7) // 8
        hit = np.flatnonzero(start >= mark)
        out.append(int(hit[0]) if hit.size else len(counts))
    return out


def chosen_experts(counts, rows_per_tile):
    E = len(counts)
    nz = np.flatnonzero(counts)
    pick = {int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), 0, E - 1}
    for s in xcd_run_starts(counts, rows_per_tile):
        pick.update({s, s - 1})
    return sorted(e for e in pick if 0 <= e < E and counts[e] > 0)


def fill_dev(shape, seed, tid, std):
    t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    rc = synth._load_dev().synth_dev_fill_normal(t.data_ptr(), synth.BF16, int(np.prod(shape)), 0,
                                                 seed, tid, std, 0)
    assert rc == 0
    return t


def host_rows(width, r0, r1, seed, tid, std):
    return synth.fill_normal_host((r1 - r0) * width, r0 * width, seed, tid, std,
                                  synth.BF16).reshape(r1 - r0, width)


@pytest.mark.parametrize("name", ["dsv3_prefill", "k2_prefill", "k2_decode", "k3_latent_prefill"])
def test_expert_rows_full_size(name):
    w = synth.WORKLOADS[name]
    t0 = time.time()
    print(f"full-size expert rows: {name} N={w.N} E={w.E} d_in={w.d_in}", flush=True)
    m = moe()
    cfg = cfg_of(w)
    x = synth.host_tensor(w, "hidden")
    idx, _, _ = oracle.route(x, synth.host_tensor(w, "w_router"), synth.host_tensor(w, "bias"),
                             w.G, w.TG, w.k, w.norm_topk_prob, w.route_scale)
    counts, offsets, perm, _ = oracle.counts_perm(idx, w.E)
    S = w.N * w.k
    # the experts' input: the hidden state, or a seeded stand-in of the latent width
    if w.L:
        x_dev = fill_dev((w.N, w.d_in), XIN_SEED, XIN_TID, 1.0)
        x_in = host_rows(w.d_in, 0, w.N, XIN_SEED, XIN_TID, 1.0)
    else:
        x_dev = to_device(x, True)
        x_in = x
    W = {}
    for n in ("w1", "w3", "w2"):
        W[n] = torch.empty(w.shapes()[n], dtype=torch.bfloat16, device="cuda")
        synth.fill_device(w, n, W[n].data_ptr())
    h = torch.empty((S, w.d_ff), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gate_up_gather(cfg, w.N, x_dev, torch.from_numpy(perm).cuda(),
                                torch.from_numpy(offsets).cuda(), W["w1"], W["w3"], h,
                                m.workspace(cfg, w.N, m.CALL_GATE_UP))
    h_in = fill_dev((S, w.d_ff), H_SEED, H_TID, H_STD)
    out = torch.empty((S, w.d_in), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_down(cfg, w.N, h_in, torch.from_numpy(offsets).cuda(), W["w2"], out,
                      m.workspace(cfg, w.N, m.CALL_DOWN))
    torch.cuda.synchronize()
    del W
    ocfg = oracle_cfg(w)
    experts = chosen_experts(counts, tile_rows(w))
    print(f"  experts {experts} (rows {[int(counts[e]) for e in experts]})", flush=True)
    rows = 0
    for e in experts:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        erow = np.full(r1 - r0, e, np.int32)
        xr = x_in[perm[r0:r1] // w.k]
        h_ref = oracle.gate_up_rows(ocfg, {e: synth.host_tensor(w, "w1", expert=e)},
                                    {e: synth.host_tensor(w, "w3", expert=e)}, xr, erow)
        # h is stored in bf16: an element beyond 12.8 rms moves by more than 5e-2 rms
        # from that rounding alone (h's tail reaches ~15 rms here), so each element
        # is allowed half a bf16 ulp of its own magnitude on top of the bar
        r_h, m_h = assert_close_bf16(as_f64(to_host(h[r0:r1])), h_ref, f"{name} gate/up e={e}",
                                     output_rounding_slack=True)
        hr = host_rows(w.d_ff, r0, r1, H_SEED, H_TID, H_STD)
        o_ref = oracle.down_rows(ocfg, {e: synth.host_tensor(w, "w2", expert=e)}, hr, erow)
        r_o, m_o = assert_close_bf16(as_f64(to_host(out[r0:r1])), o_ref, f"{name} down e={e}")
        rows += r1 - r0
        print(f"  e={e} rows={r1 - r0}: h rel L2 {r_h:.2e} max/rms {m_h:.2e}; out rel L2 "
              f"{r_o:.2e} max/rms {m_o:.2e}", flush=True)
    assert np.all(np.isfinite(as_f64(to_host(h))))
    assert np.all(np.isfinite(as_f64(to_host(out))))
    print(f"  {rows} rows of {len(experts)} experts compared in {time.time() - t0:.1f} s",
          flush=True)


def test_decode_block_output_all_tokens():
    """y on every token of the decode workload.  The oracle takes the expert
    weights from the seeded generator's device fill (bit-identical to the host
    fill, as the synth tests check), copied back to the host: regenerating the
    382 touched experts on the host would take minutes."""
    w = synth.WORKLOADS["k2_decode"]
    t0 = time.time()
    print(f"decode block output, all {w.N} tokens", flush=True)
    m = moe()
    cfg = cfg_of(w)
    dev = device_inputs(w, on_device_gen=True)
    y = torch.empty((w.N, w.d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
    m.moe_block_forward(cfg, w.N, weights_of(dev, w), dev["hidden"], y, m.workspace(
        cfg, w.N, m.CALL_BLOCK), idx, wt)
    torch.cuda.synchronize()
    x = synth.host_tensor(w, "hidden")
    r_idx, r_w, _, n_res = resolve_routing(x, synth.host_tensor(w, "w_router"),
                                           synth.host_tensor(w, "bias"), w, idx.cpu().numpy(),
                                           wt.cpu().numpy())
    for e in (0, int(r_idx[0, 0])):  # spot check: the device fill is the host fill
        assert np.array_equal(to_host(dev["w2"][e]), synth.host_tensor(w, "w2", expert=e))
    W = {n: to_host(dev[n]) for n in ("w1", "w3", "w2", "sh_w1", "sh_w3", "sh_w2")}
    del dev
    y_ref = oracle.block_tokens(oracle_cfg(w), W, x, np.arange(w.N), r_idx, r_w)
    r, m_rel = assert_close_bf16(as_f64(to_host(y)), y_ref, "k2_decode y")
    print(f"  near ties resolved: {n_res}; y rel L2 {r:.2e}, max err / rms {m_rel:.2e} "
          f"({time.time() - t0:.1f} s)", flush=True)
