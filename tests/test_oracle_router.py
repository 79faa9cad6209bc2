"""Pins for the oracle's router, checked against things other than itself.

- hand-worked examples (tests/golden/router_worked.json);
- brute force: the kept groups maximise the sum of group scores over all
  C(G, TG) subsets and the chosen experts maximise the sum of choice scores
  over all C(candidates, k) subsets;
- invariants the pages fix (k distinct experts inside the kept groups, weights
  summing to the route scale, the bias moving selection but never weights);
- closed forms (zero token, zero bias, dominant bias, one group, k = 1);
- the fp32 scores against numpy's float64 matrix product rounded to fp32.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def logit(p):
    return math.log(p / (1.0 - p))


def _golden_cases():
    with open(os.path.join(GOLDEN, "router_worked.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        for t, tok in enumerate(case["tokens"]):
            yield pytest.param(case, tok, id=f"{case['name']}-{t}")


@pytest.mark.parametrize("case,tok", list(_golden_cases()))
def test_worked_examples(case, tok):
    E = case["E"]
    score_func = case.get("score_func", "sigmoid")
    if score_func == "softmax":
        w_router = np.array([[math.log(q)] for q in case["q"]], np.float32)
    else:
        w_router = np.array([[logit(p)] for p in case["p"]], np.float32)
    bias = None if case["bias"] is None else np.array(case["bias"], np.float32)
    x = np.array([[tok["x"]]], np.float32)
    idx, w, flags = oracle.route(x, w_router, bias, case["G"], case["TG"], case["k"],
                                 case["norm_topk_prob"], case["route_scale"], score_func)
    assert idx[0].tolist() == tok["idx"]
    np.testing.assert_allclose(w[0], tok["weight"], rtol=1e-6)
    assert bool(flags[0] & oracle.FLAG_NEAR_TIE_EXPERT) == tok["near_tie"]
    assert E == w_router.shape[0]


def _random_choice(rng, E, spread=1.0):
    return rng.normal(0.5, spread, E).astype(np.float32)


@pytest.mark.parametrize("group_by_max", [False, True])
@pytest.mark.parametrize("E,G,TG,k", [(8, 4, 2, 3), (12, 3, 2, 4), (16, 4, 2, 4), (16, 8, 3, 5),
                                      (10, 1, 1, 3), (12, 6, 6, 2), (9, 3, 1, 3), (8, 2, 1, 1)])
def test_brute_force_selection(E, G, TG, k, group_by_max):
    rng = np.random.default_rng(E * 100 + G * 10 + k + 7 * group_by_max)
    per = E // G
    for _ in range(60):
        b = _random_choice(rng, E)
        idx, flags, _, _, gs = oracle.select(b, G, TG, k, group_by_max)
        # group scores: the two largest choice scores of each group summed in
        # fp32, or (a router without bias) the largest one
        for g in range(G):
            top2 = sorted(b[g * per:(g + 1) * per].tolist(), reverse=True)[:2]
            want = top2[0] if group_by_max else np.float32(np.float64(top2[0]) + np.float64(top2[1]))
            assert gs[g] == np.float32(want)
        best_groups = max(itertools.combinations(range(G), TG),
                          key=lambda s: sum(float(gs[g]) for g in s))
        cands = [e for e in range(E) if e // per in best_groups]
        best = max(itertools.combinations(cands, k), key=lambda s: sum(float(b[e]) for e in s))
        assert sorted(best) == idx.tolist()
        assert idx.tolist() == sorted(idx.tolist())


def test_invariants_on_tiny_workload():
    w = synth.WORKLOADS["tiny"]
    x = synth.host_tensor(w, "hidden")
    wr = synth.host_tensor(w, "w_router")
    bias = synth.host_tensor(w, "bias")
    idx, wt, flags = oracle.route(x, wr, bias, w.G, w.TG, w.k, True, w.route_scale)
    _, score, choice = oracle.router_scores(x, wr, bias)
    per = w.E // w.G
    for n in range(w.N):
        sel = idx[n].tolist()
        assert len(set(sel)) == w.k and sel == sorted(sel)
        gs = [sum(sorted(choice[n, g * per:(g + 1) * per].tolist(), reverse=True)[:2])
              for g in range(w.G)]
        kept = {e // per for e in sel}
        assert len(kept) <= w.TG
        # every kept group's score >= every dropped one's (up to fp32 of the sums)
        kept_full = sorted(range(w.G), key=lambda g: (-gs[g], g))[: w.TG]
        assert kept <= set(kept_full)
        cands = [e for e in range(w.E) if e // per in kept_full]
        assert min(choice[n, sel]) >= max(choice[n, e] for e in cands if e not in sel)
        # weights: the unbiased scores, renormalised, times the route scale
        np.testing.assert_allclose(wt[n].sum(), w.route_scale, rtol=1e-12)
        s64 = score[n, sel].astype(np.float64)
        np.testing.assert_allclose(wt[n], w.route_scale * s64 / s64.sum(), rtol=1e-12)
    assert not np.any(flags & oracle.FLAG_FILL_MATTERS)


def test_scores_match_library_matmul():
    w = synth.WORKLOADS["tiny"]
    x = synth.host_tensor(w, "hidden")
    wr = synth.host_tensor(w, "w_router")
    bias = synth.host_tensor(w, "bias")
    lg, s, b = oracle.router_scores(x, wr, bias)
    ref = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(lg, ref)
    np.testing.assert_allclose(s, 1.0 / (1.0 + np.exp(-ref.astype(np.float64))), rtol=1e-7)
    assert np.array_equal(b, (s + bias[None, :]).astype(np.float32))


def test_scores_from_bf16_hidden():
    w = synth.WORKLOADS["tiny"].scaled(dtype=synth.BF16)
    x = synth.host_tensor(w, "hidden")
    assert x.dtype == np.uint16
    wr = synth.host_tensor(w, "w_router")
    bias = synth.host_tensor(w, "bias")
    lg, _, _ = oracle.router_scores(x, wr, bias)
    ref = (synth.bf16_bits_to_f32(x).astype(np.float64) @ wr.astype(np.float64).T)
    assert np.array_equal(lg, ref.astype(np.float32))


def test_zero_token_closed_form():
    """A zero hidden row: logits 0, scores exactly 1/2, so the choice is the
    group rule applied to the bias alone and every weight is route_scale/k."""
    rng = np.random.default_rng(5)
    E, G, TG, k, d = 16, 4, 2, 4, 32
    x = np.zeros((1, d), np.float32)
    wr = rng.normal(0, 0.2, (E, d)).astype(np.float32)
    bias = rng.normal(0, 0.1, E).astype(np.float32)
    idx, w, _ = oracle.route(x, wr, bias, G, TG, k, True, 2.5)
    want, _, _, _, _ = oracle.select((np.float32(0.5) + bias).astype(np.float32), G, TG, k)
    assert idx[0].tolist() == want.tolist()
    assert np.all(w[0] == 2.5 / k)


def test_zero_bias_selects_top_scores():
    rng = np.random.default_rng(6)
    E, G, d, k = 24, 1, 16, 5
    x = rng.normal(0, 1, (20, d)).astype(np.float32)
    wr = rng.normal(0, 0.25, (E, d)).astype(np.float32)
    idx, _, _ = oracle.route(x, wr, np.zeros(E, np.float32), G, 1, k, True, 1.0)
    _, s, _ = oracle.router_scores(x, wr, np.zeros(E, np.float32))
    for n in range(20):
        assert idx[n].tolist() == sorted(np.argsort(-s[n], kind="stable")[:k].tolist())


def test_dominant_bias_forces_expert_without_changing_weights():
    rng = np.random.default_rng(7)
    E, G, TG, k, d = 16, 4, 2, 4, 32
    x = rng.normal(0, 1, (40, d)).astype(np.float32)
    wr = rng.normal(0, 0.2, (E, d)).astype(np.float32)
    bias = rng.normal(0, 0.01, E).astype(np.float32)
    bias[11] = 10.0
    idx, w, _ = oracle.route(x, wr, bias, G, TG, k, True, 2.5)
    _, s, _ = oracle.router_scores(x, wr, bias)
    assert all(11 in row for row in idx.tolist())  # every token: T_11 = N
    for n in range(40):
        s64 = s[n, idx[n]].astype(np.float64)
        np.testing.assert_allclose(w[n], 2.5 * s64 / s64.sum(), rtol=1e-12)


def test_single_group_is_plain_topk():
    rng = np.random.default_rng(8)
    E, k = 32, 6
    for _ in range(50):
        b = _random_choice(rng, E)
        idx, _, _, gg, _ = oracle.select(b, 1, 1, k)
        assert idx.tolist() == sorted(np.argsort(-b, kind="stable")[:k].tolist())
        assert gg == math.inf


def test_no_renorm_for_single_expert_or_flag_off():
    s = np.array([0.2, 0.9, 0.6, 0.5], np.float32)
    np.testing.assert_allclose(oracle.weights(s, np.array([1], np.int32), True, 3.0),
                               [np.float64(s[1]) * 3.0], rtol=0)
    np.testing.assert_allclose(oracle.weights(s, np.array([1, 2], np.int32), False, 3.0),
                               [np.float64(s[1]) * 3.0, np.float64(s[2]) * 3.0], rtol=0)


def test_near_tie_flags():
    b = np.array([0.9, 0.5, 0.5, 0.1], np.float32)
    _, f, ge, _, _ = oracle.select(b, 1, 1, 2)
    assert f & oracle.FLAG_NEAR_TIE_EXPERT and ge == 0.0
    b = np.array([0.9, 0.5, 0.4, 0.1], np.float32)
    _, f, ge, _, _ = oracle.select(b, 1, 1, 2)
    assert not f and abs(ge - 0.2) < 1e-6
    # groups {0,1} and {2,3} with equal top-2 sums
    b = np.array([0.9, 0.1, 0.5, 0.5], np.float32)
    _, f, _, gg, _ = oracle.select(b, 2, 1, 1)
    assert f & oracle.FLAG_NEAR_TIE_GROUP and gg == 0.0


def test_fill_matters_flag():
    # only one kept expert has a positive choice score: a 0.0 fill (instead of
    # -inf) for the dropped group would let its experts compete
    b = np.array([0.3, -0.2, -0.4, -0.5, 0.2, -0.9, -0.8, -0.7], np.float32)
    idx, f, _, _, _ = oracle.select(b, 2, 1, 2)
    assert f & oracle.FLAG_FILL_MATTERS
    assert idx.tolist() == [0, 1]


def test_valid_choice_rule():
    b = np.array([0.9, 0.5, 0.5, 0.1], np.float32)
    assert oracle.valid_choice(b, 1, 1, 2, [0, 1])
    assert oracle.valid_choice(b, 1, 1, 2, [0, 2])  # the tie may go either way
    assert not oracle.valid_choice(b, 1, 1, 2, [0, 3])
    assert not oracle.valid_choice(b, 1, 1, 2, [0, 0])
    b2 = np.array([0.9, 0.5, 0.4999999, 0.1], np.float32)
    assert oracle.valid_choice(b2, 1, 1, 2, [0, 2])  # within 2e-6 relative
    b3 = np.array([0.9, 0.5, 0.49, 0.1], np.float32)
    assert not oracle.valid_choice(b3, 1, 1, 2, [0, 2])
    bg = np.array([0.9, 0.1, 0.5, 0.5], np.float32)
    assert oracle.valid_choice(bg, 2, 1, 1, [0]) and oracle.valid_choice(bg, 2, 1, 1, [2])
    assert not oracle.valid_choice(bg, 2, 1, 1, [1])


def test_config_rejections():
    b = np.zeros(8, np.float32)
    for G, TG, k in [(3, 1, 1), (8, 1, 1), (4, 5, 1), (4, 0, 1), (4, 1, 3), (2, 1, 0)]:
        with pytest.raises(ValueError):
            oracle.select(b, G, TG, k)


# ---- softmax scoring and routers without a bias (DeepSeek-V3.2-Exp gate) ----

def test_softmax_scores_match_scipy():
    """Softmax scores: scipy's float64 softmax of the fp32 logits, rounded to
    fp32; they sum to one; without a bias the choice is the score."""
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    N, d, E = 40, 48, 24
    x = rng.normal(0, 1, (N, d)).astype(np.float32)
    wr = rng.normal(0, 1 / math.sqrt(d), (E, d)).astype(np.float32)
    lg, s, b = oracle.router_scores(x, wr, None, "softmax")
    ref = softmax(lg.astype(np.float64), axis=1).astype(np.float32)
    np.testing.assert_allclose(s, ref, rtol=2e-7, atol=0)
    np.testing.assert_allclose(s.astype(np.float64).sum(axis=1), 1.0, rtol=1e-6)
    assert np.array_equal(b, s)
    lg2, s2, b2 = oracle.router_scores(x, wr, None, "sigmoid")
    assert np.array_equal(lg, lg2) and np.array_equal(b2, s2)
    bias = rng.normal(0, 0.01, E).astype(np.float32)
    _, s3, b3 = oracle.router_scores(x, wr, bias, "softmax")
    assert np.array_equal(s3, s)
    np.testing.assert_allclose(b3, (s.astype(np.float64) + bias).astype(np.float32), rtol=0, atol=0)


@pytest.mark.parametrize("norm", [False, True])
def test_softmax_zero_token_closed_form(norm):
    """A zero token: every softmax score is 1/E, so the weights are route_scale/E
    (route_scale/k after renormalisation) and ties go to the lowest ids."""
    E, G, TG, k = 16, 4, 2, 3
    rng = np.random.default_rng(9)
    wr = rng.normal(0, 1, (E, 8)).astype(np.float32)
    x = np.zeros((1, 8), np.float32)
    idx, w, flags = oracle.route(x, wr, None, G, TG, k, norm, 3.0, "softmax")
    assert idx[0].tolist() == [0, 1, 2]
    np.testing.assert_allclose(w[0], 3.0 / k if norm else 3.0 / E, rtol=1e-7)
    assert flags[0] & oracle.FLAG_NEAR_TIE_EXPERT


def test_route_without_bias_invariants():
    """No bias, sigmoid and softmax: the chosen experts are the top-k scores of
    the groups kept by their largest score, weights are proportional to them."""
    rng = np.random.default_rng(12)
    N, d, E, G, TG, k = 64, 32, 32, 8, 3, 4
    x = rng.normal(0, 1, (N, d)).astype(np.float32)
    wr = rng.normal(0, 1 / math.sqrt(d), (E, d)).astype(np.float32)
    per = E // G
    for sf in ("sigmoid", "softmax"):
        idx, w, flags = oracle.route(x, wr, None, G, TG, k, True, 2.0, sf)
        _, s, _ = oracle.router_scores(x, wr, None, sf)
        for n in range(N):
            gmax = s[n].reshape(G, per).max(axis=1)
            kept = set(np.argsort(-gmax, kind="stable")[:TG].tolist())
            assert all(e // per in kept for e in idx[n])
            cand = [e for e in range(E) if e // per in kept]
            top = sorted(cand, key=lambda e: (-s[n, e], e))[:k]
            if not flags[n]:
                assert sorted(top) == idx[n].tolist()
            np.testing.assert_allclose(w[n], 2.0 * s[n, idx[n]] / s[n, idx[n]].astype(np.float64).sum(),
                                       rtol=1e-6)
