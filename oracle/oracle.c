/*
 * oracle.c - CPU oracle for the routed MoE block forward.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct fp64 reference,
 * written from the pages' description of the method (citation keys in
 * oracle.h).  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the GPU library shares no code with it and never calls it.
 *
 * What it computes, in the pages' order:
 *   router   - fp32 linear of the hidden state with the router weight, sigmoid
 *              scores, correction bias added for choice only, per-group sum of
 *              the two largest choice scores, the best topk_group groups kept,
 *              the top_k choice scores among them, the unbiased scores of the
 *              chosen experts renormalised and scaled      [K2-AFF], [V32-AFF]
 *   dispatch - per-expert token counts and the expert-sorted order of the
 *              flat (token, slot) pairs                                 [K3-ADD]
 *   experts  - per token and chosen expert, the gated MLP
 *              w2(act(w1 x) * (w3 x)) with SiLU, or with SiTU in its own form,
 *              summed with the routing weights                [K3-GATE], [K3-ADD]
 *   latent   - down projection before the experts, RMS normalisation and up
 *              projection after them; shared expert on the full-width input
 *              added to the output                                      [K3-ADD]
 *
 * Precision.  The router's decisions (which experts) are taken on fp32 values,
 * the precision the pages compute the router in: each logit is the exact dot
 * product rounded once to fp32, each score is sigmoid(logit) rounded once to
 * fp32, each choice score is the fp32 sum score + bias, each group score the
 * fp32 sum of two choice scores.  Everything continuous after that (weights,
 * expert MLPs, combine, norm, projections) is fp64 with no intermediate
 * rounding.  Ties are broken toward the lower index.
 *
 * Readings of points the pages leave open (listed with reasons in the design
 * notes): experts of dropped groups can never be chosen (the -inf fill of
 * [V32-AFF]; [K2-AFF] fills 0.0 - tokens where this matters are flagged); the
 * chosen experts are reported in ascending expert id; the dispatch order is
 * the stable one; renormalisation adds 1e-20 and is skipped for top_k = 1
 * ([K2-AFF]); RMS normalisation is y / sqrt(mean(y^2) + eps) * gamma.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Element i of an array stored as fp32 or as bf16 bits, widened exactly. */
static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
  return bf16_value(((const uint16_t*)p)[i]);
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* ------------------------------------------------------------------ router */

/* [K2-AFF] / [V32-AFF] gate forward: logits = x . W_r^T in fp32 (the fp64 sum
 * rounded once to fp32); score = sigmoid(logit), or ([V32-AFF]) the softmax of
 * the token's logits over all experts; choice = score + bias when the router
 * has a bias, else the score itself.  Each value is rounded to fp32, the
 * precision the pages compute in. */
int oracle_router_scores(int64_t N, int64_t d, int64_t E, const void* x, int x_dtype,
                         const float* w_router, const float* bias, int score_func, float* logit,
                         float* score, float* choice) {
  if (N < 0 || d <= 0 || E <= 0 || !x || !w_router || !score || !choice) return 1;
  if (score_func != ORACLE_SCORE_SIGMOID && score_func != ORACLE_SCORE_SOFTMAX) return 1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t n = 0; n < N; ++n) {
    float* l = (float*)malloc(sizeof(float) * (size_t)E);
    if (!l) {
      ++bad;
      continue;
    }
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i) acc += elem(x, x_dtype, n * d + i) * (double)w_router[e * d + i];
      l[e] = (float)acc;
    }
    double mx = -INFINITY, den = 0.0;
    if (score_func == ORACLE_SCORE_SOFTMAX) {
      for (int64_t e = 0; e < E; ++e) mx = (double)l[e] > mx ? (double)l[e] : mx;
      for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - mx);
    }
    for (int64_t e = 0; e < E; ++e) {
      const float s = score_func == ORACLE_SCORE_SOFTMAX ? (float)(exp((double)l[e] - mx) / den)
                                                         : (float)sigmoid((double)l[e]);
      const float b = bias ? (float)((double)s + (double)bias[e]) : s;
      if (logit) logit[n * E + e] = l[e];
      score[n * E + e] = s;
      choice[n * E + e] = b;
    }
    free(l);
  }
  return bad ? 2 : 0;
}

/* a beats b: larger value, then lower index. */
static int beats(float va, int64_t ia, float vb, int64_t ib) {
  if (va > vb) return 1;
  if (va < vb) return 0;
  return ia < ib;
}

static double rel_gap(float hi, float lo) {
  const double h = (double)hi;
  return (h - (double)lo) / fabs(h);
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* [K2-AFF]: groups are consecutive runs of E/G experts; a group's score is the
 * sum of its two largest choice scores (topk(2) then sum) -- or, for a router
 * without a bias ([V32-AFF]), its largest choice score (amax); the topk_group
 * groups with the largest scores are kept; the top_k largest choice scores
 * among the kept groups' experts are chosen.  [V32-AFF] fills the dropped
 * groups with -inf, so their experts are never chosen. */
int oracle_select(int64_t E, int G, int TG, int k, int group_by_max, const float* choice,
                  int32_t* idx_out, double* gap_expert, double* gap_group,
                  float* group_score_out) {
  if (E <= 0 || E > ORACLE_MAX_E || G <= 0 || E % G != 0 || TG < 1 || TG > G || k < 1) return -1;
  const int64_t per = E / G;
  if (per < 2 || (int64_t)k > (int64_t)TG * per) return -1;

  float gs[ORACLE_MAX_E];
  unsigned char kept[ORACLE_MAX_E];
  unsigned char chosen[ORACLE_MAX_E];
  int flags = 0;

  for (int g = 0; g < G; ++g) {
    float top1 = -INFINITY, top2 = -INFINITY;
    for (int64_t e = (int64_t)g * per; e < (int64_t)(g + 1) * per; ++e) {
      const float v = choice[e];
      if (v > top1) {
        top2 = top1;
        top1 = v;
      } else if (v > top2) {
        top2 = v;
      }
    }
    gs[g] = group_by_max ? top1 : (float)((double)top1 + (double)top2);
    kept[g] = 0;
    if (group_score_out) group_score_out[g] = gs[g];
  }

  /* keep TG groups, one at a time: the best group not yet kept */
  float last_kept = 0.0f;
  for (int t = 0; t < TG; ++t) {
    int best = -1;
    for (int g = 0; g < G; ++g)
      if (!kept[g] && (best < 0 || beats(gs[g], g, gs[best], best))) best = g;
    kept[best] = 1;
    last_kept = gs[best];
  }
  double gg = INFINITY;
  if (TG < G) {
    int next = -1;
    for (int g = 0; g < G; ++g)
      if (!kept[g] && (next < 0 || beats(gs[g], g, gs[next], next))) next = g;
    gg = rel_gap(last_kept, gs[next]);
    if (gg < ORACLE_NEAR_TIE_REL) flags |= ORACLE_FLAG_NEAR_TIE_GROUP;
  }

  /* choose k experts among the kept groups, one at a time */
  for (int64_t e = 0; e < E; ++e) chosen[e] = 0;
  float last_chosen = 0.0f;
  for (int j = 0; j < k; ++j) {
    int64_t best = -1;
    for (int64_t e = 0; e < E; ++e) {
      if (!kept[e / per] || chosen[e]) continue;
      if (best < 0 || beats(choice[e], e, choice[best], best)) best = e;
    }
    chosen[best] = 1;
    idx_out[j] = (int32_t)best;
    last_chosen = choice[best];
  }
  double ge = INFINITY;
  {
    int64_t next = -1;
    int64_t positive = 0;
    for (int64_t e = 0; e < E; ++e) {
      if (!kept[e / per]) continue;
      if (choice[e] > 0.0f) ++positive;
      if (chosen[e]) continue;
      if (next < 0 || beats(choice[e], e, choice[next], next)) next = e;
    }
    if (next >= 0) {
      ge = rel_gap(last_chosen, choice[next]);
      if (ge < ORACLE_NEAR_TIE_REL) flags |= ORACLE_FLAG_NEAR_TIE_EXPERT;
    }
    if (positive < k) flags |= ORACLE_FLAG_FILL_MATTERS;
  }
  qsort(idx_out, (size_t)k, sizeof(int32_t), cmp_i32);
  if (gap_expert) *gap_expert = ge;
  if (gap_group) *gap_group = gg;
  return flags;
}

/* [K2-AFF]: topk_weight = scores.gather(idx) (the unbiased scores); when
 * top_k > 1 and norm_topk_prob, divide by their sum + 1e-20; then multiply by
 * routed_scaling_factor.  [V32-AFF] does the same with route_scale. */
void oracle_weights(int k, int norm_topk_prob, double route_scale, const float* score,
                    const int32_t* idx, double* w_out) {
  for (int j = 0; j < k; ++j) w_out[j] = (double)score[idx[j]];
  if (k > 1 && norm_topk_prob) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += w_out[j];
    for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / (sum + 1e-20);
  }
  for (int j = 0; j < k; ++j) w_out[j] = w_out[j] * route_scale;
}

int oracle_route(int64_t N, int64_t d, int64_t E, int G, int TG, int k, int norm_topk_prob,
                 double route_scale, int score_func, const void* x, int x_dtype,
                 const float* w_router, const float* bias, int32_t* topk_idx, double* topk_weight,
                 uint8_t* flags) {
  if (N < 0 || E <= 0 || E > ORACLE_MAX_E || k < 1) return 1;
  if (N == 0) return 0;
  float* score = (float*)malloc(sizeof(float) * (size_t)(N * E));
  float* choice = (float*)malloc(sizeof(float) * (size_t)(N * E));
  if (!score || !choice) {
    free(score);
    free(choice);
    return 2;
  }
  int rc = oracle_router_scores(N, d, E, x, x_dtype, w_router, bias, score_func, NULL, score,
                                choice);
  int bad = 0;
  if (rc == 0) {
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t n = 0; n < N; ++n) {
      const int f = oracle_select(E, G, TG, k, bias == NULL, choice + n * E, topk_idx + n * k,
                                  NULL, NULL, NULL);
      if (f < 0) {
        ++bad;
        continue;
      }
      if (flags) flags[n] = (uint8_t)f;
      oracle_weights(k, norm_topk_prob, route_scale, score + n * E, topk_idx + n * k,
                     topk_weight + n * k);
    }
  }
  free(score);
  free(choice);
  return rc ? rc : (bad ? 3 : 0);
}

/* ---------------------------------------------------------------- dispatch */

/* [K3-ADD] moe_infer: tokens_per_expert is the column sum of the one-hot
 * [N, E] count matrix; idxs = argsort of the flattened chosen experts, so
 * sorted position p holds flat slot idxs[p] = n*k + j, grouped by expert.
 * Written here straight from that definition, with the stable order: expert
 * by expert, and within an expert the flat slots in increasing order. */
int oracle_counts_perm(int64_t N, int k, int64_t E, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm) {
  if (N < 0 || k < 1 || E <= 0) return 1;
  const int64_t S = N * (int64_t)k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < S; ++f) {
    const int32_t e = topk_idx[f];
    if (e < 0 || e >= E) return 2;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t p = 0;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t f = 0; f < S; ++f)
      if (topk_idx[f] == e) perm[p++] = (int32_t)f;
  for (int64_t q = 0; q < S; ++q) inv_perm[perm[q]] = (int32_t)q;
  return 0;
}

/* ------------------------------------------------------------------ experts */

/* [K3-GATE] expert: SiLU experts compute act_fn(w1(x)) * w3(x); SiTU experts
 * (situ excerpt) compute, in float32 on the pages, beta*tanh(gate/beta)*
 * sigmoid(gate) times the up branch, the up branch first passed through
 * linear_beta*tanh(up/linear_beta) when linear_beta is set; gate is w1(x),
 * up is w3(x). */
static double act_pair(const oracle_block_cfg* c, double g, double u) {
  if (c->act == ORACLE_ACT_SILU) return g * sigmoid(g) * u;
  const double beta = c->situ_beta;
  const double a = beta * tanh(g / beta) * sigmoid(g);
  if (c->situ_linear_beta > 0.0) u = c->situ_linear_beta * tanh(u / c->situ_linear_beta);
  return a * u;
}

/* The two halves of one gated MLP for one row, with w1, w3 stored
 * [d_hidden, d_model] and w2 stored [d_model, d_hidden] (nn.Linear [out, in],
 * no bias - [K3-GATE] expert):  h = act(w1 v, w3 v),  o = w2 h. */
static void gate_up_vec(const oracle_block_cfg* c, const void* w1, const void* w3, int64_t d_model,
                        int64_t d_hidden, const double* v, double* h) {
  for (int64_t i = 0; i < d_hidden; ++i) {
    double g = 0.0, u = 0.0;
    for (int64_t t = 0; t < d_model; ++t) {
      g += elem(w1, c->dtype, i * d_model + t) * v[t];
      u += elem(w3, c->dtype, i * d_model + t) * v[t];
    }
    h[i] = act_pair(c, g, u);
  }
}

static void down_vec(const oracle_block_cfg* c, const void* w2, int64_t d_model, int64_t d_hidden,
                     const double* h, double* o) {
  for (int64_t t = 0; t < d_model; ++t) {
    double acc = 0.0;
    for (int64_t i = 0; i < d_hidden; ++i) acc += elem(w2, c->dtype, t * d_hidden + i) * h[i];
    o[t] = acc;
  }
}

static void gated_mlp(const oracle_block_cfg* c, const void* w1, const void* w3, const void* w2,
                      int64_t d_model, int64_t d_hidden, const double* v, double* h, double* o) {
  gate_up_vec(c, w1, w3, d_model, d_hidden, v, h);
  down_vec(c, w2, d_model, d_hidden, h, o);
}

/* Per-row halves on given rows (each row with its expert), for checking the
 * expert calls on their own: h[r] = act(w1[e] x[r], w3[e] x[r]) and
 * out[r] = w2[e] h[r], fp64, with x and h rows of the block's element type. */
int oracle_gate_up_rows(const oracle_block_cfg* c, const void* const* w1, const void* const* w3,
                        int64_t R, const void* x_rows, const int32_t* expert, double* h) {
  const int64_t d_in = c->L ? c->L : c->d;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : bad)
  for (int64_t r = 0; r < R; ++r) {
    const int32_t e = expert[r];
    double* v = (double*)malloc(sizeof(double) * (size_t)d_in);
    if (!v || e < 0 || e >= c->E || !w1[e] || !w3[e]) {
      free(v);
      ++bad;
      continue;
    }
    for (int64_t t = 0; t < d_in; ++t) v[t] = elem(x_rows, c->dtype, r * d_in + t);
    gate_up_vec(c, w1[e], w3[e], d_in, c->d_ff, v, h + r * c->d_ff);
    free(v);
  }
  return bad ? 2 : 0;
}

int oracle_down_rows(const oracle_block_cfg* c, const void* const* w2, int64_t R,
                     const void* h_rows, const int32_t* expert, double* out) {
  const int64_t d_in = c->L ? c->L : c->d;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : bad)
  for (int64_t r = 0; r < R; ++r) {
    const int32_t e = expert[r];
    double* h = (double*)malloc(sizeof(double) * (size_t)c->d_ff);
    if (!h || e < 0 || e >= c->E || !w2[e]) {
      free(h);
      ++bad;
      continue;
    }
    for (int64_t t = 0; t < c->d_ff; ++t) h[t] = elem(h_rows, c->dtype, r * c->d_ff + t);
    down_vec(c, w2[e], d_in, c->d_ff, h, out + r * d_in);
    free(h);
  }
  return bad ? 2 : 0;
}

/* [K3-ADD] moe_infer, last step: new_x[idxs] = outs un-permutes the expert
 * rows; the k rows of a token are multiplied by their routing weights and
 * summed; here in fp64, plus an optional residual row. */
int oracle_combine(int64_t N, int k, int64_t width, int dtype, const void* out_sorted,
                   const int32_t* inv_perm, const float* w, const void* residual, double* y) {
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t c = 0; c < width; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        const int64_t p = inv_perm[n * k + j];
        acc += (double)w[n * k + j] * elem(out_sorted, dtype, p * width + c);
      }
      if (residual) acc += elem(residual, dtype, n * width + c);
      y[n * width + c] = acc;
    }
  }
  return 0;
}

/* [K3-ADD] forward: the router scores the full-width input; with the latent
 * option the input is projected down first; moe_infer sums, per token, the
 * chosen experts' outputs times their weights (in the routing weight's
 * precision); with the latent option the sum is normalised and projected up;
 * the shared experts' output on the full-width input is added last. */
int oracle_block_tokens(const oracle_block_cfg* c, const oracle_block_weights* W, const void* x,
                        int64_t n_tok, const int64_t* tokens, const int32_t* idx, const double* w,
                        double* y) {
  if (!c || !W || !x || n_tok < 0) return 1;
  const int64_t d = c->d, L = c->L, d_in = L ? L : c->d;
  const int64_t hmax = c->d_ff > c->d_sh ? c->d_ff : c->d_sh;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
  for (int64_t t = 0; t < n_tok; ++t) {
    double* xv = (double*)malloc(sizeof(double) * (size_t)d);
    double* xin = (double*)malloc(sizeof(double) * (size_t)d_in);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d_in);
    double* o = (double*)malloc(sizeof(double) * (size_t)(d > d_in ? d : d_in));
    double* h = (double*)malloc(sizeof(double) * (size_t)(hmax > 0 ? hmax : 1));
    double* yt = y + t * d;
    if (!xv || !xin || !acc || !o || !h) {
      ++bad;
      goto done;
    }
    const int64_t n = tokens[t];
    for (int64_t i = 0; i < d; ++i) xv[i] = elem(x, c->dtype, n * d + i);

    /* latent down projection (routed_expert_down_proj) */
    if (L) {
      for (int64_t r = 0; r < L; ++r) {
        double a = 0.0;
        for (int64_t i = 0; i < d; ++i) a += elem(W->w_down, c->dtype, r * d + i) * xv[i];
        xin[r] = a;
      }
    } else {
      for (int64_t i = 0; i < d; ++i) xin[i] = xv[i];
    }

    /* moe_infer: weighted sum over the chosen experts, slots in order */
    for (int64_t i = 0; i < d_in; ++i) acc[i] = 0.0;
    for (int j = 0; j < c->k; ++j) {
      const int32_t e = idx[t * c->k + j];
      if (e < 0 || e >= c->E || !W->w1[e] || !W->w3[e] || !W->w2[e]) {
        ++bad;
        goto done;
      }
      gated_mlp(c, W->w1[e], W->w3[e], W->w2[e], d_in, c->d_ff, xin, h, o);
      for (int64_t i = 0; i < d_in; ++i) acc[i] += w[t * c->k + j] * o[i];
    }

    if (L) {
      /* routed_expert_norm, then routed_expert_up_proj */
      if (c->latent_norm) {
        double ss = 0.0;
        for (int64_t i = 0; i < L; ++i) ss += acc[i] * acc[i];
        const double r = 1.0 / sqrt(ss / (double)L + c->norm_eps);
        for (int64_t i = 0; i < L; ++i) acc[i] = acc[i] * r * (double)W->gamma[i];
      }
      for (int64_t r = 0; r < d; ++r) {
        double a = 0.0;
        for (int64_t i = 0; i < L; ++i) a += elem(W->w_up, c->dtype, r * L + i) * acc[i];
        yt[r] = a;
      }
    } else {
      for (int64_t i = 0; i < d; ++i) yt[i] = acc[i];
    }

    /* y = y + shared_experts(identity) */
    if (c->d_sh) {
      gated_mlp(c, W->sh_w1, W->sh_w3, W->sh_w2, d, c->d_sh, xv, h, o);
      for (int64_t i = 0; i < d; ++i) yt[i] += o[i];
    }
  done:
    free(xv);
    free(xin);
    free(acc);
    free(o);
    free(h);
  }
  return bad ? 2 : 0;
}
