/*
 * oracle.h - interface of the CPU oracle for the MoE block forward.
 *
 * TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow, obviously correct
 * fp64 CPU implementation written from the pages' description of the method;
 * it exists to check the GPU library against.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code, header
 * or table with the GPU library, and the GPU library never calls it.
 *
 * Page citations (the pages are web pages quoting model source):
 *   [K2-AFF]  "Kimi K2 - Affinities", gate-forward excerpt (MoEGate.forward)
 *             and gate-init excerpt (MoEGate.__init__)
 *   [K3-ADD]  "Kimi K3 - Add shared output" (prefill), moe-forward excerpt
 *             (KimiSparseMoeBlock.forward and moe_infer)
 *   [K3-GATE] "Kimi K3 - Gate features" (decode), expert excerpt
 *             (KimiBlockSparseMLP) and situ excerpt (SituAndMul)
 *   [V32-AFF] "DeepSeek-V3.2-Exp - Affinities", gate-forward and gate-init
 *             excerpts (Gate.forward, Gate.__init__)
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_ACT_SILU 0
#define ORACLE_ACT_SITU 1

/* Per-token flags written by oracle_route. */
#define ORACLE_FLAG_NEAR_TIE_EXPERT 1 /* k-th and (k+1)-th choice scores within 1e-6 rel */
#define ORACLE_FLAG_NEAR_TIE_GROUP 2  /* TG-th and (TG+1)-th group scores within 1e-6 rel */
#define ORACLE_FLAG_FILL_MATTERS 4    /* fewer than k kept experts have a positive choice
                                         score: a 0.0 fill would change the choice */

#define ORACLE_MAX_E 4096
#define ORACLE_NEAR_TIE_REL 1e-6

int oracle_num_threads(void);

#define ORACLE_SCORE_SIGMOID 0
#define ORACLE_SCORE_SOFTMAX 1

/* Router scores for all tokens, rounded to fp32 as the pages compute them:
 * logit (fp32 linear), score = sigmoid(logit) or softmax over the experts,
 * choice = score + bias (bias may be NULL: choice = score). */
int oracle_router_scores(int64_t N, int64_t d, int64_t E, const void* x, int x_dtype,
                         const float* w_router, const float* bias, int score_func, float* logit,
                         float* score, float* choice);

/* Group pruning and expert choice for one token from its choice scores:
 * idx_out[k] ascending; gap_expert / gap_group are the relative gaps at the
 * k-th / TG-th boundary (+inf when there is no competitor). Returns flags. */
int oracle_select(int64_t E, int G, int TG, int k, int group_by_max, const float* choice,
                  int32_t* idx_out, double* gap_expert, double* gap_group,
                  float* group_score_out);

/* Routing weights for one token from its scores and chosen experts. */
void oracle_weights(int k, int norm_topk_prob, double route_scale, const float* score,
                    const int32_t* idx, double* w_out);

/* Full router: scores, selection, weights for all N tokens. */
int oracle_route(int64_t N, int64_t d, int64_t E, int G, int TG, int k, int norm_topk_prob,
                 double route_scale, int score_func, const void* x, int x_dtype,
                 const float* w_router, const float* bias, int32_t* topk_idx, double* topk_weight,
                 uint8_t* flags);

/* Per-expert counts, offsets and the stable dispatch permutation. */
int oracle_counts_perm(int64_t N, int k, int64_t E, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm);

typedef struct {
  int64_t d;     /* model width */
  int64_t E;     /* routed experts */
  int32_t k;     /* experts per token */
  int64_t d_ff;  /* routed expert intermediate width */
  int64_t d_sh;  /* shared expert intermediate width, 0 = none */
  int64_t L;     /* latent width, 0 = none (then d_in = d) */
  int32_t act;   /* ORACLE_ACT_* */
  double situ_beta;
  double situ_linear_beta; /* <= 0: none */
  int32_t latent_norm;
  double norm_eps;
  int32_t dtype; /* element type of x and of every expert/shared/latent weight */
} oracle_block_cfg;

typedef struct {
  const void* const* w1; /* E pointers, each [d_ff, d_in]; NULL for unused experts */
  const void* const* w3; /* E pointers, each [d_ff, d_in] */
  const void* const* w2; /* E pointers, each [d_in, d_ff] */
  const void* sh_w1;     /* [d_sh, d] */
  const void* sh_w3;     /* [d_sh, d] */
  const void* sh_w2;     /* [d, d_sh] */
  const void* w_down;    /* [L, d] */
  const void* w_up;      /* [d, L] */
  const float* gamma;    /* [L] */
} oracle_block_weights;

/* Block output rows y[t] (fp64, [n_tok, d]) for tokens tokens[t] of x ([N, d]),
 * given their chosen experts idx[t][k] and weights w[t][k]. */
int oracle_block_tokens(const oracle_block_cfg* cfg, const oracle_block_weights* wts,
                        const void* x, int64_t n_tok, const int64_t* tokens,
                        const int32_t* idx, const double* w, double* y);

/* Expert halves on given rows: h [R, d_ff] and out [R, d_in] in fp64. */
int oracle_gate_up_rows(const oracle_block_cfg* cfg, const void* const* w1, const void* const* w3,
                        int64_t R, const void* x_rows, const int32_t* expert, double* h);
int oracle_down_rows(const oracle_block_cfg* cfg, const void* const* w2, int64_t R,
                     const void* h_rows, const int32_t* expert, double* out);

/* Weighted combine: y [N, width] fp64 from expert rows (dtype), inv_perm,
 * fp32 routing weights and an optional residual (dtype). */
int oracle_combine(int64_t N, int k, int64_t width, int dtype, const void* out_sorted,
                   const int32_t* inv_perm, const float* w, const void* residual, double* y);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
