/*
 * moe.h - C ABI of libmoe: the inference forward of a DeepSeek-V3 / Kimi style
 * routed mixture-of-experts block on one AMD Instinct MI355X (gfx950).
 *
 * The operations follow these web pages, which quote the models' source:
 *   [K2-AFF]  "Kimi K2 - Affinities" (OpenModelAtlas), gate-forward excerpt
 *             (MoEGate.forward) and gate-init excerpt (MoEGate.__init__)
 *   [V32-AFF] "DeepSeek-V3.2-Exp - Affinities", gate-forward and gate-init
 *             excerpts (Gate.forward, Gate.__init__)
 *   [K3-ADD]  "Kimi K3 - Add shared output" (prefill), moe-forward excerpt
 *             (KimiSparseMoeBlock.forward and moe_infer)
 *   [K3-GATE] "Kimi K3 - Gate features" (decode), expert excerpt
 *             (KimiBlockSparseMLP) and situ excerpt (SituAndMul)
 *
 * Conventions for every call below.
 *  - Tensor arguments are DEVICE pointers to memory the caller owns (e.g.
 *    allocated by PyTorch); libmoe allocates no memory and frees none.
 *    Scratch space comes from the caller's `workspace` (device memory of at
 *    least moe_workspace_size(...) bytes, 256-byte aligned); its contents on
 *    entry are ignored and on return are unspecified.
 *  - All tensors are dense and row-major, with the shapes given per call.
 *    Weight matrices use the nn.Linear layout [out_features, in_features].
 *    Element type "dtype" is cfg->dtype (fp32, or bf16 as 16-bit patterns);
 *    the router weight, the correction bias, routing weights and the latent
 *    norm weight are always fp32; indices are int32.
 *  - Every tensor pointer must be non-NULL (unless marked optional) and
 *    16-byte aligned; every width (d, d_ff, d_latent, d_ff_shared) must be a
 *    positive multiple of 8.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without waiting for it.  Outputs are valid once the
 *    stream reaches that point.  Calls never synchronise with the host.
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error nothing is enqueued, outputs are untouched, the status says why and
 *    moe_last_error() gives a message.  No C++ exception crosses this ABI.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    must not share outputs or a workspace.
 *  - Results are deterministic: the same inputs give the same bits.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment or config value */
  MOE_ERR_UNSUPPORTED = 2, /* a mode the pages allow but libmoe does not run */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* [K3-GATE]: experts use SiLU (act_fn(w1 x) * w3 x) or SiTU. */
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_SITU = 1 } moe_act;

/* [K2-AFF] scores with the sigmoid of each logit; [V32-AFF] also offers the
 * softmax of the token's logits over all experts. */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score_func;

/* [K2-AFF] raises for any top-k method other than noaux_tc. */
typedef enum { MOE_TOPK_NOAUX_TC = 0 } moe_topk_method;

/* Which call a workspace is sized for (moe_workspace_size). */
typedef enum {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_PERMUTE = 1,
  MOE_CALL_GATE_UP = 2,
  MOE_CALL_DOWN = 3,
  MOE_CALL_COMBINE = 4,
  MOE_CALL_BLOCK = 5,
  MOE_CALL_SHARED = 6,
  MOE_CALL_LATENT = 7
} moe_call;

/* Block configuration; field names follow the pages' config fields. */
typedef struct {
  int64_t d;               /* hidden_size: router input width and block width */
  int64_t n_experts;       /* E = n_routed_experts, 2 <= E <= 1024 */
  int32_t n_group;         /* G = n_group; E % G == 0 and E / G >= 2 */
  int32_t topk_group;      /* TG = topk_group, 1 <= TG <= G */
  int32_t top_k;           /* k = num_experts_per_tok, 1 <= k <= min(16, TG * E / G) */
  int32_t norm_topk_prob;  /* renormalise the k weights (applied only when k > 1) */
  float route_scale;       /* routed_scaling_factor */
  int32_t score_func;      /* moe_score_func: SIGMOID or SOFTMAX */
  int32_t topk_method;     /* moe_topk_method: NOAUX_TC */
  int32_t training;        /* must be 0: inference only (training -> UNSUPPORTED) */
  int64_t d_ff;            /* moe_intermediate_size of a routed expert */
  int32_t act;             /* moe_act, for routed and shared experts */
  float situ_beta;         /* activation_situ_beta; 0 means 1.0 */
  float situ_linear_beta;  /* activation_situ_linear_beta; <= 0 means none */
  int64_t d_latent;        /* L: width of the latent experts; 0 = no latent MoE */
  int32_t latent_norm;     /* latent_moe_use_norm */
  float norm_eps;          /* epsilon of the latent RMS norm */
  int64_t d_ff_shared;     /* intermediate width of the shared expert; 0 = none */
  int32_t dtype;           /* moe_dtype of hidden, weights (but router/bias/gamma), outputs */
} moe_config;

/* Weights of one block.  d_in = d_latent if d_latent > 0, else d. */
typedef struct {
  const float* w_router;  /* [E, d] fp32 router weight ([K2-AFF] gate-init) */
  const float* bias;      /* [E] fp32 e_score_correction_bias, choice only; NULL: none */
  const void* w1;         /* [E, d_ff, d_in] dtype, gate projections */
  const void* w3;         /* [E, d_ff, d_in] dtype, up projections */
  const void* w2;         /* [E, d_in, d_ff] dtype, down projections */
  const void* w_down;     /* [L, d] dtype, latent down projection (latent only) */
  const float* gamma;     /* [L] fp32, latent RMS-norm weight (latent_norm only) */
  const void* w_up;       /* [d, L] dtype, latent up projection (latent only) */
  const void* sh_w1;      /* [d_ff_shared, d] dtype, shared gate (shared only) */
  const void* sh_w3;      /* [d_ff_shared, d] dtype, shared up */
  const void* sh_w2;      /* [d, d_ff_shared] dtype, shared down */
} moe_weights;

/* Host-only helpers (no device work). */
const char* moe_status_str(moe_status s);
/* Message for the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);
/* Checks a configuration alone: the limits listed in moe_config. */
moe_status moe_validate_config(const moe_config* cfg);
/* Workspace bytes `call` needs for N tokens (0 for MOE_CALL_COMBINE). */
moe_status moe_workspace_size(const moe_config* cfg, int64_t N, int32_t call, size_t* bytes);

/*
 * moe_route - the router ([K2-AFF] gate-forward; [V32-AFF] gate-forward).
 *   logits = hidden . w_router^T in fp32 (hidden widened exactly), no bias;
 *   score = sigmoid(logits), or with MOE_SCORE_SOFTMAX the softmax of the
 *   token's logits over all E experts ([V32-AFF]);
 *   choice = score + bias (selection only), or score when bias is NULL;
 *   group g = experts [g*E/G, (g+1)*E/G); group score = sum of its two largest
 *   choice values, or its largest one when bias is NULL ([V32-AFF]); the TG
 *   best groups are kept and the others dropped (their experts can never be
 *   chosen); the k largest choice values among the kept experts are chosen
 *   (ties to the lower index); weight = score of the chosen expert, divided by
 *   (sum of the k scores + 1e-20) when norm_topk_prob and k > 1, times
 *   route_scale.  ([V32-AFF] renormalises sigmoid scores only: set
 *   norm_topk_prob = 0 with softmax for that gate.)
 * hidden [N, d] dtype; w_router [E, d] fp32; bias [E] fp32 or NULL.
 * Out: topk_idx [N, k] int32, each row's experts in ascending id;
 *      topk_weight [N, k] fp32, in the same slot order.
 * N = 0 is a valid no-op.
 */
moe_status moe_route(const moe_config* cfg, int64_t N, const void* hidden, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_weight, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * moe_permute - dispatch by expert ([K3-ADD] moe_infer: the per-expert token
 * counts, the argsort of the flattened choices, the gather of token rows).
 *   tokens_per_expert[e] = number of slots (n, j) with topk_idx[n][j] == e;
 *   expert_offsets = exclusive prefix sum (expert_offsets[E] = N*k);
 *   perm[p] = flat slot n*k + j at sorted position p: slots grouped by expert
 *   and, inside an expert, in increasing slot order (a stable sort);
 *   inv_perm[n*k + j] = p;  x_sorted[p] = x_in[perm[p] / k].
 * topk_idx [N, k] int32: each row must hold k distinct experts in [0, E) (as
 *   moe_route writes them); other values give unspecified outputs but no
 *   access outside the arguments.
 * x_in [N, d_in] dtype: the experts' input (the latent input when d_latent > 0).
 * Out: tokens_per_expert [E], expert_offsets [E + 1], perm [N*k], inv_perm
 *   [N*k] int32; x_sorted [N*k, d_in] dtype (optional: NULL skips the gather).
 */
moe_status moe_permute(const moe_config* cfg, int64_t N, const int32_t* topk_idx,
                       const void* x_in, int32_t* tokens_per_expert, int32_t* expert_offsets,
                       int32_t* perm, int32_t* inv_perm, void* x_sorted, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_permute_static - moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results without a workspace.  Its
 * scratch (the dispatch masks and per-chunk bases, ceil(N/64) * E * 12 bytes
 * plus alignment) lives in a static device array of MOE_STATIC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends.  Larger
 * problems return MOE_ERR_UNSUPPORTED before anything is enqueued.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, no ordering between them) race
 * and give unspecified results; calls ordered on one stream are safe.
 */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)
moe_status moe_permute_static(const moe_config* cfg, int64_t N, const int32_t* topk_idx,
                              const void* x_in, int32_t* tokens_per_expert,
                              int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                              void* x_sorted, void* stream);

/*
 * moe_expert_gate_up - first half of every routed expert ([K3-GATE] expert
 * and situ excerpts), on the expert-sorted rows.  For each expert e and row p
 * in [expert_offsets[e], expert_offsets[e+1]):
 *   g = w1[e] . x_sorted[p], u = w3[e] . x_sorted[p] (fp32 accumulation),
 *   SiLU: h = silu(g) * u;
 *   SiTU: h = beta*tanh(g/beta)*sigmoid(g) * (lb*tanh(u/lb) if lb > 0 else u),
 *   evaluated in fp32 and rounded once to dtype.
 * x_sorted [N*k, d_in] dtype; expert_offsets [E + 1] int32 as moe_permute
 * writes it (non-decreasing, from 0 to N*k); w1, w3 [E, d_ff, d_in] dtype.
 * Out: h_sorted [N*k, d_ff] dtype.
 */
moe_status moe_expert_gate_up(const moe_config* cfg, int64_t N, const void* x_sorted,
                              const int32_t* expert_offsets, const void* w1, const void* w3,
                              void* h_sorted, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * moe_expert_gate_up_gather - moe_expert_gate_up with the row gather of
 * moe_permute folded into its activation loads ([K3-ADD] moe_infer gathers
 * x[argsort // k] before the expert loop): row p of expert e is
 * x_in[perm[p] / k], so no sorted copy of the input is written.  This is the
 * form moe_block_forward runs.
 * x_in [N, d_in] dtype; perm [N*k] int32 as moe_permute writes it (every value
 * in [0, N*k); other values are clamped to a valid row); expert_offsets, w1,
 * w3 and the output h_sorted [N*k, d_ff] as for moe_expert_gate_up.  Needs the
 * workspace of MOE_CALL_GATE_UP.
 */
moe_status moe_expert_gate_up_gather(const moe_config* cfg, int64_t N, const void* x_in,
                                     const int32_t* perm, const int32_t* expert_offsets,
                                     const void* w1, const void* w3, void* h_sorted,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_down - second half of every routed expert ([K3-GATE] expert:
 * w2 applied to the activation).  out_sorted[p] = w2[e] . h_sorted[p] for the
 * rows p of expert e, fp32 accumulation, rounded once to dtype.
 * h_sorted [N*k, d_ff] dtype; expert_offsets as above; w2 [E, d_in, d_ff].
 * Out: out_sorted [N*k, d_in] dtype.
 */
moe_status moe_expert_down(const moe_config* cfg, int64_t N, const void* h_sorted,
                           const int32_t* expert_offsets, const void* w2, void* out_sorted,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_down_scatter - moe_expert_down with the un-permute of [K3-ADD]
 * moe_infer (the outputs put back at their tokens' places before the weighted
 * sum) folded into its stores: the output row of sorted row p goes to slot
 * perm[p] = n*k + j, so out_slots holds each token's k expert rows
 * contiguously, in slot order.  The form moe_block_forward runs.
 * h_sorted, expert_offsets, w2 as for moe_expert_down; perm [N*k] int32 as
 * moe_permute writes it (a permutation of 0 .. N*k - 1: every slot is written
 * once).  Out: out_slots [N*k, d_in] dtype.  Workspace of MOE_CALL_DOWN.
 */
moe_status moe_expert_down_scatter(const moe_config* cfg, int64_t N, const void* h_sorted,
                                   const int32_t* expert_offsets, const int32_t* perm,
                                   const void* w2, void* out_slots, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * moe_combine - back to token order and weighted sum ([K3-ADD] moe_infer: the
 * un-permute, the product with the routing weights in their fp32 precision,
 * the sum over the k slots, the cast back).
 *   y[n] = residual[n] + sum_{j = 0..k-1} topk_weight[n][j] * row(n, j),
 *   row(n, j) = out_sorted[inv_perm[n*k + j]], or, with inv_perm NULL (rows
 *   already in slot order, as moe_expert_down_scatter writes them),
 *   out_sorted[n*k + j]; accumulated in fp32 in that fixed j order, rounded
 *   once to dtype.
 * out_sorted [N*k, d_in] dtype; inv_perm [N*k] int32 or NULL; topk_weight
 * [N, k] fp32; residual [N, d_in] dtype or NULL (zero).  Out: y [N, d_in]
 * dtype.  Needs no workspace.
 */
moe_status moe_combine(const moe_config* cfg, int64_t N, const void* out_sorted,
                       const int32_t* inv_perm, const float* topk_weight, const void* residual,
                       void* y, void* stream);

/*
 * moe_shared_expert - the shared expert ([K3-ADD] forward: the shared experts
 * run on the block's full-width input and their output is added to the routed
 * sum): out = sh_w2 . act(sh_w1 . hidden, sh_w3 . hidden), the same gated MLP
 * and activation as the routed experts (fp32 accumulation, activation in
 * fp32, its result rounded once to dtype), the output kept in fp32 (as
 * moe_block_forward adds it before its final rounding).
 * Needs cfg->d_ff_shared > 0.  hidden [N, d] dtype; sh_w1, sh_w3
 * [d_ff_shared, d] dtype; sh_w2 [d, d_ff_shared] dtype.  Out: out [N, d] fp32.
 * Workspace: moe_workspace_size(MOE_CALL_SHARED).
 */
moe_status moe_shared_expert(const moe_config* cfg, int64_t N, const void* hidden,
                             const void* sh_w1, const void* sh_w3, const void* sh_w2, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_latent_project - a latent projection of the K3 latent block ([K3-ADD]
 * forward): up = 0, the down projection x_lat = hidden . w_down^T (x [N, d],
 * w [d_latent, d], out [N, d_latent]); up = 1, the up projection
 * y = y_lat . w_up^T (+ residual) (x [N, d_latent], w [d, d_latent],
 * out [N, d]).  fp32 accumulation; residual [N, n_out] fp32 or NULL, added in
 * fp32; the sum rounded once to dtype.  Needs cfg->d_latent > 0.  No workspace.
 */
moe_status moe_latent_project(const moe_config* cfg, int64_t N, int32_t up, const void* x,
                              const void* w, const float* residual, void* out, void* stream);

/*
 * moe_block_forward - the whole block ([K3-ADD] forward): route on the
 * full-width hidden state; with d_latent > 0 project it down
 * (x_in = hidden . w_down^T, rounded to dtype), else x_in = hidden; permute,
 * gate/up, down and combine as above; with d_latent > 0 RMS-normalise each
 * combined row in fp32 (y / sqrt(mean(y^2) + norm_eps) * gamma, when
 * latent_norm), round it to dtype (the up projection's operand) and project
 * it up with w_up; with d_ff_shared > 0 add the shared expert (the same gated
 * MLP and activation, on the full-width hidden; its output is kept in fp32)
 * to the combined or up-projected sum in fp32, before the single final
 * rounding of y.  Intermediate roundings to dtype: the latent input x_in, each
 * expert's h and output rows, the shared expert's h, and the normalised
 * latent row.
 * The latent down projection and the shared expert need only `hidden`: they
 * run on a side stream of the current device (default priority, created on
 * the first block call and kept until the process ends), forked from `stream`
 * at the start of the call and joined back into it before the first step that
 * uses their results, so the call's work is still complete when `stream`
 * passes it.  Block calls of one process serialise on that side stream.
 * hidden [N, d] dtype.  Out: y [N, d] dtype.  Optional outputs (NULL skips):
 * topk_idx_out [N, k] int32, topk_weight_out [N, k] fp32,
 * tokens_per_expert_out [E] int32.
 */
moe_status moe_block_forward(const moe_config* cfg, int64_t N, const moe_weights* w,
                             const void* hidden, void* y, int32_t* topk_idx_out,
                             float* topk_weight_out, int32_t* tokens_per_expert_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tracing (no counterpart on the pages).  Stage boundaries of
 * moe_block_forward at which, when set, an event is recorded on the call's
 * stream, so that each stage's device time can be read with
 * hipEventElapsedTime between consecutive events.
 */
typedef enum {
  MOE_STAGE_BEGIN = 0,      /* before the router */
  MOE_STAGE_ROUTED = 1,     /* after the router (weight split, logits, selection) */
  MOE_STAGE_LATENT = 2,     /* after the latent down projection (empty on `stream`
                               when it runs on the side stream) */
  MOE_STAGE_DISPATCHED = 3, /* after mask, scan and scatter */
  MOE_STAGE_SHARED = 4,     /* after the wait for the latent input (the shared
                               expert itself runs on the side stream) */
  MOE_STAGE_GATE_UP = 5,    /* after the routed gate/up grouped GEMM */
  MOE_STAGE_DOWN = 6,       /* after the routed down grouped GEMM */
  MOE_STAGE_END = 7,        /* after combine (and norm + up projection) */
  MOE_STAGE_COUNT = 8
} moe_stage;

/* Sets, for the calling thread, the MOE_STAGE_COUNT hipEvent_t handles that
 * later moe_block_forward calls record (events = NULL clears them).  The
 * events are owned by the caller and must stay valid while set. */
moe_status moe_set_stage_events(void* const* events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H */
