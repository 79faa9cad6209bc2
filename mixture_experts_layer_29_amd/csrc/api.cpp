// api.cpp - the C ABI of libmoe (include/moe.h): host-side validation, the
// workspace plan, and the order of kernel launches for each call.
//
// Every call validates on the host first and enqueues nothing on an error.
// Launches go to the caller's stream in order; nothing here waits for the GPU
// or allocates device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "common.h"

// Scratch of moe_permute_static: one array per GPU, alive until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept per device (static_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_stage_events[MOE_STAGE_COUNT];
thread_local bool g_stage_events_set = false;

hipError_t mark(int stage, hipStream_t s) {
  if (!g_stage_events_set) return hipSuccess;
  return hipEventRecord(g_stage_events[stage], s);
}

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define OPTIONAL_PTR(p)                                                                    \
  do {                                                                                     \
    if ((p) != nullptr && !aligned16(p))                                                   \
      return fail(MOE_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p);           \
  } while (0)
#define REQUIRE_PTR(p)                                                                     \
  do {                                                                                     \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);        \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

#define CHECK_HIP(expr)                                                                    \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return fail(MOE_ERR_HIP, "%s: %s failed: %s", fn, #expr, hipGetErrorString(e_));     \
  } while (0)

int64_t d_in_of(const moe_config* c) { return c->d_latent > 0 ? c->d_latent : c->d; }
size_t esize(const moe_config* c) { return c->dtype == MOE_DTYPE_BF16 ? 2 : 4; }
bool is_bf16(const moe_config* c) { return c->dtype == MOE_DTYPE_BF16; }

constexpr int64_t kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int64_t kMaxLatent = 16384;  // row width of the fused combine + RMS norm

moe_status validate(const moe_config* c, const char* fn) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "%s: cfg is NULL", fn);
  if (c->training) return fail(MOE_ERR_UNSUPPORTED, "%s: training mode is not supported", fn);
  if (c->score_func != MOE_SCORE_SIGMOID && c->score_func != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "%s: scoring function %d is not supported", fn,
                c->score_func);
  if (c->topk_method != MOE_TOPK_NOAUX_TC)
    return fail(MOE_ERR_UNSUPPORTED, "%s: top-k method %d is not supported (noaux_tc only)", fn,
                c->topk_method);
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: dtype %d is not supported", fn, c->dtype);
  if (c->act != MOE_ACT_SILU && c->act != MOE_ACT_SITU)
    return fail(MOE_ERR_UNSUPPORTED, "%s: activation %d is not supported", fn, c->act);
  if (c->d <= 0 || c->d % 8) return fail(MOE_ERR_INVALID_ARG, "%s: d=%lld must be a positive multiple of 8", fn, (long long)c->d);
  if (c->d_ff <= 0 || c->d_ff % 8) return fail(MOE_ERR_INVALID_ARG, "%s: d_ff=%lld must be a positive multiple of 8", fn, (long long)c->d_ff);
  if (c->d_latent < 0 || c->d_latent % 8) return fail(MOE_ERR_INVALID_ARG, "%s: d_latent=%lld must be 0 or a positive multiple of 8", fn, (long long)c->d_latent);
  if (c->d_latent > kMaxLatent) return fail(MOE_ERR_UNSUPPORTED, "%s: d_latent=%lld exceeds %lld", fn, (long long)c->d_latent, (long long)kMaxLatent);
  if (c->d_ff_shared < 0 || c->d_ff_shared % 8) return fail(MOE_ERR_INVALID_ARG, "%s: d_ff_shared=%lld must be 0 or a positive multiple of 8", fn, (long long)c->d_ff_shared);
  if (c->n_experts < 2) return fail(MOE_ERR_INVALID_ARG, "%s: n_experts=%lld must be >= 2", fn, (long long)c->n_experts);
  if (c->n_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "%s: n_experts=%lld exceeds %lld", fn, (long long)c->n_experts, (long long)kMaxExperts);
  if (c->n_group < 1 || c->n_experts % c->n_group)
    return fail(MOE_ERR_INVALID_ARG, "%s: n_group=%d must divide n_experts=%lld", fn, c->n_group, (long long)c->n_experts);
  const int64_t per = c->n_experts / c->n_group;
  if (per < 2) return fail(MOE_ERR_INVALID_ARG, "%s: groups need at least 2 experts (E/G=%lld)", fn, (long long)per);
  if (c->topk_group < 1 || c->topk_group > c->n_group)
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_group=%d must be in [1, n_group=%d]", fn, c->topk_group, c->n_group);
  if (c->top_k < 1 || c->top_k > (int64_t)c->topk_group * per)
    return fail(MOE_ERR_INVALID_ARG, "%s: top_k=%d must be in [1, topk_group*E/G=%lld]", fn, c->top_k, (long long)(c->topk_group * per));
  if (c->top_k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "%s: top_k=%d exceeds %d", fn, c->top_k, kMaxTopK);
  if (!std::isfinite(c->route_scale)) return fail(MOE_ERR_INVALID_ARG, "%s: route_scale is not finite", fn);
  if (c->act == MOE_ACT_SITU) {
    if (!std::isfinite(c->situ_beta) || c->situ_beta < 0.0f)
      return fail(MOE_ERR_INVALID_ARG, "%s: situ_beta must be finite and >= 0", fn);
    if (!std::isfinite(c->situ_linear_beta)) return fail(MOE_ERR_INVALID_ARG, "%s: situ_linear_beta is not finite", fn);
  }
  if (c->d_latent > 0 && (!std::isfinite(c->norm_eps) || c->norm_eps < 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "%s: norm_eps must be finite and >= 0", fn);
  return MOE_OK;
}

moe_status validate_n(const moe_config* c, int64_t N, const char* fn) {
  if (N < 0) return fail(MOE_ERR_INVALID_ARG, "%s: N=%lld is negative", fn, (long long)N);
  if (N * (int64_t)c->top_k > INT32_MAX || N > INT32_MAX / 64)
    return fail(MOE_ERR_INVALID_ARG, "%s: N=%lld is too large (N*k must fit int32)", fn, (long long)N);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Workspace plan.
struct Plan {
  size_t bytes = 0;
  size_t w_split = 0, logits = 0, idx = 0, wts = 0, bits = 0, base = 0, counts = 0, offsets = 0;
  size_t mt_off = 0, tile_seg = 0, perm = 0, inv_perm = 0, x_lat = 0, h = 0, out = 0;
  size_t sh_h = 0, sh_out = 0, y_lat = 0;
  int rb = 4;              // row blocks of 32 per grouped-GEMM tile (bf16)
  int waves_gate_up = 4;   // waves per grouped-GEMM work-group (bf16), gate/up
  int waves_down = 4;      //   and down products
  int rows_per_tile = 128; // rows per grouped-GEMM m-tile
  int64_t tile_cap = 0;
  int64_t dp = 0;          // router width padded to 64
  int64_t n_chunks = 0;
  int router_rb = 1;       // router product (bf16): tile height in row blocks,
  int64_t router_splits = 1, router_split_blocks = 0;  // and its K ranges
};

struct Carver {
  size_t off = 0;
  size_t take(size_t b) {
    const size_t at = off;
    off += (b + 255) & ~size_t(255);
    return at;
  }
};

// Height (in 32-row blocks) of the routed grouped-GEMM tiles.  A tile streams
// its weight columns once for all of its rows, so the tile should hold a whole
// expert segment where it can (each extra m-tile of an expert re-streams the
// expert's weights); tiles shorter than their maximum issue only the MFMAs of
// their rows.  Taller tiles need more accumulator registers (one wave per SIMD
// and a larger activation stage in LDS), so short segments (decode) use short
// tiles.  Widths that are not multiples of 64 take the clamped K-tail path,
// which runs 1-block tiles.
int choose_rb(const moe_config* c, int64_t N) {
  const int64_t d_in = c->d_latent > 0 ? c->d_latent : c->d;
  if (d_in % 64 || c->d_ff % 64) return 1;
  const double avg = (double)N * c->top_k / (double)c->n_experts;
  if (avg >= 64.0) return 8;
  if (avg >= 24.0) return 4;
  if (avg >= 12.0) return 2;
  return 1;
}

constexpr int64_t kDenseMinRows = 512;

// Dense products (shared expert, latent projections) reuse every weight tile
// across all m-tiles, so they are bound by the operand traffic into each CU
// rather than by HBM: the tallest tile that still gives every CU a tile has
// the most flops per byte loaded.
int dense_rb(int64_t rows, int64_t K, int64_t n_cols, int epi) {
  if (K % 64) return 1;
  const int64_t cols_per_tile = epi == moe::EPI_GATE_UP ? 128 : 256;
  const int64_t n_tiles = (n_cols + cols_per_tile - 1) / cols_per_tile;
  for (int rb : {8, 4, 2}) {
    if ((rows + rb * 32 - 1) / (rb * 32) * n_tiles >= 240) return rb;
  }
  return 1;
}

// Router product (bf16 path): [N, 3 dp] x [E, 3 dp]^T, tiles of rb*32 rows by
// 256 experts.  There are few such tiles (N/256 at prefill, 8 at decode) and
// each would stream all of W_r, so K is cut into ranges (at least 8 blocks of
// 64 each) until the tiles and ranges fill the GPU once; the selection kernel
// adds the partial products in range order.
void plan_router(const moe_config* c, int64_t N, Plan& p) {
  const int64_t nkb = 3 * p.dp / 64;
  p.router_rb = N >= 4096 ? 8 : (N >= 1024 ? 4 : (N >= 256 ? 2 : 1));
  p.router_splits = 1;
  p.router_split_blocks = nkb;
  if (!is_bf16(c)) return;
  const int64_t mt = (N + p.router_rb * 32 - 1) / (p.router_rb * 32);
  const int64_t tiles = mt * ((c->n_experts + 255) / 256);
  if (tiles <= 0 || tiles >= 256) return;
  int64_t want = (256 + tiles - 1) / tiles;
  const int64_t most = nkb / 8 > 1 ? nkb / 8 : 1;
  if (want > most) want = most;
  p.router_split_blocks = (nkb + want - 1) / want;
  p.router_splits = (nkb + p.router_split_blocks - 1) / p.router_split_blocks;
}

Plan make_plan(const moe_config* c, int64_t N, int call) {
  Plan p;
  const int64_t E = c->n_experts, k = c->top_k, S = N * k;
  const size_t es = esize(c);
  p.rb = choose_rb(c, N);
  // two waves per SIMD pay off when the tiles are tall: measured on MI355X,
  // gate/up gains with 256-row tiles (from ~130 rows per expert on), down
  // only from ~170 rows per expert
  const double avg_rows = (double)N * c->top_k / (double)c->n_experts;
  p.waves_gate_up = p.rb == 8 ? 8 : 4;
  p.waves_down = (p.rb == 8 && avg_rows >= 160.0) ? 8 : 4;
  p.rows_per_tile = is_bf16(c) ? p.rb * 32 : moe::gemm_f32_rows_per_tile();
  p.tile_cap = S / p.rows_per_tile + (E < S ? E : S) + 1;
  p.dp = (c->d + 63) / 64 * 64;
  p.n_chunks = (N + 63) / 64;
  plan_router(c, N, p);
  Carver cv;
  const bool block = call == MOE_CALL_BLOCK;
  if (call == MOE_CALL_ROUTE || block) {
    if (is_bf16(c)) p.w_split = cv.take((size_t)E * 3 * p.dp * 2);
    p.logits = cv.take((size_t)p.router_splits * N * E * 4);
  }
  if (call == MOE_CALL_PERMUTE || block) {
    p.bits = cv.take((size_t)p.n_chunks * E * 8);
    p.base = cv.take((size_t)p.n_chunks * E * 4);
  }
  if (call == MOE_CALL_GATE_UP || call == MOE_CALL_DOWN || block) {
    p.mt_off = cv.take((size_t)(E + 1 + 9) * 4);  // m-tile prefix, then the XCD split
    p.tile_seg = cv.take((size_t)p.tile_cap * 4);
  }
  if (call == MOE_CALL_SHARED) p.sh_h = cv.take((size_t)N * c->d_ff_shared * es);
  if (block) {
    const int64_t d_in = d_in_of(c);
    p.idx = cv.take((size_t)S * 4);
    p.wts = cv.take((size_t)S * 4);
    p.counts = cv.take((size_t)E * 4);
    p.offsets = cv.take((size_t)(E + 1) * 4);
    p.perm = cv.take((size_t)S * 4);
    p.inv_perm = cv.take((size_t)S * 4);
    p.h = cv.take((size_t)S * c->d_ff * es);
    p.out = cv.take((size_t)S * d_in * es);
    if (c->d_latent > 0) {
      p.x_lat = cv.take((size_t)N * c->d_latent * es);
      p.y_lat = cv.take((size_t)N * c->d_latent * es);
    }
    if (c->d_ff_shared > 0) {
      p.sh_h = cv.take((size_t)N * c->d_ff_shared * es);
      p.sh_out = cv.take((size_t)N * c->d * 4);  // fp32: added before the final rounding
    }
  }
  p.bytes = cv.off;
  return p;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(const Plan& p, void* ws, size_t ws_bytes, const char* fn) {
  if (p.bytes == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, p.bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace is not 256-byte aligned", fn);
  if (ws_bytes < p.bytes)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, p.bytes);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Launch sequences (arguments already validated).

moe::GemmArgs gemm_args() {
  moe::GemmArgs a;
  std::memset(&a, 0, sizeof a);
  a.a_div = 1;
  a.beta = 1.0f;
  return a;
}

hipError_t dense_gemm(const moe_config* c, const void* A, int64_t rows, int64_t K, const void* B0,
                      const void* B1, int64_t n_cols, void* C, int epi, const void* residual,
                      hipStream_t s) {
  moe::GemmArgs a = gemm_args();
  a.A = A;
  a.lda = K;
  a.a_rows = rows;
  a.B0 = B0;
  a.B1 = B1;
  a.K = K;
  a.n_cols = n_cols;
  a.dense_rows = rows;
  a.C = C;
  a.ldc = n_cols;
  a.c_rows = rows;
  a.residual = residual;
  a.ld_res = n_cols;
  a.act = c->act;
  a.beta = c->situ_beta > 0.0f ? c->situ_beta : 1.0f;
  a.lbeta = c->situ_linear_beta;
  if (is_bf16(c)) {
    // from 512 rows on, the MFMA-bound tile kernel; short products (decode)
    // are bound by their weights and stream them with the grouped kernel's
    // tiles, the tallest that still give every CU a tile
    if (rows >= kDenseMinRows && moe::gemm_dense_supported(a, epi))
      return moe::launch_gemm_dense(a, epi, s);
    const int rb = dense_rb(rows, K, n_cols, epi);
    return moe::launch_gemm_bf16(a, epi, moe::A_DIRECT, rb, rb >= 4 ? 8 : 4, 0, s);
  }
  return moe::launch_gemm_f32(a, epi, moe::A_DIRECT, 0, s);
}

moe::GemmArgs grouped_args(const moe_config* c, const Plan& p, int64_t N, const void* A,
                           const int32_t* a_map, int64_t a_rows, int64_t K,
                           const int32_t* seg_off, const void* B0, const void* B1,
                           int64_t n_cols, void* C, void* ws, const int32_t* c_map) {
  moe::GemmArgs a = gemm_args();
  a.A = A;
  a.lda = K;
  a.a_map = a_map;
  a.a_div = c->top_k;
  a.a_rows = a_rows;
  a.B0 = B0;
  a.B1 = B1;
  a.b_seg_stride = n_cols * K;
  // an expert's weights are read by its own tiles only: non-temporal loads
  // for experts whose rows fit one m-tile (cached for the others, whose
  // m-tiles share them in L2)
  a.b_stream = 2;
  a.K = K;
  a.n_cols = n_cols;
  a.seg_off = seg_off;
  a.mt_off = at<int32_t>(ws, p.mt_off);
  a.n_seg = c->n_experts;
  a.tile_seg = at<int32_t>(ws, p.tile_seg);
  a.tile_cap = p.tile_cap;
  a.C = C;
  a.c_map = c_map;
  a.ldc = n_cols;
  a.c_rows = N * c->top_k;
  a.act = c->act;
  a.beta = c->situ_beta > 0.0f ? c->situ_beta : 1.0f;
  a.lbeta = c->situ_linear_beta;
  return a;
}

hipError_t grouped_gemm(const moe_config* c, const Plan& p, int64_t N, const void* A, int amode,
                        const int32_t* a_map, int64_t a_rows, int64_t K, const int32_t* seg_off,
                        const void* B0, const void* B1, int64_t n_cols, void* C, int epi,
                        void* ws, hipStream_t s, const int32_t* c_map = nullptr) {
  const moe::GemmArgs a =
      grouped_args(c, p, N, A, a_map, a_rows, K, seg_off, B0, B1, n_cols, C, ws, c_map);
  if (is_bf16(c)) {
    const int waves = epi == moe::EPI_GATE_UP ? p.waves_gate_up : p.waves_down;
    return moe::launch_gemm_bf16(a, epi, amode, p.rb, waves, p.tile_cap, s);
  }
  return moe::launch_gemm_f32(a, epi, amode, p.tile_cap, s);
}

// Shared expert: h = act(x . sh_w1^T, x . sh_w3^T) rounded to the block dtype,
// then out = h . sh_w2^T kept in fp32.
hipError_t shared_expert(const moe_config* c, int64_t N, const void* x, const void* w1,
                         const void* w3, const void* w2, void* h, float* out, hipStream_t s) {
  hipError_t e = dense_gemm(c, x, N, c->d, w1, w3, c->d_ff_shared, h, moe::EPI_GATE_UP, nullptr, s);
  if (e != hipSuccess) return e;
  return dense_gemm(c, h, N, c->d_ff_shared, w2, nullptr, c->d, out,
                    is_bf16(c) ? moe::EPI_STORE_F32 : moe::EPI_STORE, nullptr, s);
}

moe_status run_route(const moe_config* c, int64_t N, const void* hidden, const float* w_router,
                     const float* bias, int32_t* idx, float* wts, void* ws, const Plan& p,
                     hipStream_t s, const char* fn) {
  const int64_t E = c->n_experts;
  float* logits = at<float>(ws, p.logits);
  if (is_bf16(c)) {
    moe::bf16_t* split = at<moe::bf16_t>(ws, p.w_split);
    CHECK_HIP(moe::launch_router_split(w_router, E, c->d, p.dp, split, s));
    moe::GemmArgs a = gemm_args();
    a.A = hidden;
    a.lda = c->d;
    a.a_rows = N;
    a.a_period = p.dp;
    a.a_valid = c->d;
    a.B0 = split;
    a.K = 3 * p.dp;
    a.n_cols = E;
    a.dense_rows = N;
    a.C = logits;
    a.ldc = E;
    a.c_rows = N;
    a.k_splits = p.router_splits;
    a.k_split_blocks = p.router_split_blocks;
    a.c_split_stride = N * E;
    CHECK_HIP(moe::launch_gemm_bf16(a, moe::EPI_STORE_F32, moe::A_REPEAT, p.router_rb, 4, 0, s));
  } else {
    CHECK_HIP(dense_gemm(c, hidden, N, c->d, w_router, nullptr, E, logits, moe::EPI_STORE, nullptr, s));
  }
  const int parts = is_bf16(c) ? (int)p.router_splits : 1;
  CHECK_HIP(moe::launch_route_select(logits, parts, N * E, bias,
                                     c->score_func == MOE_SCORE_SOFTMAX ? 1 : 0, N, E,
                                     c->n_group, c->topk_group, c->top_k,
                                     c->norm_topk_prob ? 1 : 0, c->route_scale, idx, wts, s));
  return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void** out, const char* fn) {
  int dev = -1;
  CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d supported", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(MOE_ERR_HIP, "%s: no device address for the static scratch", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The block runs the products that need only its input -- the latent down
// projection, then the shared expert -- on a side stream of the device, beside
// the router and the dispatch, whose kernels are few and short: the dense
// products fill the CUs they leave idle.  One side stream (default priority)
// and its events per device (fork; latent input ready; shared output ready),
// created on first use and kept until the process ends.  A block call holds
// g_side_mutex from its fork to its last wait, so concurrent calls do not
// interleave their records of the events.
struct Side {
  hipStream_t stream;
  hipEvent_t fork, latent, join;
};
std::mutex g_side_mutex;
Side g_side[kMaxDevices] = {};

// The current device's side stream; the caller holds g_side_mutex.
moe_status side_stream(Side* out, const char* fn) {
  int dev = -1;
  CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d supported", fn, dev,
                kMaxDevices);
  Side& sd = g_side[dev];
  if (!sd.stream) {
    Side n{};
    CHECK_HIP(hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking));
    CHECK_HIP(hipEventCreateWithFlags(&n.fork, hipEventDisableTiming));
    CHECK_HIP(hipEventCreateWithFlags(&n.latent, hipEventDisableTiming));
    CHECK_HIP(hipEventCreateWithFlags(&n.join, hipEventDisableTiming));
    sd = n;
  }
  *out = sd;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_validate_config(const moe_config* cfg) {
  moe_status st = validate(cfg, "moe_validate_config");
  return st == MOE_OK ? ok() : st;
}

moe_status moe_workspace_size(const moe_config* cfg, int64_t N, int32_t call, size_t* bytes) {
  const char* fn = "moe_workspace_size";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  if (call < MOE_CALL_ROUTE || call > MOE_CALL_LATENT) return fail(MOE_ERR_INVALID_ARG, "%s: unknown call %d", fn, call);
  if (call == MOE_CALL_SHARED && cfg->d_ff_shared <= 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: the config has no shared expert", fn);
  *bytes = make_plan(cfg, N, call).bytes;
  return ok();
}

moe_status moe_route(const moe_config* cfg, int64_t N, const void* hidden, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_weight, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const char* fn = "moe_route";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE_PTR(hidden);
  REQUIRE_PTR(w_router);
  OPTIONAL_PTR(bias);  // a router without a bias
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_weight);
  const Plan p = make_plan(cfg, N, MOE_CALL_ROUTE);
  if ((st = check_ws(p, workspace, workspace_bytes, fn)) != MOE_OK) return st;
  st = run_route(cfg, N, hidden, w_router, bias, topk_idx, topk_weight, workspace, p,
                 static_cast<hipStream_t>(stream), fn);
  return st == MOE_OK ? ok() : st;
}

static moe_status permute_args(const moe_config* cfg, int64_t N, const int32_t* topk_idx,
                               const void* x_in, const int32_t* tokens_per_expert,
                               const int32_t* expert_offsets, const int32_t* perm,
                               const int32_t* inv_perm, const void* x_sorted, const char* fn) {
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  REQUIRE_PTR(tokens_per_expert);
  REQUIRE_PTR(expert_offsets);
  if (N > 0) {
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(perm);
    REQUIRE_PTR(inv_perm);
    if (x_sorted) {
      REQUIRE_PTR(x_in);
      REQUIRE_PTR(x_sorted);
    }
  }
  return MOE_OK;
}

// Dispatch launches with the masks and chunk bases at `scratch` (laid out by
// the plan of MOE_CALL_PERMUTE).  Every entry of both is written before it is
// read, so the scratch needs no clearing.
static moe_status run_permute(const moe_config* cfg, int64_t N, const int32_t* topk_idx,
                              const void* x_in, int32_t* tokens_per_expert,
                              int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                              void* x_sorted, void* scratch, const Plan& p, hipStream_t s,
                              const char* fn) {
  const int64_t E = cfg->n_experts;
  const int k = cfg->top_k;
  uint64_t* bits = at<uint64_t>(scratch, p.bits);
  int32_t* base = at<int32_t>(scratch, p.base);
  CHECK_HIP(moe::launch_dispatch_mask(topk_idx, N, k, E, bits, s));
  CHECK_HIP(moe::launch_dispatch_scan(bits, p.n_chunks, E, tokens_per_expert, expert_offsets, base,
                                      0, nullptr, nullptr, 0, s));
  CHECK_HIP(moe::launch_dispatch_scatter(topk_idx, N, k, E, bits, base, perm, inv_perm, s));
  if (x_sorted && N > 0)
    CHECK_HIP(moe::launch_gather_rows(x_in, N, d_in_of(cfg), (int)esize(cfg), perm, k, N * k,
                                      x_sorted, s));
  return ok();
}

moe_status moe_permute(const moe_config* cfg, int64_t N, const int32_t* topk_idx, const void* x_in,
                       int32_t* tokens_per_expert, int32_t* expert_offsets, int32_t* perm,
                       int32_t* inv_perm, void* x_sorted, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const char* fn = "moe_permute";
  moe_status st = permute_args(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm,
                               inv_perm, x_sorted, fn);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(cfg, N, MOE_CALL_PERMUTE);
  if ((st = check_ws(p, workspace, workspace_bytes, fn)) != MOE_OK) return st;
  return run_permute(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm, inv_perm,
                     x_sorted, workspace, p, static_cast<hipStream_t>(stream), fn);
}

moe_status moe_permute_static(const moe_config* cfg, int64_t N, const int32_t* topk_idx,
                              const void* x_in, int32_t* tokens_per_expert,
                              int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm,
                              void* x_sorted, void* stream) {
  const char* fn = "moe_permute_static";
  moe_status st = permute_args(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm,
                               inv_perm, x_sorted, fn);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(cfg, N, MOE_CALL_PERMUTE);
  if (p.bytes > MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: N=%lld tokens over E=%lld experts need %zu bytes of dispatch scratch; the "
                "static scratch holds %zu (ceil(N/64) * E * 12 bytes must fit)", fn, (long long)N,
                (long long)cfg->n_experts, p.bytes, (size_t)MOE_STATIC_SCRATCH_BYTES);
  void* ptr = nullptr;  // this device's copy of the static scratch
  if ((st = static_scratch(&ptr, fn)) != MOE_OK) return st;
  return run_permute(cfg, N, topk_idx, x_in, tokens_per_expert, expert_offsets, perm, inv_perm,
                     x_sorted, ptr, p, static_cast<hipStream_t>(stream), fn);
}

static moe_status expert_call(const moe_config* cfg, int64_t N, const void* A,
                              const int32_t* perm, const int32_t* expert_offsets, const void* B0,
                              const void* B1, void* C, void* workspace, size_t workspace_bytes,
                              void* stream, bool gate_up, const char* fn) {
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE_PTR(A);
  if (perm) REQUIRE_PTR(perm);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(B0);
  if (gate_up) REQUIRE_PTR(B1);
  REQUIRE_PTR(C);
  const Plan p = make_plan(cfg, N, gate_up ? MOE_CALL_GATE_UP : MOE_CALL_DOWN);
  if ((st = check_ws(p, workspace, workspace_bytes, fn)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CHECK_HIP(moe::launch_tiles_from_offsets(expert_offsets, cfg->n_experts, p.rows_per_tile,
                                           at<int32_t>(workspace, p.mt_off),
                                           at<int32_t>(workspace, p.tile_seg), p.tile_cap, s));
  const int64_t d_in = d_in_of(cfg);
  if (gate_up && perm) {
    CHECK_HIP(grouped_gemm(cfg, p, N, A, moe::A_GATHER, perm, N, d_in, expert_offsets, B0, B1,
                           cfg->d_ff, C, moe::EPI_GATE_UP, workspace, s));
  } else if (gate_up) {
    CHECK_HIP(grouped_gemm(cfg, p, N, A, moe::A_DIRECT, nullptr, N * cfg->top_k, d_in,
                           expert_offsets, B0, B1, cfg->d_ff, C, moe::EPI_GATE_UP, workspace, s));
  } else {
    // down: with perm, row p is written to its slot perm[p]
    CHECK_HIP(grouped_gemm(cfg, p, N, A, moe::A_DIRECT, nullptr, N * cfg->top_k, cfg->d_ff,
                           expert_offsets, B0, nullptr, d_in, C, moe::EPI_STORE, workspace, s,
                           perm));
  }
  return ok();
}

moe_status moe_expert_gate_up(const moe_config* cfg, int64_t N, const void* x_sorted,
                              const int32_t* expert_offsets, const void* w1, const void* w3,
                              void* h_sorted, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return expert_call(cfg, N, x_sorted, nullptr, expert_offsets, w1, w3, h_sorted, workspace,
                     workspace_bytes, stream, true, "moe_expert_gate_up");
}

moe_status moe_expert_gate_up_gather(const moe_config* cfg, int64_t N, const void* x_in,
                                     const int32_t* perm, const int32_t* expert_offsets,
                                     const void* w1, const void* w3, void* h_sorted,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_expert_gate_up_gather";
  if (N > 0 && !perm) return fail(MOE_ERR_INVALID_ARG, "%s: perm is NULL", fn);
  return expert_call(cfg, N, x_in, perm, expert_offsets, w1, w3, h_sorted, workspace,
                     workspace_bytes, stream, true, fn);
}

moe_status moe_expert_down(const moe_config* cfg, int64_t N, const void* h_sorted,
                           const int32_t* expert_offsets, const void* w2, void* out_sorted,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return expert_call(cfg, N, h_sorted, nullptr, expert_offsets, w2, nullptr, out_sorted,
                     workspace, workspace_bytes, stream, false, "moe_expert_down");
}

moe_status moe_expert_down_scatter(const moe_config* cfg, int64_t N, const void* h_sorted,
                                   const int32_t* expert_offsets, const int32_t* perm,
                                   const void* w2, void* out_slots, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const char* fn = "moe_expert_down_scatter";
  if (N > 0 && !perm) return fail(MOE_ERR_INVALID_ARG, "%s: perm is NULL", fn);
  return expert_call(cfg, N, h_sorted, perm, expert_offsets, w2, nullptr, out_slots, workspace,
                     workspace_bytes, stream, false, fn);
}

moe_status moe_combine(const moe_config* cfg, int64_t N, const void* out_sorted,
                       const int32_t* inv_perm, const float* topk_weight, const void* residual,
                       void* y, void* stream) {
  const char* fn = "moe_combine";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (N == 0) return ok();
  REQUIRE_PTR(out_sorted);
  REQUIRE_PTR(topk_weight);
  REQUIRE_PTR(y);
  if (residual && !aligned16(residual))
    return fail(MOE_ERR_INVALID_ARG, "%s: residual is not 16-byte aligned", fn);
  CHECK_HIP(moe::launch_combine(out_sorted, inv_perm, topk_weight, residual,
                                is_bf16(cfg) ? 0 : 1, y, N, cfg->top_k,
                                d_in_of(cfg), N * cfg->top_k, is_bf16(cfg) ? 1 : 0,
                                static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status moe_shared_expert(const moe_config* cfg, int64_t N, const void* hidden,
                             const void* sh_w1, const void* sh_w3, const void* sh_w2, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_shared_expert";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (cfg->d_ff_shared <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: the config has no shared expert", fn);
  if (N == 0) return ok();
  REQUIRE_PTR(hidden);
  REQUIRE_PTR(sh_w1);
  REQUIRE_PTR(sh_w3);
  REQUIRE_PTR(sh_w2);
  REQUIRE_PTR(out);
  const Plan p = make_plan(cfg, N, MOE_CALL_SHARED);
  if ((st = check_ws(p, workspace, workspace_bytes, fn)) != MOE_OK) return st;
  CHECK_HIP(shared_expert(cfg, N, hidden, sh_w1, sh_w3, sh_w2, at<void>(workspace, p.sh_h), out,
                          static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status moe_latent_project(const moe_config* cfg, int64_t N, int32_t up, const void* x,
                              const void* w, const float* residual, void* out, void* stream) {
  const char* fn = "moe_latent_project";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (cfg->d_latent <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: the config has no latent width", fn);
  if (up != 0 && up != 1) return fail(MOE_ERR_INVALID_ARG, "%s: up=%d must be 0 or 1", fn, up);
  if (N == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(w);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(residual);
  const int64_t K = up ? cfg->d_latent : cfg->d, n_out = up ? cfg->d : cfg->d_latent;
  const int epi = residual ? moe::EPI_STORE_RES : moe::EPI_STORE;
  CHECK_HIP(dense_gemm(cfg, x, N, K, w, nullptr, n_out, out, epi, residual,
                       static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status moe_block_forward(const moe_config* cfg, int64_t N, const moe_weights* w,
                             const void* hidden, void* y, int32_t* topk_idx_out,
                             float* topk_weight_out, int32_t* tokens_per_expert_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_block_forward";
  moe_status st = validate(cfg, fn);
  if (st != MOE_OK) return st;
  if ((st = validate_n(cfg, N, fn)) != MOE_OK) return st;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "%s: w is NULL", fn);
  if (N == 0) return ok();
  REQUIRE_PTR(hidden);
  REQUIRE_PTR(y);
  REQUIRE_PTR(w->w_router);
  OPTIONAL_PTR(w->bias);  // a router without a bias
  REQUIRE_PTR(w->w1);
  REQUIRE_PTR(w->w3);
  REQUIRE_PTR(w->w2);
  if (cfg->d_latent > 0) {
    REQUIRE_PTR(w->w_down);
    REQUIRE_PTR(w->w_up);
    if (cfg->latent_norm) REQUIRE_PTR(w->gamma);
  }
  if (cfg->d_ff_shared > 0) {
    REQUIRE_PTR(w->sh_w1);
    REQUIRE_PTR(w->sh_w3);
    REQUIRE_PTR(w->sh_w2);
  }
  if (topk_idx_out && !aligned16(topk_idx_out))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_idx_out is not 16-byte aligned", fn);
  if (topk_weight_out && !aligned16(topk_weight_out))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_weight_out is not 16-byte aligned", fn);
  if (tokens_per_expert_out && !aligned16(tokens_per_expert_out))
    return fail(MOE_ERR_INVALID_ARG, "%s: tokens_per_expert_out is not 16-byte aligned", fn);
  const Plan p = make_plan(cfg, N, MOE_CALL_BLOCK);
  if ((st = check_ws(p, workspace, workspace_bytes, fn)) != MOE_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = workspace;
  const int64_t E = cfg->n_experts, k = cfg->top_k, S = N * k;
  const int64_t d = cfg->d, L = cfg->d_latent, d_in = d_in_of(cfg);
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, p.idx);
  float* wts = topk_weight_out ? topk_weight_out : at<float>(ws, p.wts);
  int32_t* counts = tokens_per_expert_out ? tokens_per_expert_out : at<int32_t>(ws, p.counts);
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* perm = at<int32_t>(ws, p.perm);
  int32_t* inv = at<int32_t>(ws, p.inv_perm);

  // latent down projection and shared expert on the full-width input, forked
  // to the side stream; the routed GEMMs wait for the latent input, the output
  // that adds the shared expert for its output
  CHECK_HIP(mark(MOE_STAGE_BEGIN, s));
  void* sh_out = nullptr;
  void* x_lat = L > 0 ? at<void>(ws, p.x_lat) : nullptr;
  std::unique_lock<std::mutex> side_lock;
  Side side{};
  const bool on_side = L > 0 || cfg->d_ff_shared > 0;
  if (cfg->d_ff_shared > 0) sh_out = at<void>(ws, p.sh_out);
  if (on_side) {
    side_lock = std::unique_lock<std::mutex>(g_side_mutex);
    if ((st = side_stream(&side, fn)) != MOE_OK) return st;
    CHECK_HIP(hipEventRecord(side.fork, s));
    CHECK_HIP(hipStreamWaitEvent(side.stream, side.fork, 0));
    if (L > 0) {
      CHECK_HIP(dense_gemm(cfg, hidden, N, d, w->w_down, nullptr, L, x_lat, moe::EPI_STORE,
                           nullptr, side.stream));
      CHECK_HIP(hipEventRecord(side.latent, side.stream));
    }
    if (cfg->d_ff_shared > 0) {
      CHECK_HIP(shared_expert(cfg, N, hidden, w->sh_w1, w->sh_w3, w->sh_w2,
                              at<void>(ws, p.sh_h), static_cast<float*>(sh_out), side.stream));
      CHECK_HIP(hipEventRecord(side.join, side.stream));
    }
  }

  // router on the full-width input
  st = run_route(cfg, N, hidden, w->w_router, w->bias, idx, wts, ws, p, s, fn);
  if (st != MOE_OK) return st;
  CHECK_HIP(mark(MOE_STAGE_ROUTED, s));

  const void* x_in = L > 0 ? x_lat : hidden;
  CHECK_HIP(mark(MOE_STAGE_LATENT, s));

  // dispatch
  uint64_t* bits = at<uint64_t>(ws, p.bits);
  int32_t* base = at<int32_t>(ws, p.base);
  CHECK_HIP(moe::launch_dispatch_mask(idx, N, (int)k, E, bits, s));
  CHECK_HIP(moe::launch_dispatch_scan(bits, p.n_chunks, E, counts, offsets, base, p.rows_per_tile,
                                      at<int32_t>(ws, p.mt_off), at<int32_t>(ws, p.tile_seg),
                                      p.tile_cap, s));
  CHECK_HIP(moe::launch_dispatch_scatter(idx, N, (int)k, E, bits, base, perm, inv, s));
  CHECK_HIP(mark(MOE_STAGE_DISPATCHED, s));

  // the routed GEMMs read the latent input
  if (L > 0) CHECK_HIP(hipStreamWaitEvent(s, side.latent, 0));

  CHECK_HIP(mark(MOE_STAGE_SHARED, s));

  // routed experts: rows gathered through the permutation
  void* h = at<void>(ws, p.h);
  void* out = at<void>(ws, p.out);
  // down: each row written to its token's slot, so the combine reads a
  // token's k rows contiguously
  CHECK_HIP(grouped_gemm(cfg, p, N, x_in, moe::A_GATHER, perm, N, d_in, offsets, w->w1, w->w3,
                         cfg->d_ff, h, moe::EPI_GATE_UP, ws, s));
  CHECK_HIP(mark(MOE_STAGE_GATE_UP, s));
  CHECK_HIP(grouped_gemm(cfg, p, N, h, moe::A_DIRECT, nullptr, S, cfg->d_ff, offsets, w->w2,
                         nullptr, d_in, out, moe::EPI_STORE, ws, s, perm));
  CHECK_HIP(mark(MOE_STAGE_DOWN, s));

  if (L > 0) {
    void* y_lat = at<void>(ws, p.y_lat);
    CHECK_HIP(moe::launch_combine_rmsnorm(out, nullptr, wts, w->gamma, cfg->norm_eps,
                                          cfg->latent_norm ? 1 : 0, y_lat, N, (int)k, L, S,
                                          is_bf16(cfg) ? 1 : 0, s));
    if (sh_out) CHECK_HIP(hipStreamWaitEvent(s, side.join, 0));
    CHECK_HIP(dense_gemm(cfg, y_lat, N, L, w->w_up, nullptr, d, y,
                         sh_out ? moe::EPI_STORE_RES : moe::EPI_STORE, sh_out, s));
  } else {
    if (sh_out) CHECK_HIP(hipStreamWaitEvent(s, side.join, 0));
    CHECK_HIP(moe::launch_combine(out, nullptr, wts, sh_out, 1, y, N, (int)k, d, S,
                                  is_bf16(cfg) ? 1 : 0, s));
  }
  CHECK_HIP(mark(MOE_STAGE_END, s));
  return ok();
}

moe_status moe_set_stage_events(void* const* events, int32_t n_events) {
  const char* fn = "moe_set_stage_events";
  if (!events) {
    g_stage_events_set = false;
    return ok();
  }
  if (n_events != MOE_STAGE_COUNT)
    return fail(MOE_ERR_INVALID_ARG, "%s: %d events given, %d needed", fn, n_events, (int)MOE_STAGE_COUNT);
  for (int i = 0; i < MOE_STAGE_COUNT; ++i) {
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "%s: event %d is NULL", fn, i);
    g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_stage_events_set = true;
  return ok();
}

}  // extern "C"
