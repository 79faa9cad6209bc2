// route.hip - the router's kernels (Kimi K2 "Affinities" page, gate-forward
// excerpt; DeepSeek-V3.2-Exp "Affinities" page, gate-forward excerpt).
//
// The router's linear layer is fp32 on the pages.  With a bf16 hidden state the
// product runs on the bf16 MFMA units without losing fp32 accuracy: each fp32
// weight w is split exactly into three bf16 terms hi + mid + lo (8 significant
// bits each, 24 in all), every product of a bf16 hidden value with a bf16 term
// is exact in fp32, and the MFMA accumulates all three in fp32.  The split is
// laid out as one bf16 matrix [E, 3 * dp] (dp = d rounded up to 64, zero pad),
// so the dense streaming GEMM computes logits = [x x x] . split^T directly.
//
// moe_route_select then takes one token per wave: sigmoid scores (or the
// softmax over the token's experts, DeepSeek-V3.2-Exp gate), bias added for
// the choice only (a router may have none), per-group sum of the two largest
// choice values (the largest one when there is no bias), the best topk_group
// groups, the top_k choice values among them by k rounds of a wave-wide
// arg-max (larger value, then lower index), weights from the unbiased scores,
// renormalised (+1e-20, when top_k > 1 and asked for) and scaled.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bf16_t rne_bf16(float f) { return f32_to_bf16(f); }

// w_split[e][part * dp + i] = part-th bf16 term of w_router[e][i] (0 for i >= d).
__global__ __launch_bounds__(kThreads) void moe_router_split(const float* __restrict__ w,
                                                             int64_t E, int64_t d, int64_t dp,
                                                             bf16_t* __restrict__ out) {
  const int64_t total = E * dp;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t e = i / dp, c = i - e * dp;
    const float v = c < d ? w[e * d + c] : 0.0f;
    const bf16_t hi = rne_bf16(v);
    const float r1 = v - bf16_to_f32(hi);  // exact (Sterbenz)
    const bf16_t mid = rne_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);  // exact, at most 8 significant bits
    const bf16_t lo = rne_bf16(r2);
    bf16_t* row = out + e * 3 * dp;
    row[c] = hi;
    row[dp + c] = mid;
    row[2 * dp + c] = lo;
  }
}

// (value, index) order used for every choice: larger value wins, then lower index.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide arg-max of (v, i) with a payload p; every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i, float& p) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m, 64);
    const int oi = __shfl_xor(i, m, 64);
    const float op = __shfl_xor(p, m, 64);
    if (beats(ov, oi, v, i)) {
      v = ov;
      i = oi;
      p = op;
    }
  }
}

constexpr int kMaxG = 1024;

// One token per wave; P = values per lane (expert e = i * 64 + lane).
template <int P>
__global__ __launch_bounds__(kThreads) void moe_route_select(
    const float* __restrict__ logits, int n_parts, int64_t part_stride,
    const float* __restrict__ bias, int softmax, int64_t N, int E, int G,
    int TG, int k, int norm, float scale, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_weight) {
  __shared__ float sh_b[4][kMaxG];   // choice values (group stage only)
  __shared__ float sh_gs[4][kMaxG];  // group scores
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  const bool live = n < N;

  float s[P], b[P];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = i * 64 + lane;
    if (live && e < E) {
      // the router product may arrive as partial sums over K ranges: added
      // in range order, so the logit does not depend on the launch
      const float* src = logits + n * E + e;
      float l = src[0];
      // loads in batches of 8 (independent), then added in range order
      for (int q0 = 1; q0 < n_parts; q0 += 8) {
        float part[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) part[q] = q0 + q < n_parts ? src[(q0 + q) * part_stride] : 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q0 + q < n_parts) l += part[q];
        }
      }
      s[i] = l;
      lmax = fmaxf(lmax, l);
    } else {
      s[i] = -INFINITY;
    }
  }
  if (softmax) {
    // softmax over the token's E logits: exp(l - max) / sum, in fp32
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, m, 64));
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      s[i] = (i * 64 + lane < E) ? expf(s[i] - lmax) : 0.0f;
      sum += s[i];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int i = 0; i < P; ++i) s[i] *= inv;
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) s[i] = (i * 64 + lane < E) ? 1.0f / (1.0f + expf(-s[i])) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = i * 64 + lane;
    b[i] = (live && e < E) ? (bias ? s[i] + bias[e] : s[i]) : -INFINITY;
  }

  if (G > 1) {
    const int per = E / G;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = i * 64 + lane;
      if (e < E) sh_b[wave][e] = b[i];
    }
    __syncthreads();
    // group g: sum of its two largest choice values (the largest alone for a
    // router without a bias)
    for (int g = lane; g < G; g += 64) {
      float t1 = -INFINITY, t2 = -INFINITY;
      for (int e = g * per; e < (g + 1) * per; ++e) {
        const float v = sh_b[wave][e];
        if (v > t1) {
          t2 = t1;
          t1 = v;
        } else if (v > t2) {
          t2 = v;
        }
      }
      sh_gs[wave][g] = bias ? t1 + t2 : t1;
    }
    __syncthreads();
    // keep TG groups: TG rounds of arg-max over the group scores; a kept
    // group's score is replaced by +inf, which no real group score reaches
    for (int r = 0; r < TG; ++r) {
      float bv = -INFINITY, dummy = 0.0f;
      int bi = 0x7FFFFFFF;
      for (int g = lane; g < G; g += 64) {
        const float v = sh_gs[wave][g];
        if (v != INFINITY && beats(v, g, bv, bi)) {
          bv = v;
          bi = g;
        }
      }
      wave_argmax(bv, bi, dummy);
      if (lane == 0) sh_gs[wave][bi] = INFINITY;
      __syncthreads();
    }
    // experts of groups not kept can never be chosen
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = i * 64 + lane;
      if (e < E && sh_gs[wave][e / per] != INFINITY) b[i] = -INFINITY;
    }
  }

  // top-k: k rounds of arg-max; the winner's value is retired
  int sel_e[16];
  float sel_s[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sel_e[j] = 0x7FFFFFFF;
    sel_s[j] = 0.0f;
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY, bs = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int e = i * 64 + lane;
      if (e < E && b[i] != -INFINITY && beats(b[i], e, bv, bi)) {
        bv = b[i];
        bi = e;
        bs = s[i];
      }
    }
    wave_argmax(bv, bi, bs);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i * 64 + lane == bi) b[i] = -INFINITY;
    }
    // store into slot j (j is uniform; unrolled select keeps registers static)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q == j) {
        sel_e[q] = bi;
        sel_s[q] = bs;
      }
    }
  }

  // ascending expert id (insertion sort of at most 16 uniform values)
#pragma unroll
  for (int a = 1; a < 16; ++a) {
#pragma unroll
    for (int c = a; c > 0; --c) {
      if (sel_e[c] < sel_e[c - 1]) {
        const int te = sel_e[c];
        sel_e[c] = sel_e[c - 1];
        sel_e[c - 1] = te;
        const float ts = sel_s[c];
        sel_s[c] = sel_s[c - 1];
        sel_s[c - 1] = ts;
      }
    }
  }

  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < k) sum += sel_s[q];
  }
  const bool renorm = norm && k > 1;
  if (live) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < k && lane == q) {
        float w = sel_s[q];
        if (renorm) w = w / (sum + 1e-20f);
        topk_idx[n * k + q] = sel_e[q];
        topk_weight[n * k + q] = w * scale;
      }
    }
  }
}

template <int P>
hipError_t launch_select(const float* logits, int n_parts, int64_t part_stride, const float* bias,
                         int softmax, int64_t N, int64_t E, int G, int TG, int k, int norm,
                         float scale, int32_t* idx, float* w, hipStream_t s) {
  const int64_t grid = (N + 3) / 4;
  moe_route_select<P><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(
      logits, n_parts, part_stride, bias, softmax, N, (int)E, G, TG, k, norm, scale, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_split(const float* w_router, int64_t E, int64_t d, int64_t dp,
                               bf16_t* w_split, hipStream_t s) {
  const int64_t total = E * dp;
  int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > 16384) grid = 16384;
  moe_router_split<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(w_router, E, d, dp, w_split);
  return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, int n_parts, int64_t part_stride,
                               const float* bias, int softmax, int64_t N, int64_t E,
                               int G, int TG, int k, int norm, float scale, int32_t* topk_idx,
                               float* topk_weight, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (n_parts < 1) return hipErrorInvalidValue;
  const int64_t P = (E + 63) / 64;
#define MOE_SELECT(PP)                                                                       \
  return launch_select<PP>(logits, n_parts, part_stride, bias, softmax, N, E, G, TG, k, norm, scale, \
                           topk_idx, topk_weight, s)
  if (P <= 1) MOE_SELECT(1);
  if (P <= 2) MOE_SELECT(2);
  if (P <= 4) MOE_SELECT(4);
  if (P <= 8) MOE_SELECT(8);
  if (P <= 16) MOE_SELECT(16);
#undef MOE_SELECT
  return hipErrorInvalidValue;
}

}  // namespace moe
