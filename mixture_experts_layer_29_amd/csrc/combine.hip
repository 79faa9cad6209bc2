// combine.hip - back to token order and weighted sum (Kimi K3 "Add shared
// output" page, moe-forward excerpt: the un-permute, the product with the fp32
// routing weights, the sum over the k slots, and for the latent block the
// routed-expert norm that precedes the up projection).
//
// One work-group per token row.  The k expert rows are read through inv_perm
// (expert-sorted rows), or, when the down product has already written them in
// slot order, as the token's k contiguous rows n k .. n k + k - 1; they are
// multiplied by their weights and summed in fp32 in slot order j = 0..k-1 (a
// fixed order: results do not depend on scheduling), a residual row (the
// shared expert's output, kept in fp32 by the block) is added, and the sum is
// rounded once.  The latent variant keeps the fp32 row in registers, forms its
// mean square with a fixed-shape tree, and applies y / sqrt(mean(y^2) + eps) *
// gamma before the single rounding.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;            // elements per thread per step
constexpr int kMaxSteps = 8;       // rows up to 256 * 8 * 8 = 16384 elements (norm variant)

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[kVec]) {
  if (BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  } else {
    const float* p = static_cast<const float*>(base) + off;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&v)[kVec]) {
  if (BF16) {
    u32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(base) + off) = q;
  } else {
    float* p = static_cast<float*>(base) + off;
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// Weighted sum of the k expert rows of token n at columns [c, c + 8).
template <bool BF16>
__device__ __forceinline__ void weighted_sum(const void* out_sorted, const int32_t* pos,
                                             const float* w, int k, int64_t width, int64_t c,
                                             float (&acc)[kVec]) {
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.0f;
  for (int j = 0; j < k; ++j) {
    if (pos[j] < 0) continue;
    float v[kVec];
    load8<BF16>(out_sorted, (int64_t)pos[j] * width + c, v);
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc[i] += w[j] * v[i];
  }
}

template <bool BF16, bool RES_F32>
__global__ __launch_bounds__(kThreads) void moe_combine(const void* __restrict__ out_sorted,
                                                        const int32_t* __restrict__ inv_perm,
                                                        const float* __restrict__ wts,
                                                        const void* __restrict__ residual,
                                                        void* __restrict__ y, int64_t N, int k,
                                                        int64_t width, int64_t rows) {
  __shared__ int32_t pos[16];
  __shared__ float w[16];
  const int64_t n = blockIdx.x;
  if (threadIdx.x < k) {
    const int64_t slot = n * k + threadIdx.x;
    const int64_t p = inv_perm ? inv_perm[slot] : slot;
    pos[threadIdx.x] = (p >= 0 && p < rows) ? (int32_t)p : -1;
    w[threadIdx.x] = wts[slot];
  }
  __syncthreads();
  for (int64_t c = (int64_t)threadIdx.x * kVec; c < width; c += kThreads * kVec) {
    float acc[kVec];
    weighted_sum<BF16>(out_sorted, pos, w, k, width, c, acc);
    if (residual) {
      float r[kVec];
      load8<BF16 && !RES_F32>(residual, n * width + c, r);
#pragma unroll
      for (int i = 0; i < kVec; ++i) acc[i] += r[i];
    }
    store8<BF16>(y, n * width + c, acc);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void moe_combine_rmsnorm(
    const void* __restrict__ out_sorted, const int32_t* __restrict__ inv_perm,
    const float* __restrict__ wts, const float* __restrict__ gamma, float eps, int norm,
    void* __restrict__ y, int64_t N, int k, int64_t width, int64_t rows) {
  __shared__ int32_t pos[16];
  __shared__ float w[16];
  __shared__ float red[kThreads];
  const int64_t n = blockIdx.x;
  if (threadIdx.x < k) {
    const int64_t slot = n * k + threadIdx.x;
    const int64_t p = inv_perm ? inv_perm[slot] : slot;
    pos[threadIdx.x] = (p >= 0 && p < rows) ? (int32_t)p : -1;
    w[threadIdx.x] = wts[slot];
  }
  __syncthreads();
  float acc[kMaxSteps][kVec];
  float ss = 0.0f;
#pragma unroll
  for (int st = 0; st < kMaxSteps; ++st) {
    const int64_t c = ((int64_t)st * kThreads + threadIdx.x) * kVec;
    if (c < width) {
      weighted_sum<BF16>(out_sorted, pos, w, k, width, c, acc[st]);
#pragma unroll
      for (int i = 0; i < kVec; ++i) ss += acc[st][i] * acc[st][i];
    }
  }
  float scale = 1.0f;
  if (norm) {
    red[threadIdx.x] = ss;
    __syncthreads();
    for (int half = kThreads / 2; half > 0; half >>= 1) {
      if (threadIdx.x < half) red[threadIdx.x] += red[threadIdx.x + half];
      __syncthreads();
    }
    scale = 1.0f / sqrtf(red[0] / (float)width + eps);
  }
#pragma unroll
  for (int st = 0; st < kMaxSteps; ++st) {
    const int64_t c = ((int64_t)st * kThreads + threadIdx.x) * kVec;
    if (c < width) {
      float v[kVec];
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        v[i] = acc[st][i];
        if (norm) v[i] = v[i] * scale * gamma[c + i];
      }
      store8<BF16>(y, n * width + c, v);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* out_sorted, const int32_t* inv_perm, const float* w,
                          const void* residual, int res_f32, void* y, int64_t N, int k,
                          int64_t width, int64_t rows, int bf16, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const dim3 g((unsigned)N), b(kThreads);
  if (bf16 && res_f32) {
    moe_combine<true, true><<<g, b, 0, s>>>(out_sorted, inv_perm, w, residual, y, N, k, width, rows);
  } else if (bf16) {
    moe_combine<true, false><<<g, b, 0, s>>>(out_sorted, inv_perm, w, residual, y, N, k, width,
                                             rows);
  } else {
    moe_combine<false, true><<<g, b, 0, s>>>(out_sorted, inv_perm, w, residual, y, N, k, width,
                                             rows);
  }
  return hipGetLastError();
}

int64_t combine_rmsnorm_max_width() { return (int64_t)kThreads * kVec * kMaxSteps; }

hipError_t launch_combine_rmsnorm(const void* out_sorted, const int32_t* inv_perm, const float* w,
                                  const float* gamma, float eps, int norm, void* y, int64_t N,
                                  int k, int64_t width, int64_t rows, int bf16, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (width > combine_rmsnorm_max_width()) return hipErrorInvalidValue;
  if (bf16) {
    moe_combine_rmsnorm<true><<<dim3((unsigned)N), dim3(kThreads), 0, s>>>(
        out_sorted, inv_perm, w, gamma, eps, norm, y, N, k, width, rows);
  } else {
    moe_combine_rmsnorm<false><<<dim3((unsigned)N), dim3(kThreads), 0, s>>>(
        out_sorted, inv_perm, w, gamma, eps, norm, y, N, k, width, rows);
  }
  return hipGetLastError();
}

}  // namespace moe
