// gemm_f32.hip - fp32 SIMT GEMM for blocks stored in fp32 (the tiny workload):
// the same products, segments, gather and epilogues as the bf16 MFMA kernel
// (C[row, col] = sum_k A[row, k] * W[col, k], weights [cols, K]), on plain FMAs.
// A 64 x 64 output tile per work-group (for the gate/up product, 64 columns of
// both w1 and w3), 256 threads of 4 x 4 outputs, K in steps of 16 through LDS.
#include "gemm_common.h"

namespace moe {
namespace {

using gemm::TileLoc;

constexpr int kThreads = 256;
constexpr int kRows = 64;

template <int EPI, int AMODE>
__global__ __launch_bounds__(kThreads) void moe_gemm_f32(GemmArgs a, int64_t n_tiles_n) {
  __shared__ float As[16][kRows + 1];
  __shared__ float Bs[2][16][64 + 1];
  const int tid = threadIdx.x;
  int64_t L, end, step;
  gemm::tile_range<kRows>(a, blockIdx.x, gridDim.x, n_tiles_n, L, end, step);
  for (; L < end; L += step) {
  TileLoc t;
  if (!gemm::locate<kRows>(a, L, n_tiles_n, t)) continue;
  const int64_t K = a.K;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t col0 = t.j * 64;
  const float* W0 = static_cast<const float*>(a.B0) + t.seg * a.b_seg_stride;
  const float* W1 =
      EPI == EPI_GATE_UP ? static_cast<const float*>(a.B1) + t.seg * a.b_seg_stride : W0;

  // loader roles: thread -> (row / column lr = tid / 4, k quad lq = 4 * (tid % 4))
  const int lr = tid >> 2, lq = (tid & 3) * 4;
  const bool arow_ok = lr < t.rows;
  int64_t asrc = t.row0 + (arow_ok ? lr : 0);
  if (AMODE == A_GATHER) asrc = a.a_map[asrc] / a.a_div;
  asrc = asrc < 0 ? 0 : (asrc >= a.a_rows ? a.a_rows - 1 : asrc);
  const int64_t bcol = col0 + lr;
  const bool bcol_ok = bcol < a.n_cols;

  float acc[2][4][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[c][i][j] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t k = k0 + lq + e;
      As[lq + e][lr] = (arow_ok && k < K) ? static_cast<const float*>(a.A)[asrc * a.lda + k] : 0.0f;
      const bool bk = bcol_ok && k < K;
      Bs[0][lq + e][lr] = bk ? W0[bcol * K + k] : 0.0f;
      if (EPI == EPI_GATE_UP) Bs[1][lq + e][lr] = bk ? W1[bcol * K + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs[0][kk][tx * 4 + j];
        b1[j] = EPI == EPI_GATE_UP ? Bs[1][kk][tx * 4 + j] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][i][j] += av[i] * b0[j];
          if (EPI == EPI_GATE_UP) acc[1][i][j] += av[i] * b1[j];
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= t.rows) continue;
    const int64_t orow = t.row0 + row;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + tx * 4 + j;
      if (col >= a.n_cols) continue;
      float v = acc[0][i][j];
      if (EPI == EPI_GATE_UP) v = gemm::act_pair(a.act, acc[0][i][j], acc[1][i][j], a.beta, a.lbeta);
      if (EPI == EPI_STORE_RES) v += static_cast<const float*>(a.residual)[orow * a.ld_res + col];
      const int64_t crow = (EPI == EPI_STORE && a.c_map) ? a.c_map[orow] : orow;
      static_cast<float*>(a.C)[crow * a.ldc + col] = v;
    }
  }
  }
}

template <int EPI, int AMODE>
hipError_t launch(const GemmArgs& a, int64_t mt_cap, hipStream_t s) {
  const int64_t n_tiles_n = (a.n_cols + 63) / 64;
  const int64_t mt = a.seg_off ? mt_cap : (a.dense_rows + kRows - 1) / kRows;
  const int64_t grid = gemm::round8(mt * n_tiles_n);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_f32<EPI, AMODE><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, n_tiles_n);
  return hipGetLastError();
}

}  // namespace

int gemm_f32_rows_per_tile() { return kRows; }

hipError_t launch_gemm_f32(const GemmArgs& a, int epi, int amode, int64_t mt_cap, hipStream_t s) {
  if (a.k_splits > 1) return hipErrorInvalidValue;  // split-K is a bf16-path option only
  if (epi == EPI_GATE_UP && amode == A_DIRECT) return launch<EPI_GATE_UP, A_DIRECT>(a, mt_cap, s);
  if (epi == EPI_GATE_UP && amode == A_GATHER) return launch<EPI_GATE_UP, A_GATHER>(a, mt_cap, s);
  if ((epi == EPI_STORE || epi == EPI_STORE_F32) && amode == A_DIRECT)
    return launch<EPI_STORE, A_DIRECT>(a, mt_cap, s);
  if (epi == EPI_STORE_RES && amode == A_DIRECT) return launch<EPI_STORE_RES, A_DIRECT>(a, mt_cap, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
