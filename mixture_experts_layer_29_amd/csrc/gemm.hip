// gemm.hip - the grouped GEMMs of the routed experts, and the dense GEMMs of the
// shared expert, the latent projections and the router.
//
// Every product here is C[row, col] = sum_k A[row, k] * W[col, k]: activations
// A row-major, weights W in nn.Linear layout [cols, K] (the expert excerpt of the
// Kimi K3 "Gate features" page: w1, w3 [d_ff, d_in], w2 [d_in, d_ff], no bias).
// Rows are grouped in segments (one per expert, from the expert offsets of the
// dispatch), or form one dense segment.
//
// bf16 kernel (moe_gemm_bf16), designed for CDNA4's MFMA units and for the fact
// that at every MoE size of interest the expert weights, not the flops, set the
// time (each weight byte feeds only T_e rows):
//  - a work-group (4 waves) owns one (segment, n-tile, m-tile); each wave owns two
//    32-column blocks of the output and streams its weight rows straight from
//    HBM into registers in the operand layout of v_mfma_f32_32x32x16_bf16, with a
//    register ring D blocks deep (no LDS round trip for the weights: each weight
//    element is used by exactly one wave);
//  - the activation tile (up to RB x 32 rows x 64 k) is shared by the 4 waves
//    through double-buffered LDS (rows padded to 144 B: conflict-free b128 reads);
//    in gather mode its rows are read through the dispatch permutation, so the
//    expert-sorted copy of the input never has to be written;
//  - row blocks of 32 without rows are skipped, so one kernel serves decode
//    (a few rows per expert) and prefill (hundreds);
//  - tiles are numbered segment-major, then n-tile, then m-tile, and mapped to
//    work-group ids so that consecutive tile numbers land on the same XCD: the
//    m-tiles sharing a weight tile and the n-tiles sharing an activation tile run
//    together under one L2;
//  - the epilogue applies SiLU/SiTU-and-mul (fp32) or adds a residual, and
//    rounds once.
// The K axis inside a 64-block is visited in a lane order of our choosing (the
// same for both operands), which lets each lane read 64 contiguous bytes of a
// weight row per block.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLds = 72;  // bf16 per LDS row: 64 + 8 pad

__device__ __forceinline__ int remap_xcd(int bid, int nwg) {
  const int per = nwg >> 3;  // nwg is a multiple of 8
  return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ float act_pair(int act, float g, float u, float beta, float lbeta) {
  if (act == ACT_SILU) return g / (1.0f + expf(-g)) * u;
  const float a = beta * tanhf(g / beta) * (1.0f / (1.0f + expf(-g)));
  const float up = lbeta > 0.0f ? lbeta * tanhf(u / lbeta) : u;
  return a * up;
}

struct TileLoc {
  int64_t seg;
  int64_t row0;   // first row of the tile (in the segment-concatenated row space)
  int rows;       // rows of the tile that exist (1 .. BM)
  int64_t j;      // n-tile
};

// Locates logical tile L; returns false when L is past the last tile.
template <int BM>
__device__ __forceinline__ bool locate(const GemmArgs& a, int64_t L, int64_t n_tiles_n, TileLoc& t) {
  if (a.seg_off) {
    // tile_seg[u] is the segment of m-tile u, or -1 past the last m-tile
    const int64_t u = L / n_tiles_n;
    if (u >= a.tile_cap) return false;
    const int32_t seg = a.tile_seg[u];
    if (seg < 0) return false;
    const int64_t MB = a.mt_off[seg];
    const int64_t mt = a.mt_off[seg + 1] - MB;
    const int64_t r = L - MB * n_tiles_n;
    const int64_t j = r / mt, i = r - j * mt;
    const int64_t s0 = a.seg_off[seg];
    const int64_t s1 = min((int64_t)a.seg_off[seg + 1], a.c_rows);
    t.seg = seg;
    t.row0 = s0 + i * BM;
    t.rows = (int)min((int64_t)BM, s1 - t.row0);
    t.j = j;
    return t.row0 >= 0 && t.rows > 0;
  }
  const int64_t mt = (a.dense_rows + BM - 1) / BM;
  if (L >= mt * n_tiles_n) return false;
  const int64_t j = L / mt, i = L - j * mt;
  t.seg = 0;
  t.row0 = i * BM;
  t.rows = (int)min((int64_t)BM, a.dense_rows - t.row0);
  t.j = j;
  return true;
}

template <int RB, int EPI, int AMODE, int D>
__global__ __launch_bounds__(kThreads) void moe_gemm_bf16(GemmArgs a, int64_t n_tiles_n) {
  constexpr int BM = RB * 32;
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;  // output columns per wave
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM][kLds];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  TileLoc t;
  if (!locate<BM>(a, remap_xcd(blockIdx.x, gridDim.x), n_tiles_n, t)) return;
  const int nrb = (t.rows + 31) >> 5;
  const int64_t K = a.K;
  const int64_t nkb = (K + 63) >> 6;

  // ---- weight pointers of this lane (column lane&31 of the wave's two blocks)
  const int64_t cb0 = t.j * (kWaves * CPW) + (int64_t)wave * CPW;
  const int64_t cb1 = (EPI == EPI_GATE_UP) ? cb0 : cb0 + 32;
  const int64_t cl = lane & 31;
  const bool ok0 = cb0 + cl < a.n_cols, ok1 = cb1 + cl < a.n_cols;
  const int64_t c0 = ok0 ? cb0 + cl : a.n_cols - 1;
  const int64_t c1 = ok1 ? cb1 + cl : a.n_cols - 1;
  const bf16_t* W0 = static_cast<const bf16_t*>(a.B0) + t.seg * a.b_seg_stride;
  const bf16_t* W1 = static_cast<const bf16_t*>(EPI == EPI_GATE_UP ? a.B1 : a.B0) + t.seg * a.b_seg_stride;
  const int kq = (lane >> 5) * 32;  // this lane's 32-element half of each 64-block
  const bf16_t* bp0 = W0 + c0 * K + kq;
  const bf16_t* bp1 = W1 + c1 * K + kq;

  // ---- activation rows this thread stages (RB chunks of 16 B)
  const int seg8 = tid & 7;
  const bf16_t* ap[RB];
  bool arow_ok[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int row = (tid >> 3) + 32 * r;
    arow_ok[r] = row < t.rows;
    int64_t src = t.row0 + (arow_ok[r] ? row : 0);
    if (AMODE == A_GATHER) {
      int64_t slot = a.a_map[src];
      src = slot / a.a_div;
    }
    src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
    ap[r] = static_cast<const bf16_t*>(a.A) + src * a.lda + seg8 * 8;
  }

  auto load_a = [&](int64_t kb, u32x4 (&areg)[RB]) {
    int64_t col;
    bool kok;
    if (AMODE == A_REPEAT) {
      const int64_t per_blocks = a.a_period >> 6;
      col = (kb % per_blocks) * 64;
      kok = col + seg8 * 8 < a.a_valid;
    } else {
      col = kb * 64;
      kok = col + seg8 * 8 < K;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (arow_ok[r] && kok) {
        areg[r] = *reinterpret_cast<const u32x4*>(ap[r] + col);
      } else {
        areg[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a = [&](int buf, const u32x4 (&areg)[RB]) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = (tid >> 3) + 32 * r;
      if (r < nrb) *reinterpret_cast<u32x4*>(&As[buf][row][seg8 * 8]) = areg[r];
    }
  };

  u32x4 breg[D][2][4];
  auto load_b = [&](int64_t kb, u32x4 (&b)[2][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t k = kb * 64 + kq + s * 8;
      if (k < K) {
        b[0][s] = *reinterpret_cast<const u32x4*>(bp0 + kb * 64 + s * 8);
        b[1][s] = *reinterpret_cast<const u32x4*>(bp1 + kb * 64 + s * 8);
      } else {
        b[0][s] = u32x4{0u, 0u, 0u, 0u};
        b[1][s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][c][r] = 0.0f;
    }
  }

  auto compute = [&](int buf, const u32x4 (&b)[2][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb) {
          af[rb] = *reinterpret_cast<const bf16x8*>(&As[buf][rb * 32 + (lane & 31)][(lane >> 5) * 32 + s * 8]);
        }
      }
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, b[0][s]);
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, b[1][s]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb) {
          acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], b0, acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], b1, acc[rb][1], 0, 0, 0);
        }
      }
    }
  };

  // ---- software pipeline: A one block ahead through LDS, B D blocks ahead in registers
  {
    u32x4 areg[RB];
    load_a(0, areg);
#pragma unroll
    for (int q = 0; q < D; ++q) {
      if (q < nkb) load_b(q, breg[q]);
    }
    store_a(0, areg);
  }
  __syncthreads();

  for (int64_t kb0 = 0; kb0 < nkb; kb0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int64_t kb = kb0 + q;
      if (kb < nkb) {
        u32x4 areg[RB];
        const bool more = kb + 1 < nkb;
        if (more) load_a(kb + 1, areg);
        compute((int)(kb & 1), breg[q]);
        if (kb + D < nkb) load_b(kb + D, breg[q]);
        if (more) store_a((int)((kb + 1) & 1), areg);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: lane holds column lane&31 and rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (rb >= nrb) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= t.rows) continue;
      const int64_t orow = t.row0 + row;
      if (EPI == EPI_GATE_UP) {
        if (ok0) {
          const float h = act_pair(a.act, acc[rb][0][r], acc[rb][1][r], a.beta, a.lbeta);
          static_cast<bf16_t*>(a.C)[orow * a.ldc + c0] = f32_to_bf16(h);
        }
      } else if (EPI == EPI_STORE_F32) {
        if (ok0) static_cast<float*>(a.C)[orow * a.ldc + c0] = acc[rb][0][r];
        if (ok1) static_cast<float*>(a.C)[orow * a.ldc + c1] = acc[rb][1][r];
      } else {
        float v0 = acc[rb][0][r], v1 = acc[rb][1][r];
        if (EPI == EPI_STORE_RES) {
          const bf16_t* res = static_cast<const bf16_t*>(a.residual) + orow * a.ld_res;
          if (ok0) v0 += bf16_to_f32(res[c0]);
          if (ok1) v1 += bf16_to_f32(res[c1]);
        }
        if (ok0) static_cast<bf16_t*>(a.C)[orow * a.ldc + c0] = f32_to_bf16(v0);
        if (ok1) static_cast<bf16_t*>(a.C)[orow * a.ldc + c1] = f32_to_bf16(v1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64 x 64 output tile (for EPI_GATE_UP: 64 columns of both
// products), 256 threads of 4 x 4 outputs, K in steps of 16 through LDS.
constexpr int kF32Rows = 64;

template <int EPI, int AMODE>
__global__ __launch_bounds__(kThreads) void moe_gemm_f32(GemmArgs a, int64_t n_tiles_n) {
  __shared__ float As[16][kF32Rows + 1];
  __shared__ float Bs[2][16][64 + 1];
  const int tid = threadIdx.x;
  TileLoc t;
  if (!locate<kF32Rows>(a, remap_xcd(blockIdx.x, gridDim.x), n_tiles_n, t)) return;
  const int64_t K = a.K;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t col0 = t.j * 64;
  const float* W0 = static_cast<const float*>(a.B0) + t.seg * a.b_seg_stride;
  const float* W1 = EPI == EPI_GATE_UP ? static_cast<const float*>(a.B1) + t.seg * a.b_seg_stride : W0;

  // loader roles: thread -> (row r = tid / 4, k quad q = tid % 4)
  const int lr = tid >> 2, lq = (tid & 3) * 4;
  int64_t asrc;
  {
    const bool ok = lr < t.rows;
    int64_t src = t.row0 + (ok ? lr : 0);
    if (AMODE == A_GATHER) src = a.a_map[src] / a.a_div;
    asrc = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
  }
  const bool arow_ok = lr < t.rows;
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
      float av = 0.0f;
      if (arow_ok && k < K) {
        if (AMODE == A_REPEAT) {
          const int64_t col = k % a.a_period;
          av = col < a.a_valid ? static_cast<const float*>(a.A)[asrc * a.lda + col] : 0.0f;
        } else {
          av = static_cast<const float*>(a.A)[asrc * a.lda + k];
        }
      }
      As[lq + e][lr] = av;
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
        b1[j] = Bs[1][kk][tx * 4 + j];
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
      if (EPI == EPI_GATE_UP) v = act_pair(a.act, acc[0][i][j], acc[1][i][j], a.beta, a.lbeta);
      if (EPI == EPI_STORE_RES) v += static_cast<const float*>(a.residual)[orow * a.ld_res + col];
      static_cast<float*>(a.C)[orow * a.ldc + col] = v;
    }
  }
}

int64_t round8(int64_t n) { return (n + 7) & ~(int64_t)7; }

template <int RB, int EPI, int AMODE>
hipError_t launch_rb(const GemmArgs& a, int64_t mt_cap, hipStream_t s) {
  constexpr int D = (RB >= 4) ? 3 : 2;
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;
  const int64_t n_tiles_n = (a.n_cols + kWaves * CPW - 1) / (kWaves * CPW);
  const int64_t mt = a.seg_off ? mt_cap : (a.dense_rows + RB * 32 - 1) / (RB * 32);
  const int64_t grid = round8(mt * n_tiles_n);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_bf16<RB, EPI, AMODE, D><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, n_tiles_n);
  return hipGetLastError();
}

template <int EPI, int AMODE>
hipError_t launch_rb_any(const GemmArgs& a, int rb, int64_t mt_cap, hipStream_t s) {
  switch (rb) {
    case 1: return launch_rb<1, EPI, AMODE>(a, mt_cap, s);
    case 2: return launch_rb<2, EPI, AMODE>(a, mt_cap, s);
    case 4: return launch_rb<4, EPI, AMODE>(a, mt_cap, s);
    default: return hipErrorInvalidValue;
  }
}

template <int EPI, int AMODE>
hipError_t launch_f32(const GemmArgs& a, int64_t mt_cap, hipStream_t s) {
  const int64_t n_tiles_n = (a.n_cols + 63) / 64;
  const int64_t mt = a.seg_off ? mt_cap : (a.dense_rows + kF32Rows - 1) / kF32Rows;
  const int64_t grid = round8(mt * n_tiles_n);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_f32<EPI, AMODE><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, n_tiles_n);
  return hipGetLastError();
}

}  // namespace

int gemm_f32_rows_per_tile() { return kF32Rows; }

hipError_t launch_gemm_bf16(const GemmArgs& a, int epi, int amode, int rb, int64_t mt_cap,
                            hipStream_t s) {
  if (epi == EPI_GATE_UP && amode == A_DIRECT) return launch_rb_any<EPI_GATE_UP, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_GATE_UP && amode == A_GATHER) return launch_rb_any<EPI_GATE_UP, A_GATHER>(a, rb, mt_cap, s);
  if (epi == EPI_STORE && amode == A_DIRECT) return launch_rb_any<EPI_STORE, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_STORE_RES && amode == A_DIRECT) return launch_rb_any<EPI_STORE_RES, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_STORE_F32 && amode == A_REPEAT) return launch_rb_any<EPI_STORE_F32, A_REPEAT>(a, rb, mt_cap, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GemmArgs& a, int epi, int amode, int64_t mt_cap, hipStream_t s) {
  if (epi == EPI_GATE_UP && amode == A_DIRECT) return launch_f32<EPI_GATE_UP, A_DIRECT>(a, mt_cap, s);
  if (epi == EPI_GATE_UP && amode == A_GATHER) return launch_f32<EPI_GATE_UP, A_GATHER>(a, mt_cap, s);
  if ((epi == EPI_STORE || epi == EPI_STORE_F32) && amode == A_DIRECT) return launch_f32<EPI_STORE, A_DIRECT>(a, mt_cap, s);
  if (epi == EPI_STORE_RES && amode == A_DIRECT) return launch_f32<EPI_STORE_RES, A_DIRECT>(a, mt_cap, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
