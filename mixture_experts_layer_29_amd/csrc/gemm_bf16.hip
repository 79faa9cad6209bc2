// gemm_bf16.hip - bf16 MFMA GEMM for the routed experts (grouped over the
// expert-sorted row segments) and for the dense products of the block (shared
// expert, latent projections, router).
//
// Every product is C[row, col] = sum_k A[row, k] * W[col, k]: activations A
// row-major, weights W in nn.Linear layout [cols, K] (the expert excerpt of the
// Kimi K3 "Gate features" page: w1, w3 [d_ff, d_in], w2 [d_in, d_ff], no bias).
//
// Design for CDNA4, where at every MoE size of interest the expert weights, not
// the flops, set the time (each weight byte feeds only the T_e rows routed to
// its expert):
//  - a work-group (4 waves) owns one (segment, n-tile, m-tile); each wave owns
//    two 32-column blocks of the output and streams its weight rows straight
//    from HBM into registers in the operand layout of
//    v_mfma_f32_32x32x16_bf16, D blocks of 64 k ahead (no LDS round trip for
//    weights: each weight element feeds exactly one wave);
//  - the activation tile (up to RB x 32 rows x 64 k) is shared by the 4 waves
//    through double-buffered LDS, loaded into registers two blocks ahead; in
//    gather mode its rows are read through the dispatch permutation, so no
//    expert-sorted copy of the input is ever written;
//  - the steady-state loop has no branches and no data-dependent waits: every
//    load is unconditional, the loads of an iteration are issued in the order
//    A(kb+2), B(kb+D) so that the in-order vmcnt wait before an LDS store never
//    waits on weight loads issued after it; the last blocks are peeled;
//  - the number of 32-row blocks that hold rows is a template parameter, so a
//    tile with few rows issues only the MFMAs it needs (decode tiles of a few
//    rows and prefill tiles of hundreds run the same kernel);
//  - tiles are numbered segment-major, then n-tile, then m-tile, and mapped to
//    work-group ids so that consecutive tiles land on the same XCD (weight and
//    activation tiles shared under one L2);
//  - the epilogue stages the fp32 accumulators through LDS, applies
//    SiLU/SiTU-and-mul or the residual add in fp32, rounds once and writes
//    16-byte row-contiguous chunks.
// Inside a 64-wide K block the lanes visit K in an order of our choosing, the
// same for both operands, which lets a lane read 64 contiguous bytes of its
// weight row per block.
#include "gemm_common.h"

namespace moe {
namespace {

using gemm::TileLoc;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLdsA = 72;    // bf16 per LDS activation row: 64 + 8 pad (conflict-free b128 reads)
constexpr int kLdsOut = 72;  // fp32 per LDS epilogue row: 64 + 8 pad
constexpr int kLdsBytesOut = kWaves * 32 * kLdsOut * 4;

template <int RB>
struct Smem {
  static constexpr int kA = 2 * RB * 32 * kLdsA * 2;
  static constexpr int kBytes = kA > kLdsBytesOut ? kA : kLdsBytesOut;
};

template <int NR, int RB, int EPI, int AMODE, int D, bool KT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const TileLoc& t, uint8_t* smem) {
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;  // output columns per wave
  constexpr int U = (D % 2 == 0) ? D : 2 * D;          // unroll: ring slots stay static
  bf16_t(*As)[RB * 32][kLdsA] = reinterpret_cast<bf16_t(*)[RB * 32][kLdsA]>(smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t K = a.K;
  const int64_t nkb = (K + 63) >> 6;

  // ---- weight rows of this lane: column lane&31 of the wave's two blocks
  const int64_t cb0 = t.j * (kWaves * CPW) + (int64_t)wave * CPW;
  const int64_t cb1 = (EPI == EPI_GATE_UP) ? cb0 : cb0 + 32;
  const int64_t cl = lane & 31;
  const int64_t c0 = min(cb0 + cl, a.n_cols - 1);
  const int64_t c1 = min(cb1 + cl, a.n_cols - 1);
  const bf16_t* W0 = static_cast<const bf16_t*>(a.B0) + t.seg * a.b_seg_stride;
  const bf16_t* W1 =
      static_cast<const bf16_t*>(EPI == EPI_GATE_UP ? a.B1 : a.B0) + t.seg * a.b_seg_stride;
  const int kq = (lane >> 5) * 32;  // this lane's 32-element half of each 64-block
  const bf16_t* bp0 = W0 + c0 * K + kq;
  const bf16_t* bp1 = W1 + c1 * K + kq;

  // ---- activation rows this thread stages: NR chunks of 16 bytes
  const int seg8 = tid & 7;
  const bf16_t* ap[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = (tid >> 3) + 32 * r;
    int64_t src = t.row0 + (row < t.rows ? row : 0);
    if (AMODE == A_GATHER) src = a.a_map[src] / a.a_div;
    src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
    ap[r] = static_cast<const bf16_t*>(a.A) + src * a.lda + seg8 * 8;
  }
  const int64_t a_per_blocks = AMODE == A_REPEAT ? (a.a_period >> 6) : 1;

  auto a_col = [&](int64_t kb) -> int64_t {
    int64_t col = (AMODE == A_REPEAT ? (kb % a_per_blocks) : kb) * 64;
    if (AMODE == A_REPEAT) {
      // columns past the valid width meet zero weights: any finite value will do
      col = min(col, a.a_valid - 8 - seg8 * 8);
    } else if (KT) {
      col = min(col, K - 8 - seg8 * 8);
    }
    return col;
  };
  auto load_a = [&](int64_t kb, u32x4 (&areg)[NR]) {
    const int64_t col = a_col(kb);
#pragma unroll
    for (int r = 0; r < NR; ++r) areg[r] = *reinterpret_cast<const u32x4*>(ap[r] + col);
  };
  auto store_a = [&](int buf, int64_t kb, const u32x4 (&areg)[NR]) {
    bool live = true;
    if (KT && AMODE != A_REPEAT) live = kb * 64 + seg8 * 8 < K;  // zero past the K tail
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int row = (tid >> 3) + 32 * r;
      u32x4 v = areg[r];
      if (KT && AMODE != A_REPEAT && !live) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&As[buf][row][seg8 * 8]) = v;
    }
  };

  u32x4 breg[D][2][4];
  auto load_b = [&](int64_t kb, u32x4 (&b)[2][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int64_t off = kb * 64 + s * 8;
      if (KT) off = min(off, K - 8 - kq);  // stay inside the row; A is zero there
      b[0][s] = *reinterpret_cast<const u32x4*>(bp0 + off);
      b[1][s] = *reinterpret_cast<const u32x4*>(bp1 + off);
    }
  };

  f32x16 acc[NR][2];
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][c][r] = 0.0f;
    }
  }

  auto compute = [&](int buf, const u32x4 (&b)[2][4]) {
    // all of the block's activation fragments first, then the MFMAs
    bf16x8 af[4][NR];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        af[s][rb] = *reinterpret_cast<const bf16x8*>(
            &As[buf][rb * 32 + (lane & 31)][(lane >> 5) * 32 + s * 8]);
      }
    }
    // keep the scheduler from sinking each read next to its MFMA (which would
    // expose the LDS latency once per MFMA pair)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, b[0][s]);
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, b[1][s]);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][rb], b0, acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][rb], b1, acc[rb][1], 0, 0, 0);
      }
    }
  };

  // ---- prologue
  u32x4 areg[2][NR];
  load_a(0, areg[0]);
#pragma unroll
  for (int q = 0; q < D; ++q) {
    if (q < nkb) load_b(q, breg[q]);
  }
  if (nkb > 1) load_a(1, areg[1]);
  store_a(0, 0, areg[0]);
  __syncthreads();

  // ---- steady state: every sub-iteration has kb + D < nkb (so kb + 2 < nkb too)
  int64_t kb0 = 0;
  for (; kb0 + (U - 1) + D < nkb; kb0 += U) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int64_t kb = kb0 + q;
      load_a(kb + 2, areg[q % 2]);
      compute(q % 2, breg[q % D]);
      load_b(kb + D, breg[q % D]);
      store_a((q + 1) % 2, kb + 1, areg[(q + 1) % 2]);
      __syncthreads();
    }
  }
  // ---- drain: fewer than U + D blocks remain
#pragma unroll
  for (int q = 0; q < U + D; ++q) {
    const int64_t kb = kb0 + q;
    if (kb < nkb) {
      if (kb + 2 < nkb) load_a(kb + 2, areg[q % 2]);
      compute(q % 2, breg[q % D]);
      if (kb + D < nkb) load_b(kb + D, breg[q % D]);
      if (kb + 1 < nkb) store_a((q + 1) % 2, kb + 1, areg[(q + 1) % 2]);
      __syncthreads();
    }
  }

  // ---- epilogue: through LDS as fp32, 16-byte row-contiguous stores.
  // MFMA layout: lane holds column lane&31, rows 8*(r/4) + 4*(lane/32) + r%4.
  float(*S)[32][kLdsOut] = reinterpret_cast<float(*)[32][kLdsOut]>(smem);
#pragma unroll
  for (int rb = 0; rb < NR; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      S[wave][row][lane & 31] = acc[rb][0][r];
      S[wave][row][32 + (lane & 31)] = acc[rb][1][r];
    }
    __syncthreads();
    if (EPI == EPI_GATE_UP) {
      // wave tile: 32 rows x 32 h-columns = 128 chunks of 8
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i;
        const int row = c >> 2, cc = c & 3;
        const int tr = rb * 32 + row;
        const int64_t col = cb0 + cc * 8;
        if (tr < t.rows && col < a.n_cols) {
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8]);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8 + 4]);
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(&S[wave][row][32 + cc * 8]);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(&S[wave][row][32 + cc * 8 + 4]);
          u32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float h0 = gemm::act_pair(a.act, e < 2 ? g0[2 * e] : g1[2 * e - 4],
                                            e < 2 ? u0[2 * e] : u1[2 * e - 4], a.beta, a.lbeta);
            const float h1 = gemm::act_pair(a.act, e < 2 ? g0[2 * e + 1] : g1[2 * e - 3],
                                            e < 2 ? u0[2 * e + 1] : u1[2 * e - 3], a.beta,
                                            a.lbeta);
            o[e] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
          }
          *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.C) + (t.row0 + tr) * a.ldc + col) = o;
        }
      }
    } else {
      // wave tile: 32 rows x 64 columns = 256 chunks of 8
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lane + 64 * i;
        const int row = c >> 3, cc = c & 7;
        const int tr = rb * 32 + row;
        const int64_t col = cb0 + cc * 8;
        if (tr < t.rows && col < a.n_cols) {
          const int64_t orow = t.row0 + tr;
          f32x4 v0 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8]);
          f32x4 v1 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8 + 4]);
          if (EPI == EPI_STORE_F32) {
            // router logits: any expert count, so scalar stores up to n_cols
            float* dst = static_cast<float*>(a.C) + orow * a.ldc + col;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (col + e < a.n_cols) dst[e] = e < 4 ? v0[e] : v1[e - 4];
            }
          } else {
            if (EPI == EPI_STORE_RES) {
              const u32x4 rq = *reinterpret_cast<const u32x4*>(
                  static_cast<const bf16_t*>(a.residual) + orow * a.ld_res + col);
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                v0[2 * e] += __uint_as_float(rq[e] << 16);
                v0[2 * e + 1] += __uint_as_float(rq[e] & 0xFFFF0000u);
                v1[2 * e] += __uint_as_float(rq[2 + e] << 16);
                v1[2 * e + 1] += __uint_as_float(rq[2 + e] & 0xFFFF0000u);
              }
            }
            u32x4 o;
            o[0] = (uint32_t)f32_to_bf16(v0[0]) | ((uint32_t)f32_to_bf16(v0[1]) << 16);
            o[1] = (uint32_t)f32_to_bf16(v0[2]) | ((uint32_t)f32_to_bf16(v0[3]) << 16);
            o[2] = (uint32_t)f32_to_bf16(v1[0]) | ((uint32_t)f32_to_bf16(v1[1]) << 16);
            o[3] = (uint32_t)f32_to_bf16(v1[2]) | ((uint32_t)f32_to_bf16(v1[3]) << 16);
            *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.C) + orow * a.ldc + col) = o;
          }
        }
      }
    }
    __syncthreads();
  }
}

// RB = 4 tiles hold 128 accumulators per lane: one wave per SIMD, all registers.
template <int RB, int EPI, int AMODE, int D, bool KT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, RB >= 4 ? 1 : 2)))
void moe_gemm_bf16(GemmArgs a, int64_t n_tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<RB>::kBytes];
  TileLoc t;
  if (!gemm::locate<RB * 32>(a, gemm::remap_xcd(blockIdx.x, gridDim.x), n_tiles_n, t)) return;
  const int nrb = (t.rows + 31) >> 5;
  if (nrb <= 1) {
    gemm_tile<1, RB, EPI, AMODE, D, KT>(a, t, smem);
  } else if (nrb == 2) {
    if constexpr (RB >= 2) gemm_tile<2, RB, EPI, AMODE, D, KT>(a, t, smem);
  } else if (nrb == 3) {
    if constexpr (RB >= 3) gemm_tile<3, RB, EPI, AMODE, D, KT>(a, t, smem);
  } else {
    if constexpr (RB >= 4) gemm_tile<4, RB, EPI, AMODE, D, KT>(a, t, smem);
  }
}

template <int RB, int EPI, int AMODE, bool KT>
hipError_t launch_rb(const GemmArgs& a, int64_t mt_cap, hipStream_t s) {
  constexpr int D = (RB >= 4) ? 3 : 4;
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;
  const int64_t n_tiles_n = (a.n_cols + kWaves * CPW - 1) / (kWaves * CPW);
  const int64_t mt = a.seg_off ? mt_cap : (a.dense_rows + RB * 32 - 1) / (RB * 32);
  const int64_t grid = gemm::round8(mt * n_tiles_n);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_bf16<RB, EPI, AMODE, D, KT><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a, n_tiles_n);
  return hipGetLastError();
}

template <int EPI, int AMODE>
hipError_t launch_any(const GemmArgs& a, int rb, int64_t mt_cap, hipStream_t s) {
  const bool kt = (a.K % 64) != 0 && AMODE != A_REPEAT;
  if (kt) {
    if constexpr (AMODE != A_REPEAT) {
      switch (rb) {
        case 1: return launch_rb<1, EPI, AMODE, true>(a, mt_cap, s);
        case 2: return launch_rb<2, EPI, AMODE, true>(a, mt_cap, s);
        case 4: return launch_rb<4, EPI, AMODE, true>(a, mt_cap, s);
        default: return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (rb) {
    case 1: return launch_rb<1, EPI, AMODE, false>(a, mt_cap, s);
    case 2: return launch_rb<2, EPI, AMODE, false>(a, mt_cap, s);
    case 4: return launch_rb<4, EPI, AMODE, false>(a, mt_cap, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int epi, int amode, int rb, int64_t mt_cap,
                            hipStream_t s) {
  if (epi == EPI_GATE_UP && amode == A_DIRECT) return launch_any<EPI_GATE_UP, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_GATE_UP && amode == A_GATHER) return launch_any<EPI_GATE_UP, A_GATHER>(a, rb, mt_cap, s);
  if (epi == EPI_STORE && amode == A_DIRECT) return launch_any<EPI_STORE, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_STORE_RES && amode == A_DIRECT) return launch_any<EPI_STORE_RES, A_DIRECT>(a, rb, mt_cap, s);
  if (epi == EPI_STORE_F32 && amode == A_REPEAT) return launch_any<EPI_STORE_F32, A_REPEAT>(a, rb, mt_cap, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
