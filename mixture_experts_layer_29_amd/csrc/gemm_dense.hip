// gemm_dense.hip - the block's dense products on MFMA: the shared expert
// (gate/up with the activation, and down) and the latent down and up
// projections (the Kimi K3 "Add shared output" page, moe-forward excerpt).
//
// C[row, col] = sum_k A[row, k] * W[col, k]: activations A [M, K] row-major,
// weights W [cols, K] in nn.Linear layout.  At prefill sizes (M = 4096-8192
// tokens, K = 2048-7168) every weight tile feeds all M rows, so these products
// are bound by the matrix cores, not by HBM, and the kernel is built to keep
// the MFMAs busy:
//  - a work-group computes a 256 x 256 tile (256 rows by 256 weight rows; for
//    gate/up the weight rows are 128 gate and 128 up rows of the same 128
//    output columns, interleaved in blocks of 32) on 8 waves, two per SIMD;
//    a wave owns 128 rows x 64 weight rows: 4 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16, 8 MFMAs per 16-deep step;
//  - both operands are copied HBM/L2 -> LDS by the load units
//    (global_load_lds_dwordx4) in 32-deep K blocks: 64-byte rows whose
//    16-byte chunks are XOR-swizzled by bits 2..3 of the row, so each 16-lane
//    group of a fragment read touches distinct banks.  Five 32 KB stages fill
//    the 160 KB of LDS, the copies running three blocks (~3000 MFMA cycles)
//    ahead of their use, which covers the latency of L2 misses under load;
//  - one barrier per K block, placed between its two steps and pipelined
//    across: before it a wave reads the fragments of step 1 while the MFMAs
//    of step 0 run; the barrier makes the next block visible (every wave has
//    waited for its own copies of it) and frees the oldest stage for the
//    next copy; after it the wave reads the next block's step-0 fragments
//    while the MFMAs of step 1 run.  So no fragment read waits in the open
//    after a barrier, and the MFMAs stop only for the barrier itself;
//  - the MFMA takes the weight fragment as its first operand, so each lane
//    ends with four consecutive output columns of one row and the epilogue
//    (activation, fp32 output, or fp32 residual add, one rounding) stores
//    straight from registers;
//  - tiles are numbered in bands of four row blocks that run across the
//    weight blocks, and XCD x takes the x-th contiguous range of that order,
//    so the 32 work-groups an XCD runs at once cover about four row blocks
//    by eight weight blocks and share their operands in its L2.
#include "gemm_common.h"
#include "gemm_lds.h"
#include "gemm_plan.h"

namespace moe {
namespace {

using namespace lds;

constexpr int kBM = 256;                        // rows per tile
constexpr int kBN = 256;                        // weight rows per tile
constexpr int kBK = 32;                         // K per block
constexpr int kRow = kBK * 2;                   // 64 bytes of a row per block
constexpr int kHalf = kBM * kRow;               // 16 KB: the A (or B) part of a stage
constexpr int kStage = 2 * kHalf;               // 32 KB
constexpr int kStages = 5;                      // 160 KB of LDS
constexpr int kLoads = 2 * kBM / 16;            // 16-row copies per stage (A then B): 32
constexpr int kWaves = 8;
constexpr int kLoadsPerWave = kLoads / kWaves;  // 4
// At the barrier of block kb a wave needs its copies of block kb + 1; the
// copies of blocks kb + 2 .. kb + kStages - 2 may still be in flight.
constexpr int kWait = kLoadsPerWave * (kStages - 3);
constexpr int kBand = 4;                        // row blocks per band of the tile order

// Byte offset of 16-byte chunk c (0..3) of row r in a stage half.
__device__ __forceinline__ int swz64(int r, int c) { return r * kRow + ((c ^ ((r >> 2) & 3)) << 4); }

template <int EPI>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moe_gemm_dense(GemmArgs a, int64_t m_blocks, int64_t n_blocks, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStage];
  constexpr int OUT_COLS = EPI == EPI_GATE_UP ? kBN / 2 : kBN;

  int tid;  // see gemm_bf16.hip: recomputed per-lane indices beat held ones
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // work-group b runs on XCD b % 8: XCD x takes tiles [x per_xcd, (x + 1) per_xcd)
  // of the banded order
  const int64_t b = blockIdx.x, j = b >> 3;
  const int64_t t = (b & 7) * per_xcd + j;
  if (j >= per_xcd || t >= m_blocks * n_blocks) return;
  const int64_t band = t / (kBand * n_blocks), in_band = t - band * (kBand * n_blocks);
  const int64_t band_h = min((int64_t)kBand, m_blocks - band * kBand);
  const int64_t mb = band * kBand + in_band % band_h, nb = in_band / band_h;
  const int64_t row0 = mb * kBM, col0 = nb * OUT_COLS;
  const int64_t M = a.dense_rows, K = a.K, nkb = K / kBK;

  // ---- this lane's 16-byte source of each of the wave's 4 copies per K
  // block: copy q (0..31) fills stage rows 16 (q % 16) + lane / 4 of A
  // (q < 16) or B; lane l writes chunk l % 4 of its row, which holds source
  // chunk (l % 4) ^ ((row >> 2) & 3)
  const bf16_t* src[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int q = wave * kLoadsPerWave + i;
    const int r = 16 * (q & 15) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((r >> 2) & 3);
    if (q < 16) {
      const int64_t row = min(row0 + r, M - 1);
      src[i] = static_cast<const bf16_t*>(a.A) + row * a.lda + chunk * 8;
    } else {
      const bf16_t* w;
      int64_t wrow;
      if (EPI == EPI_GATE_UP) {
        const int blk = r >> 5;
        w = static_cast<const bf16_t*>((blk & 1) ? a.B1 : a.B0);
        wrow = col0 + (blk >> 1) * 32 + (r & 31);
      } else {
        w = static_cast<const bf16_t*>(a.B0);
        wrow = col0 + r;
      }
      wrow = min(wrow, a.n_cols - 1);
      src[i] = w + wrow * K + chunk * 8;
    }
  }
  // block kb into its stage; blocks past the end fetch the last one again
  // (into a stage that nobody reads afterwards), so every block issues the
  // same copies and the wait count is one constant
  auto issue = [&](int64_t kb, int stage) {
    kb = kb < nkb ? kb : nkb - 1;
    uint8_t* const base = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int q = wave * kLoadsPerWave + i;
      dma16<false>(src[i] + kb * kBK, base + (q < 16 ? 0 : kHalf) + (q & 15) * 1024);
    }
  };

  // ---- wave tile: rows 128 wm .. +127 (row blocks 4 wm .. 4 wm + 3), weight
  // rows 64 wn .. +63 (blocks 2 wn, 2 wn + 1)
  const int wm = wave >> 2, wn = wave & 3;
  const int rsel = lane & 31, cbase = (lane >> 5) * 4;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.0f;
    }
  }
  // fragments of step s (0, 1) of a block, in register set s: lane half h
  // reads chunk 2 h + s
  bf16x8 af[2][4], bf[2][2];
  auto read_frags = [&](int stage, int s) {
    const uint8_t* st = smem + stage * kStage;
    const int c = 2 * (lane >> 5) + s;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      bf[s][jj] = *reinterpret_cast<const bf16x8*>(st + kHalf + swz64((2 * wn + jj) * 32 + rsel, c));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[s][i] = *reinterpret_cast<const bf16x8*>(st + swz64((4 * wm + i) * 32 + rsel, c));
  };
  // the 8 MFMAs of register set s, interleaved with the 6 fragment reads
  // issued just before (MFMA, read, MFMA, read, ...)
  auto mfmas = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s][jj], af[s][i], acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: blocks 0 .. kStages - 2 in flight; block 0 landed
  // everywhere; its step-0 fragments in registers
#pragma unroll
  for (int q = 0; q < kStages - 1; ++q) issue(q, q);
  wait_vm<kLoadsPerWave * (kStages - 2)>();
  wg_barrier();
  read_frags(0, 0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- main loop.  Block kb sits in stage kb % kStages.  Its barrier comes
  // after the step-1 reads and step-0 MFMAs: every wave's copies of block
  // kb + 1 have landed by then (kWait of the wave's younger copies may stay in
  // flight), and every wave is done with block kb - 1, whose stage then takes
  // block kb + kStages - 1.
  int stage = 0;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int next = stage + 1 == kStages ? 0 : stage + 1;
    const int prev = stage == 0 ? kStages - 1 : stage - 1;
    read_frags(stage, 1);
    mfmas(0);
    wait_vm<kWait>();
    wg_barrier();
    issue(kb + kStages - 1, prev);
    // (after the last block this reads a stage nobody uses: unconditional, so
    // the compiler's LDS wait counts see one straight-line order)
    read_frags(next, 0);
    mfmas(1);
    stage = next;
  }
  wait_vm<0>();  // no copy may land in the LDS of the next work-group

  // ---- epilogue from registers: lane l holds row 32 i + l % 32 of its row
  // blocks and, per accumulator, weight rows 8 g + 4 (l / 32) + 0..3 of its
  // 32-row weight block (g = 0..3)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t orow = row0 + (4 * wm + i) * 32 + rsel;
    if (orow >= M) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (EPI == EPI_GATE_UP) {
        const int64_t col = col0 + 32 * wn + 8 * g + cbase;
        if (col >= a.n_cols) continue;
        uint32_t o[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float h0 = gemm::act_pair(a.act, acc[i][0][4 * g + 2 * e], acc[i][1][4 * g + 2 * e],
                                          a.beta, a.lbeta);
          const float h1 = gemm::act_pair(a.act, acc[i][0][4 * g + 2 * e + 1],
                                          acc[i][1][4 * g + 2 * e + 1], a.beta, a.lbeta);
          o[e] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
        }
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.C) + orow * a.ldc + col) =
            make_uint2(o[0], o[1]);
      } else {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int64_t col = col0 + 64 * wn + 32 * jj + 8 * g + cbase;
          if (col >= a.n_cols) continue;
          f32x4 v = {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                     acc[i][jj][4 * g + 3]};
          if (EPI == EPI_STORE_RES)
            v += *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.residual) +
                                                 orow * a.ld_res + col);
          if (EPI == EPI_STORE_F32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.C) + orow * a.ldc + col) = v;
          } else {
            const uint32_t o0 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            const uint32_t o1 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(a.C) + orow * a.ldc + col) =
                make_uint2(o0, o1);
          }
        }
      }
    }
  }
}

template <int EPI>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  constexpr int OUT_COLS = EPI == EPI_GATE_UP ? kBN / 2 : kBN;
  const int64_t mbs = (a.dense_rows + kBM - 1) / kBM;
  const int64_t nbs = (a.n_cols + OUT_COLS - 1) / OUT_COLS;
  const int64_t per_xcd = (mbs * nbs + 7) / 8;
  const int64_t grid = 8 * per_xcd;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_dense<EPI><<<dim3((unsigned)grid), dim3(64 * kWaves), 0, s>>>(a, mbs, nbs, per_xcd);
  return hipGetLastError();
}

}  // namespace

bool gemm_dense_supported(const GemmArgs& a, int epi) {
  if (epi != EPI_GATE_UP && epi != EPI_STORE && epi != EPI_STORE_F32 && epi != EPI_STORE_RES)
    return false;
  // whole 32-deep K blocks; 16-byte rows for the copies and 4-column stores
  return a.K % kBK == 0 && a.K > 0 && a.lda % 8 == 0 && a.ldc % 4 == 0 && a.n_cols % 4 == 0 &&
         (epi != EPI_STORE_RES || a.ld_res % 4 == 0);
}

hipError_t launch_gemm_dense(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_GATE_UP: return launch<EPI_GATE_UP>(a, s);
    case EPI_STORE: return launch<EPI_STORE>(a, s);
    case EPI_STORE_F32: return launch<EPI_STORE_F32>(a, s);
    case EPI_STORE_RES: return launch<EPI_STORE_RES>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
