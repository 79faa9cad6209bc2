// gemm_bf16.hip - bf16 MFMA GEMM for the routed experts (grouped over the
// expert-sorted row segments) and for the dense products of the block (shared
// expert, latent projections, router).
//
// Every product is C[row, col] = sum_k A[row, k] * W[col, k]: activations A
// row-major, weights W in nn.Linear layout [cols, K] (the expert excerpt of the
// Kimi K3 "Gate features" page: w1, w3 [d_ff, d_in], w2 [d_in, d_ff], no bias).
//
// Design for CDNA4.  At the MoE sizes of interest the expert weights set the
// time, and each weight byte feeds only the T_e rows routed to its expert, so
// the kernel is built to stream every expert's weights once at close to full
// HBM bandwidth with the MFMAs for its rows running underneath:
//  - a work-group owns one (segment, n-tile, m-tile); tiles are up to RB x 32
//    rows high so that a whole expert segment usually fits one tile (every
//    extra m-tile of an expert would stream its weights again);
//  - four column pairs per tile, each of two 32-column blocks of the output
//    (the gate and the up block of the same columns for the gate/up product);
//    with 4 waves a wave owns a pair, with 8 (two per SIMD) the two waves of a
//    pair split its row blocks;
//  - both operands are copied from HBM straight into LDS by the load units
//    (global_load_lds_dwordx4: 16 bytes per lane, 8 lanes per 128-byte piece
//    of a row, no registers held while in flight).  The weights stream as
//    sub-blocks of one 32-column block x 64 k per pair (16 KB per work-group),
//    SB-1 sub-blocks ahead in an SB-stage ring; the activations of a 64-k block
//    serve its two column sub-blocks and are loaded NA-1 blocks ahead in NA
//    stages (the ring plan depends on the tile's row blocks).  Each visit of a
//    weight row reads a whole 128-byte piece (shorter pieces cost DRAM
//    efficiency);
//  - waits are explicit vmcnt counts followed by a plain work-group barrier, so
//    loads for later sub-blocks stay in flight.  Every sub-iteration issues the
//    same loads (past either end of K the last block is fetched again into a
//    stage nobody reads), so the counts are compile-time constants, derived
//    from the issue order;
//  - LDS tiles are unpadded 128-byte rows whose 16-byte chunks are
//    XOR-swizzled by bits 1..3 of the row (each lane fetches the chunk that
//    belongs at its fixed LDS slot): the MFMA-layout reads touch all 64 banks
//    once per 16 lanes;
//  - fragments are read in the operand layout of v_mfma_f32_32x32x16_bf16, the
//    reads for the next MFMA step interleaved with the current step's MFMAs;
//    the number of 32-row blocks that hold rows is a template parameter, so a
//    tile with few rows issues only the MFMAs (and activation loads) it needs;
//  - in gather mode activation rows are read through the dispatch
//    permutation, so no expert-sorted copy of the input is ever written;
//  - tiles are numbered segment-major, then n-tile, then m-tile; the experts
//    are split into 8 runs of about equal cost, one per XCD, so the n-tiles
//    of an expert share its activation rows in one L2;
//  - a tile's fixed work (table lookups, ring ramp, epilogue) is up to an
//    eighth of it: 4-wave tiles of up to 4 row blocks plan their rings in
//    half the LDS and run two work-groups per CU, so that one streams while
//    the other starts or ends a tile; taller tiles keep the whole CU;
//  - the epilogue stages the fp32 accumulators through LDS, applies
//    SiLU/SiTU-and-mul or the residual add in fp32, rounds once and writes
//    16-byte row-contiguous chunks (for the down product of the block, to the
//    rows' token slots).  The bf16 outputs are stored non-temporal: output
//    lines left to age in L2 slow the weight stream of the tiles still
//    running (paired in one process, K3 latent prefill 11.37 -> 11.11 ms per
//    block, gate/up -3.4%, DeepSeek-V3 prefill -2.8%); the fp32 outputs (router
//    logits, read at once by the selection) keep the default policy.
// Inside a 64-wide K block the lanes visit K in an order of our choosing, the
// same for both operands (lane half h takes elements 32h .. 32h+31, eight per
// MFMA step).
#include <type_traits>

#include "gemm_common.h"
#include "gemm_lds.h"
#include "gemm_plan.h"

namespace moe {
namespace {

using gemm::TileLoc;
using namespace lds;

using namespace plan;
constexpr int kLdsOut = 72;                         // fp32 per LDS epilogue row: 64 + 8 pad

// Waves per work-group, W: 4 (one per column pair and SIMD), or, for tiles of
// 4 or more row blocks, 8 (two per column pair and SIMD, splitting the row
// blocks), so that one wave's LDS reads run while the other's MFMAs do: a
// single wave cannot feed its MFMAs from LDS (~1 KB per 34 cycles per wave on
// gfx950).  Eight waves pay off when the tiles are mostly full.
//
// LDS of an RB-block kernel: the largest plan of its tiles, or the epilogue.
template <int RB, int W = 4, int LDS = kLdsMax>
struct Smem {
  template <int NR>
  static constexpr int ring_max() {
    if constexpr (NR == 0) {
      return 0;
    } else {
      constexpr int b = Ring<NR, LDS>::kBytes, r = ring_max<NR - 1>();
      return b > r ? b : r;
    }
  }
  static constexpr int kEpi = W * 32 * kLdsOut * 4;
  static constexpr int kBytes = ring_max<RB>() > kEpi ? ring_max<RB>() : kEpi;
  static_assert(kBytes <= LDS, "LDS plan exceeds the budget");
};

// NR: 32-row blocks holding rows.  The weight ring has SB = Smem<RB>::kSB
// stages of one column sub-block each.  W waves; this wave serves column pair
// cw and, of the tile's NR row blocks, the NRH starting at block rb0 (all of
// them when W = 4; with W = 8 the waves h = 0 and h = 1 of a pair take the
// first ceil(NR/2) and the last floor(NR/2)).  It also loads NRH of the
// tile's 4 NR activation loads (8 rows each) and 4 * 4 / (W / 4) of its
// column pair's weight loads per sub-block.
template <int NR, int NRH, int W, int RB, int EPI, int AMODE, bool KT, int LDS>
__device__ __forceinline__ void gemm_body(const GemmArgs& a, const TileLoc& t, uint8_t* smem,
                                          const int cw, const int h) {
  constexpr int SB = Ring<NR, LDS>::kNB;   // weight stages
  constexpr int NA = Ring<NR, LDS>::kNA;   // activation stages
  constexpr int kBL = W == 8 ? 2 : 4;      // weight loads per wave per sub-block
  constexpr int NRA = NRH > 0 ? NRH : 1;   // array extents
  constexpr int C0 = W == 8 ? (NR + 1) / 2 : NR;  // row blocks of the h = 0 wave
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;  // output columns per wave
  constexpr int ATILE = Ring<NR, LDS>::kATile;
  uint8_t* const As = smem;                            // [NA][NR*32 rows][128 B]
  uint8_t* const Bs = smem + NA * ATILE;               // [SB][pair][32 rows][128 B]

  // The thread id passes through an opaque move at the start of every tile, so
  // the per-lane row and chunk indices below are recomputed per tile (a few ALU
  // ops) rather than hoisted out of the tile loop for every tile height of the
  // switch and held in registers across it (which made the 8-wave forms spill).
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rb0 = h ? C0 : 0;                          // first row block of this wave
  const int a_base = h ? kPairs * C0 + cw * NRH : cw * NRH;  // first activation load
  const int64_t K = a.K;                // row length of both operands
  const int64_t kbase = t.kb0;          // the tile's K range: blocks kbase .. kbase+nkb-1
  const int64_t nkb = t.kb1 - t.kb0;
  const int slot = lane & 7;  // LDS chunk slot this lane's load lands in

  // ---- weights: sub-block (kb, c) holds the 32 rows of column block c of the
  // pair (c = 0: columns cb0.., c = 1: columns cb1..); load ib fills rows
  // 8 ib .. 8 ib + 7, this wave issuing loads ib = b_base .. b_base + kBL - 1
  const int b_base = W == 8 ? 2 * h : 0;
  const int64_t cb0 = t.j * (kPairs * CPW) + (int64_t)cw * CPW;
  const int64_t cb1 = (EPI == EPI_GATE_UP) ? cb0 : cb0 + 32;
  const bf16_t* W0 = static_cast<const bf16_t*>(a.B0) + t.seg * a.b_seg_stride;
  const bf16_t* W1 =
      static_cast<const bf16_t*>(EPI == EPI_GATE_UP ? a.B1 : a.B0) + t.seg * a.b_seg_stride;
  const bf16_t* brow[2][kBL];  // this lane's source (row, chunk) per column block and load
  int bchunk[kBL];
#pragma unroll
  for (int i = 0; i < kBL; ++i) {
    const int r = 8 * (b_base + i) + (lane >> 3);
    bchunk[i] = slot ^ ((r >> 1) & 7);
    // columns past the end reload the last column (their outputs are dropped)
    const int64_t c0 = min(cb0 + r, a.n_cols - 1);
    const int64_t c1 = min(cb1 + r, a.n_cols - 1);
    brow[0][i] = W0 + c0 * K + bchunk[i] * 8;
    brow[1][i] = W1 + c1 * K + bchunk[i] * 8;
  }

  // ---- activations: this wave's load i fills tile rows 8(a_base + i) .. +7
  const bf16_t* ap[NRA];
  int achunk[NRA];
#pragma unroll
  for (int i = 0; i < NRH; ++i) {
    const int row = 8 * (a_base + i) + (lane >> 3);
    achunk[i] = slot ^ ((row >> 1) & 7);
    int64_t src = t.row0 + (row < t.rows ? row : 0);
    if (AMODE == A_GATHER) src = a.a_map[src] / a.a_div;
    src = src < 0 ? 0 : (src >= a.a_rows ? a.a_rows - 1 : src);
    ap[i] = static_cast<const bf16_t*>(a.A) + src * a.lda + achunk[i] * 8;
  }
  const int64_t a_per_blocks = AMODE == A_REPEAT ? (a.a_period >> 6) : 1;

  // block indices (relative to kbase) are clamped to [0, nkb): a load past
  // either end fetches a real block again, into a stage that nobody reads
  // before it is refilled
  auto issue_a = [&](int64_t kb, int stage) {
    kb = kbase + (kb < 0 ? 0 : (kb >= nkb ? nkb - 1 : kb));
    const int64_t col = (AMODE == A_REPEAT ? (kb % a_per_blocks) : kb) * 64;
    uint8_t* const dst = As + stage * ATILE + a_base * 1024;
#pragma unroll
    for (int i = 0; i < NRH; ++i) {
      int64_t c = col;
      // past the valid width: A_REPEAT meets zero weights, the K tail is zeroed
      // in LDS after the copy; either way the address stays inside the row
      if (AMODE == A_REPEAT) c = min(c, a.a_valid - 8 - achunk[i] * 8);
      else if (KT) c = min(c, K - 8 - achunk[i] * 8);
      dma16<false>(ap[i] + c, dst + i * 1024);
    }
  };
  // Weights that no other tile reads (a segment of one m-tile, or every
  // weight of the launch) are loaded non-temporal: they stream from HBM
  // without taking L2 (and last-level cache) space from the reused
  // activation rows, which measures ~13% faster on MI355X.  An expert spread
  // over several m-tiles keeps cached loads, so its m-tiles, which run side by
  // side, share its weights in L2.
  const bool nt = a.b_stream == 1 || (a.b_stream == 2 && t.mt == 1);
  auto issue_b = [&](int64_t kb, int cblk, int stage) {
    kb = kbase + (kb < 0 ? 0 : (kb >= nkb ? nkb - 1 : kb));
    uint8_t* const dst = Bs + stage * kBStage + cw * kBPair + b_base * 1024;
    if (nt) {
#pragma unroll
      for (int i = 0; i < kBL; ++i) {
        int64_t off = kb * 64;
        if (KT) off = min(off, K - 8 - bchunk[i] * 8);  // A is zero there
        dma16<true>(brow[cblk][i] + off, dst + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBL; ++i) {
        int64_t off = kb * 64;
        if (KT) off = min(off, K - 8 - bchunk[i] * 8);
        dma16<false>(brow[cblk][i] + off, dst + i * 1024);
      }
    }
  };
  // K tail: zero this lane's activation chunks of the last block that lie past K
  auto zero_a_tail = [&](int64_t kb, int stage) {
    uint8_t* const dst = As + stage * ATILE + a_base * 1024;
#pragma unroll
    for (int i = 0; i < NRH; ++i) {
      if ((kbase + kb) * 64 + achunk[i] * 8 >= K)
        *reinterpret_cast<u32x4*>(dst + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    wait_lgkm0();
  };

  f32x16 acc[NRA][2];
#pragma unroll
  for (int rb = 0; rb < NRA; ++rb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][c][r] = 0.0f;
    }
  }

  // One column sub-block from LDS: 4 MFMA steps; in step s lane half h reads
  // chunk 4h + s of its rows.  The activation fragments of a K block are read
  // from LDS once, in its first sub-block, and kept in registers for the
  // second (LDS bandwidth is shared with the load units' writes).  Step s+1's
  // fragments are read between step s's MFMAs (a wave issues an MFMA only
  // every few dozen cycles).
  const int rsel = lane & 31;
  const int cbase = (lane >> 5) * 4;
  // The activation fragments of a K block stay in registers for its second
  // sub-block while they fit next to the accumulators (up to 6 row blocks
  // with W = 4, 3 with W = 8, which has half the registers, and 2 with W = 4
  // at two work-groups per CU, which also has half); beyond that they are
  // read again.
  constexpr bool kKeepA = NRH <= (W == 4 ? (LDS == kLdsMax ? 6 : 2) : 3);
  bf16x8 afk[kKeepA ? 4 : 2][NRA];  // activation fragments (all steps, or two)
  auto compute0 = [&](auto col_tag, const uint8_t* at, const uint8_t* bt) {
    constexpr int COL = decltype(col_tag)::value;
    bf16x8 bf[2];
    // weights first: MFMA rb then waits only for the reads up to A row block rb
    auto read_frags = [&](int s, bf16x8& fb) {
      const int c = cbase + s;
      fb = *reinterpret_cast<const bf16x8*>(bt + swz(rsel, c));
#pragma unroll
      for (int rb = 0; rb < NRH; ++rb) {
        afk[kKeepA ? s : (s & 1)][rb] =
            *reinterpret_cast<const bf16x8*>(at + swz((rb0 + rb) * 32 + rsel, c));
      }
    };
    read_frags(0, bf[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read_frags(s + 1, bf[(s + 1) & 1]);
#pragma unroll
      for (int rb = 0; rb < NRH; ++rb) {
        acc[rb][COL] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afk[kKeepA ? s : (s & 1)][rb],
                                                               bf[s & 1], acc[rb][COL], 0, 0, 0);
      }
      if (s < 3) {
        // MFMA, read, MFMA, read, ...: the reads hide under the MFMAs
#pragma unroll
        for (int i = 0; i < NRH; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute1 = [&](const uint8_t* at, const uint8_t* bt) {
    if constexpr (!kKeepA) {
      compute0(std::integral_constant<int, 1>{}, at, bt);
    } else {
      bf16x8 bf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bf[s] = *reinterpret_cast<const bf16x8*>(bt + swz(rsel, cbase + s));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int rb = 0; rb < NRH; ++rb) {
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afk[s][rb], bf[s], acc[rb][1], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline over sub-iterations u = 2 kb + c.  Sub-iteration u reads
  // weight stage u % SB and activation stage kb % NA; it issues sub-block
  // u + SB - 1 into stage (u - 1) % SB and, for even u, A(kb + NA - 1) into
  // stage (kb - 1) % NA.  The activation tile is shared by all waves, so the
  // barrier of even u comes before its activation issue (every wave's part of
  // A(kb) has landed, and every wave is done with A(kb - 1), whose second
  // sub-block ended at u - 1).  With W = 4 a wave alone reads its pair's slice
  // of a weight stage, so it issues its weights before the wait and needs no
  // barrier at odd u (its own reads of sub-block u - 1 are done); with W = 8
  // two waves share a slice, and every sub-iteration runs wait, barrier,
  // issue.  The same issues happen for the sub-iterations before 0 (the
  // prologue): blocks below 0 fetch block 0 again into stages that are
  // refilled before anyone reads them, as blocks past the end fetch the last
  // block into stages nobody reads.
  constexpr int kWaitEven = wait_count<W, NA, SB, NRH, kBL>(true);
  constexpr int kWaitOdd = wait_count<W, NA, SB, NRH, kBL>(false);
  static_assert(kWaitEven < 64 && kWaitOdd < 64, "vmcnt range");
  constexpr int kLead = (SB - 1) > 2 * (NA - 1) ? (SB - 1) : 2 * (NA - 1);
  auto mod = [](int v, int m) { return ((v % m) + m) % m; };
#pragma unroll
  for (int q = -kLead; q < 0; ++q) {
    const int ub = q + SB - 1;  // sub-block issued at sub-iteration q
    if constexpr (W == 8) {
      if ((q & 1) == 0) issue_a(q / 2 + NA - 1, mod(q / 2 + NA - 1, NA));
      issue_b(ub >> 1, ub & 1, mod(ub, SB));
    } else {
      issue_b(ub >> 1, ub & 1, mod(ub, SB));
      if ((q & 1) == 0) issue_a(q / 2 + NA - 1, mod(q / 2 + NA - 1, NA));
    }
  }

  int sb = 0;  // weight stage of the sub-block being consumed
  int sa = 0;  // activation stage of K block kb
  const uint8_t* const bt0 = Bs + cw * kBPair;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int sb_prev = sb == 0 ? SB - 1 : sb - 1;
    const int sa_prev = sa == 0 ? NA - 1 : sa - 1;
    if constexpr (W == 4) {
      // c = 0
      issue_b((2 * kb + SB - 1) >> 1, (SB - 1) & 1, sb_prev);
      wait_vm<kWaitEven>();
      if (KT && AMODE != A_REPEAT && kb == nkb - 1) zero_a_tail(kb, sa);
      wg_barrier();
      issue_a(kb + NA - 1, sa_prev);
      compute0(std::integral_constant<int, 0>{}, As + sa * ATILE, bt0 + sb * kBStage);
      sb = (sb + 1 == SB) ? 0 : sb + 1;
      // c = 1: no barrier (the wave's own weight slice)
      issue_b((2 * kb + SB) >> 1, SB & 1, sb == 0 ? SB - 1 : sb - 1);
      wait_vm<kWaitOdd>();
      compute1(As + sa * ATILE, bt0 + sb * kBStage);
      sb = (sb + 1 == SB) ? 0 : sb + 1;
    } else {
      // c = 0
      wait_vm<kWaitEven>();
      if (KT && AMODE != A_REPEAT && kb == nkb - 1) zero_a_tail(kb, sa);
      wg_barrier();
      issue_a(kb + NA - 1, sa_prev);
      issue_b((2 * kb + SB - 1) >> 1, (SB - 1) & 1, sb_prev);
      compute0(std::integral_constant<int, 0>{}, As + sa * ATILE, bt0 + sb * kBStage);
      sb = (sb + 1 == SB) ? 0 : sb + 1;
      // c = 1
      wait_vm<kWaitOdd>();
      wg_barrier();
      issue_b((2 * kb + SB) >> 1, SB & 1, sb == 0 ? SB - 1 : sb - 1);
      compute1(As + sa * ATILE, bt0 + sb * kBStage);
      sb = (sb + 1 == SB) ? 0 : sb + 1;
    }
    sa = (sa + 1 == NA) ? 0 : sa + 1;
  }
  wait_vm<0>();
  __syncthreads();

  // ---- epilogue: through LDS as fp32 (each wave its own 32 x 72 region, so
  // its writes and reads are ordered by the wave itself), 16-byte
  // row-contiguous stores.
  // MFMA layout: lane holds column lane&31, rows 8*(r/4) + 4*(lane/32) + r%4.
  float(*S)[32][kLdsOut] = reinterpret_cast<float(*)[32][kLdsOut]>(smem);
#pragma unroll
  for (int rb = 0; rb < NRH; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      S[wave][row][lane & 31] = acc[rb][0][r];
      S[wave][row][32 + (lane & 31)] = acc[rb][1][r];
    }
    wait_lgkm0();
    if (EPI == EPI_GATE_UP) {
      // wave tile: 32 rows x 32 h-columns = 128 chunks of 8
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i;
        const int row = c >> 2, cc = c & 3;
        const int tr = (rb0 + rb) * 32 + row;
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
          __builtin_nontemporal_store(
              o, reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.C) + (t.row0 + tr) * a.ldc + col));
        }
      }
    } else {
      // wave tile: 32 rows x 64 columns = 256 chunks of 8
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lane + 64 * i;
        const int row = c >> 3, cc = c & 7;
        const int tr = (rb0 + rb) * 32 + row;
        const int64_t col = cb0 + cc * 8;
        if (tr < t.rows && col < a.n_cols) {
          const int64_t orow = t.row0 + tr;
          f32x4 v0 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8]);
          f32x4 v1 = *reinterpret_cast<const f32x4*>(&S[wave][row][cc * 8 + 4]);
          if (EPI == EPI_STORE_F32) {
            // fp32 output (router logits, the shared expert's output); a
            // split-K range writes its own partial product.  Any column count
            // (the router's is the expert count): scalar stores at a ragged end.
            float* dst = static_cast<float*>(a.C) + t.split * a.c_split_stride + orow * a.ldc + col;
            if (col + 8 <= a.n_cols && ((a.ldc | col) & 3) == 0) {
              *reinterpret_cast<f32x4*>(dst) = v0;
              *reinterpret_cast<f32x4*>(dst + 4) = v1;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                if (col + e < a.n_cols) dst[e] = e < 4 ? v0[e] : v1[e - 4];
              }
            }
          } else {
            if (EPI == EPI_STORE_RES) {
              const float* rp = static_cast<const float*>(a.residual) + orow * a.ld_res + col;
              v0 += *reinterpret_cast<const f32x4*>(rp);
              v1 += *reinterpret_cast<const f32x4*>(rp + 4);
            }
            u32x4 o;
            o[0] = (uint32_t)f32_to_bf16(v0[0]) | ((uint32_t)f32_to_bf16(v0[1]) << 16);
            o[1] = (uint32_t)f32_to_bf16(v0[2]) | ((uint32_t)f32_to_bf16(v0[3]) << 16);
            o[2] = (uint32_t)f32_to_bf16(v1[0]) | ((uint32_t)f32_to_bf16(v1[1]) << 16);
            o[3] = (uint32_t)f32_to_bf16(v1[2]) | ((uint32_t)f32_to_bf16(v1[3]) << 16);
            // slot order: the row goes to its token's slot (un-permuted here,
            // so the combine reads each token's k rows contiguously)
            const int64_t crow = (EPI == EPI_STORE && a.c_map) ? a.c_map[orow] : orow;
            __builtin_nontemporal_store(
                o, reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.C) + crow * a.ldc + col));
          }
        }
      }
    }
    wait_lgkm0();  // this wave's reads of its region done before the next block's writes
  }
  __syncthreads();  // the LDS is free for the next tile
}

template <int NR, int RB, int W, int EPI, int AMODE, bool KT, int LDS = kLdsMax>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const TileLoc& t, uint8_t* smem) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (W == 4) {
    gemm_body<NR, NR, 4, RB, EPI, AMODE, KT, LDS>(a, t, smem, wave, 0);
  } else {
    if (wave < kPairs) gemm_body<NR, (NR + 1) / 2, 8, RB, EPI, AMODE, KT, LDS>(a, t, smem, wave, 0);
    else gemm_body<NR, NR / 2, 8, RB, EPI, AMODE, KT, LDS>(a, t, smem, wave - kPairs, 1);
  }
}


// With the whole LDS (LDS = kLdsMax) one work-group runs per CU: with 4 waves
// each may use a SIMD's whole register file, with 8 waves half of it.  With
// half of it (kLdsHalf, 4-wave tiles of up to 4 row blocks) two work-groups
// share a CU, two waves per SIMD: while one fills its rings at a tile's start
// or drains them into its epilogue, the other streams.
template <int RB, int W, int EPI, int AMODE, bool KT, int LDS>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(
    W / 4 * (LDS == kLdsMax ? 1 : 2), W / 4 * (LDS == kLdsMax ? 1 : 2))))
void moe_gemm_bf16(GemmArgs a, int64_t n_tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<RB, W, LDS>::kBytes];
  int64_t L, end, step;
  gemm::tile_range<RB * 32>(a, blockIdx.x, gridDim.x, n_tiles_n, L, end, step);
  for (; L < end; L += step) {
  TileLoc t;
  if (!gemm::locate<RB * 32>(a, L, n_tiles_n, t)) continue;
  const int nrb = (t.rows + 31) >> 5;
  switch (nrb) {
    case 1: gemm_tile<1, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 2: if constexpr (RB >= 2) gemm_tile<2, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 3: if constexpr (RB >= 3) gemm_tile<3, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 4: if constexpr (RB >= 4) gemm_tile<4, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 5: if constexpr (RB >= 5) gemm_tile<5, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 6: if constexpr (RB >= 6) gemm_tile<6, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    case 7: if constexpr (RB >= 7) gemm_tile<7, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
    default: if constexpr (RB >= 8) gemm_tile<8, RB, W, EPI, AMODE, KT, LDS>(a, t, smem); break;
  }
  }
}

template <int RB, int W, int EPI, int AMODE, bool KT, int LDS = kLdsMax>
hipError_t launch_rb(const GemmArgs& a, int64_t mt_cap, hipStream_t s) {
  constexpr int CPW = (EPI == EPI_GATE_UP) ? 32 : 64;
  const int64_t n_tiles_n = (a.n_cols + kPairs * CPW - 1) / (kPairs * CPW);
  const int64_t mt = a.seg_off ? mt_cap
                              : (a.dense_rows + RB * 32 - 1) / (RB * 32) *
                                    (a.k_splits > 1 ? a.k_splits : 1);
  const int64_t grid = gemm::round8(mt * n_tiles_n);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  moe_gemm_bf16<RB, W, EPI, AMODE, KT, LDS><<<dim3((unsigned)grid), dim3(64 * W), 0, s>>>(a, n_tiles_n);
  return hipGetLastError();
}

// Tile heights: rb in {1, 2, 4, 6, 8} row blocks of 32; waves 8 (rb 4 and 8,
// not the router) or 4.  A K that is not a multiple of 64 (odd shapes only)
// runs the clamped variant, with rb = 1.
template <int EPI, int AMODE>
hipError_t launch_any(const GemmArgs& a, int rb, int waves, int64_t mt_cap, hipStream_t s) {
  const bool kt = (a.K % 64) != 0 && AMODE != A_REPEAT;
  if (kt) {
    if constexpr (AMODE != A_REPEAT) {
      if (rb == 1) return launch_rb<1, 4, EPI, AMODE, true>(a, mt_cap, s);
    }
    return hipErrorInvalidValue;
  }
  const bool w8 = waves == 8 && AMODE != A_REPEAT;
  // 4-wave tiles of up to 4 row blocks share a CU two by two (half the LDS
  // each); the router's product keeps the whole CU
  constexpr int kHalf = AMODE == A_REPEAT ? kLdsMax : kLdsHalf;
  switch (rb) {
    case 1: return launch_rb<1, 4, EPI, AMODE, false, kHalf>(a, mt_cap, s);
    case 2: return launch_rb<2, 4, EPI, AMODE, false, kHalf>(a, mt_cap, s);
    case 4:
      if constexpr (AMODE != A_REPEAT) {
        if (w8) return launch_rb<4, 8, EPI, AMODE, false>(a, mt_cap, s);
      }
      return launch_rb<4, 4, EPI, AMODE, false, kHalf>(a, mt_cap, s);
    case 6:
      if constexpr (AMODE != A_REPEAT) return launch_rb<6, 4, EPI, AMODE, false>(a, mt_cap, s);
      return hipErrorInvalidValue;
    case 8:
      // 256-row gate/up tiles always run 8 waves: with 4, their activation
      // epilogue is too large to unroll over 8 row blocks
      if constexpr (AMODE != A_REPEAT) {
        if (w8 || EPI == EPI_GATE_UP) return launch_rb<8, 8, EPI, AMODE, false>(a, mt_cap, s);
      }
      if constexpr (EPI != EPI_GATE_UP) return launch_rb<8, 4, EPI, AMODE, false>(a, mt_cap, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int epi, int amode, int rb, int waves,
                            int64_t mt_cap, hipStream_t s) {
  if (epi == EPI_GATE_UP && amode == A_DIRECT)
    return launch_any<EPI_GATE_UP, A_DIRECT>(a, rb, waves, mt_cap, s);
  if (epi == EPI_GATE_UP && amode == A_GATHER)
    return launch_any<EPI_GATE_UP, A_GATHER>(a, rb, waves, mt_cap, s);
  if (epi == EPI_STORE && amode == A_DIRECT)
    return launch_any<EPI_STORE, A_DIRECT>(a, rb, waves, mt_cap, s);
  if (epi == EPI_STORE_RES && amode == A_DIRECT)
    return launch_any<EPI_STORE_RES, A_DIRECT>(a, rb, waves, mt_cap, s);
  if (epi == EPI_STORE_F32 && amode == A_DIRECT)
    return launch_any<EPI_STORE_F32, A_DIRECT>(a, rb, waves, mt_cap, s);
  if (epi == EPI_STORE_F32 && amode == A_REPEAT)
    return launch_any<EPI_STORE_F32, A_REPEAT>(a, rb, waves, mt_cap, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
