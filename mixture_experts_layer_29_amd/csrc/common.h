// common.h - internal declarations shared by libmoe's HIP sources.
//
// Not part of the ABI (that is include/moe.h).  Holds the bf16 helpers, the
// MFMA vector types, the argument blocks of the kernel launchers and the
// launchers' prototypes.  Every launcher enqueues on the given stream and
// returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16_t)((u >> 16) | 0x40u);
  return (bf16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Activation kinds of the expert epilogues.
enum Act : int { ACT_SILU = 0, ACT_SITU = 1 };

// ---------------------------------------------------------------------------
// Grouped / dense GEMM: C[row, col] = sum_k A[row, k] * B[col, k] over row
// segments (one segment per expert, or one dense segment), B in nn.Linear
// layout [cols, K] per segment.
enum Epi : int {
  EPI_STORE = 0,       // C = acc (rounded to the output type)
  EPI_STORE_F32 = 1,   // C = acc as fp32 (router logits)
  EPI_GATE_UP = 2,     // C = act(acc_gate, acc_up), B0 = gate, B1 = up
  EPI_STORE_RES = 3,   // C = acc + residual (fp32 residual, one rounding)
};

enum AMode : int {
  A_DIRECT = 0,  // row p of the segment is row (seg_row0 + p) of A
  A_GATHER = 1,  // row p reads token a_map[seg_row0 + p] / a_div of A
  A_REPEAT = 2,  // dense; column kk of A is kk mod a_period (zero past a_valid)
};

struct GemmArgs {
  const void* A;          // activations
  int64_t lda;            // elements per A row
  const int32_t* a_map;   // A_GATHER: sorted row -> flat slot (perm)
  int32_t a_div;          // A_GATHER: slots per token (k)
  int64_t a_rows;         // rows of A (for clamping gathered indices)
  int64_t a_period;       // A_REPEAT: period of the K axis (padded width)
  int64_t a_valid;        // A_REPEAT: valid columns within a period
  const void* B0;         // weights, segment 0
  const void* B1;         // second weights (EPI_GATE_UP: up projection) or null
  int64_t b_seg_stride;   // elements between consecutive segments' weights
  int32_t b_stream;       // weight loads: 0 cached; 1 non-temporal; 2 non-temporal for a
                          // segment of one m-tile (its weights are read by no other tile)
  int64_t K;              // reduction length
  int64_t n_cols;         // output columns per segment
  const int32_t* seg_off; // [S+1] segment row offsets, or null for one dense segment
  int64_t dense_rows;     // rows of the dense segment (seg_off == null)
  int64_t k_splits;       // dense only: K is cut into this many ranges (0 or 1: none),
  int64_t k_split_blocks; //   each of this many 64-wide blocks, every range non-empty;
  int64_t c_split_stride; //   range s writes its partial product at C + s * c_split_stride
  const int32_t* mt_off;  // [S+1] m-tile prefix, then [9] first segment of each XCD's run
                          // (grouped only)
  int64_t n_seg;          // S, segments (grouped only)
  const int32_t* tile_seg;// m-tile -> segment, -1 past the last (grouped only)
  int64_t tile_cap;       // entries of tile_seg
  void* C;                // output
  int64_t ldc;
  const int32_t* c_map;   // grouped EPI_STORE: row p of the product is written to row
                          // c_map[p] of C (the slot order of the dispatch), or null
  int64_t c_rows;         // rows of C: tile rows at or past it are never touched
  const void* residual;   // EPI_STORE_RES: fp32 [rows, ld_res]
  int64_t ld_res;
  int32_t act;            // EPI_GATE_UP activation
  float beta;             // SiTU beta
  float lbeta;            // SiTU linear beta (<= 0: none)
};

// bf16 MFMA streaming GEMM; rb = row blocks of 32 per work-group (1, 2, 4, 6,
// 8), waves = 4 or 8 per work-group (8: rb 4 and 8 only, two per SIMD);
// grid capacity `mt_cap` m-tiles (grouped) is an upper bound of mt_off[S].
hipError_t launch_gemm_bf16(const GemmArgs& a, int epi, int amode, int rb, int waves,
                            int64_t mt_cap, hipStream_t s);
// bf16 MFMA GEMM for the dense products (one segment, A_DIRECT): 256 x 256
// tiles on 8 waves.  gemm_dense_supported: whole 64-deep K blocks and aligned
// rows; any EPI but the router's split-K fp32 partials.
bool gemm_dense_supported(const GemmArgs& a, int epi);
hipError_t launch_gemm_dense(const GemmArgs& a, int epi, hipStream_t s);
// fp32 SIMT GEMM for fp32 blocks (64-row m-tiles).
hipError_t launch_gemm_f32(const GemmArgs& a, int epi, int amode, int64_t mt_cap, hipStream_t s);
int gemm_f32_rows_per_tile();

// ---------------------------------------------------------------------------
// Router.
hipError_t launch_router_split(const float* w_router, int64_t E, int64_t d, int64_t dp,
                               bf16_t* w_split, hipStream_t s);
hipError_t launch_route_select(const float* logits, int n_parts, int64_t part_stride,
                               const float* bias, int softmax, int64_t N, int64_t E,
                               int G, int TG, int k, int norm, float scale, int32_t* topk_idx,
                               float* topk_weight, hipStream_t s);

// ---------------------------------------------------------------------------
// Dispatch.
hipError_t launch_dispatch_mask(const int32_t* topk_idx, int64_t N, int k, int64_t E,
                                uint64_t* bits, hipStream_t s);
// counts, offsets, absolute per-chunk bases, and (if rows_per_tile > 0) the
// m-tile table of the grouped GEMM.
hipError_t launch_dispatch_scan(const uint64_t* bits, int64_t n_chunks, int64_t E,
                                int32_t* counts, int32_t* offsets, int32_t* base,
                                int rows_per_tile, int32_t* mt_off, int32_t* tile_seg,
                                int64_t tile_cap, hipStream_t s);
hipError_t launch_dispatch_scatter(const int32_t* topk_idx, int64_t N, int k, int64_t E,
                                   const uint64_t* bits, const int32_t* base, int32_t* perm,
                                   int32_t* inv_perm, hipStream_t s);
hipError_t launch_gather_rows(const void* x, int64_t N, int64_t width, int elem_bytes,
                              const int32_t* perm, int k, int64_t rows, void* x_sorted,
                              hipStream_t s);
// m-tile table from caller-given expert offsets.
hipError_t launch_tiles_from_offsets(const int32_t* offsets, int64_t E, int rows_per_tile,
                                     int32_t* mt_off, int32_t* tile_seg, int64_t tile_cap,
                                     hipStream_t s);

// ---------------------------------------------------------------------------
// Combine.
// inv_perm: row of slot n*k + j in out_sorted, or NULL when out holds the rows in
// slot order; residual: [N, width] of the output type, or fp32 when res_f32 (or NULL)
hipError_t launch_combine(const void* out_sorted, const int32_t* inv_perm, const float* w,
                          const void* residual, int res_f32, void* y, int64_t N, int k,
                          int64_t width, int64_t rows, int bf16, hipStream_t s);
hipError_t launch_combine_rmsnorm(const void* out_sorted, const int32_t* inv_perm, const float* w,
                                  const float* gamma, float eps, int norm, void* y, int64_t N,
                                  int k, int64_t width, int64_t rows, int bf16, hipStream_t s);

}  // namespace moe
