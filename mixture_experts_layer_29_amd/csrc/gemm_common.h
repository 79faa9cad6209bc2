// gemm_common.h - pieces shared by the bf16 MFMA and the fp32 GEMM kernels:
// tile location, the XCD-aware work-group order, and the expert activations.
#pragma once

#include "common.h"

namespace moe {
namespace gemm {

// Work-groups are dispatched to the 8 XCDs round-robin (id % 8); work-group id
// runs as the (id / 8)-th of its XCD's grid / 8 work-groups.  Grouped
// products: the dispatch scan split the segments into 8 runs of about equal
// estimated cost (mt_off[S+1 .. S+9]), and XCD x takes the tiles of its run
// (contiguous: the tiles of one expert share its activation rows in the XCD's
// L2), its work-groups striding through them.  Dense products: the T tiles
// are cut into 8 contiguous runs of ceil(T/8).  A work-group processes tiles
// first, first + step, ... below end.
template <int BM>
__device__ __forceinline__ void tile_range(const GemmArgs& a, int64_t bid, int64_t nwg,
                                           int64_t n_tiles_n, int64_t& first, int64_t& end,
                                           int64_t& step) {
  const int64_t x = bid & 7, i = bid >> 3;
  step = nwg >> 3;
  if (a.seg_off) {
    const int32_t* xs = a.mt_off + a.n_seg + 1;
    first = (int64_t)a.mt_off[xs[x]] * n_tiles_n + i;
    end = (int64_t)a.mt_off[xs[x + 1]] * n_tiles_n;
    return;
  }
  const int64_t T = (a.dense_rows + BM - 1) / BM * n_tiles_n * (a.k_splits > 1 ? a.k_splits : 1);
  const int64_t per = (T + 7) >> 3;
  first = x * per + i;
  end = min(T, (x + 1) * per);
  step = i < per ? per : 1;  // one tile each (the grid holds 8 * per work-groups)
  if (i >= per) first = end;
}

// Expert activations (Kimi K3 "Gate features" page: expert and situ excerpts):
// SiLU: silu(g) * u;  SiTU: beta*tanh(g/beta)*sigmoid(g) * (lb*tanh(u/lb) or u),
// all in fp32.
__device__ __forceinline__ float act_pair(int act, float g, float u, float beta, float lbeta) {
  if (act == ACT_SILU) return g / (1.0f + expf(-g)) * u;
  const float a = beta * tanhf(g / beta) * (1.0f / (1.0f + expf(-g)));
  const float up = lbeta > 0.0f ? lbeta * tanhf(u / lbeta) : u;
  return a * up;
}

struct TileLoc {
  int64_t seg;
  int64_t mt;     // m-tiles of the segment (grouped), 0 for a dense product
  int64_t row0;   // first row of the tile in the concatenated row space
  int rows;       // rows of the tile that exist (1 .. BM)
  int64_t j;      // n-tile
  int64_t split;  // K range (dense split-K), else 0
  int64_t kb0;    // first 64-wide K block of the tile's K range
  int64_t kb1;    // one past its last block
};

// Logical tile L -> (segment, m-tile, n-tile, K range).  Grouped: tiles are
// numbered segment by segment; inside a segment n-tile-major with the m-tiles
// adjacent, so the m-tiles that share one weight tile run side by side.
// Dense: the same with one segment, repeated for each K range of a split-K
// product.  False when L is past the last tile.
template <int BM>
__device__ __forceinline__ bool locate(const GemmArgs& a, int64_t L, int64_t n_tiles_n,
                                       TileLoc& t) {
  if (a.seg_off) {
    const int64_t u = L / n_tiles_n;  // m-tile index
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
    t.mt = mt;
    t.row0 = s0 + i * BM;
    t.rows = (int)min((int64_t)BM, s1 - t.row0);
    t.j = j;
    t.split = 0;
    t.kb0 = 0;
    t.kb1 = (a.K + 63) >> 6;
    return t.row0 >= 0 && t.rows > 0;
  }
  const int64_t mt = (a.dense_rows + BM - 1) / BM;
  const int64_t per_split = mt * n_tiles_n;
  const int64_t splits = a.k_splits > 1 ? a.k_splits : 1;
  if (L >= per_split * splits) return false;
  const int64_t q = L / per_split;
  L -= q * per_split;
  const int64_t j = L / mt, i = L - j * mt;
  const int64_t nkb = (a.K + 63) >> 6;
  t.seg = 0;
  t.mt = 0;
  t.row0 = i * BM;
  t.rows = (int)min((int64_t)BM, a.dense_rows - t.row0);
  t.j = j;
  t.split = q;
  t.kb0 = splits > 1 ? q * a.k_split_blocks : 0;
  t.kb1 = splits > 1 ? min(nkb, t.kb0 + a.k_split_blocks) : nkb;
  return t.kb1 > t.kb0;
}

inline int64_t round8(int64_t n) { return (n + 7) & ~(int64_t)7; }

}  // namespace gemm
}  // namespace moe
