// permute.hip - dispatch of the (token, slot) pairs by expert (Kimi K3 "Add
// shared output" page, moe-forward excerpt: the one-hot count of chosen
// experts, the argsort of the flattened choices and the row gather).
//
// The sorted order is the stable one: expert by expert, and within an expert
// the flat slots n*k + j in increasing order.  Since a token never holds an
// expert twice, a slot's rank inside its expert's segment is the number of
// earlier tokens that chose the same expert.  That count is built from
// bit masks, without sorting and without float or order-dependent atomics:
//   mask    - per chunk of 64 tokens and per expert, the 64-bit set of tokens
//             of the chunk that chose the expert (LDS atomic OR);
//   scan    - per expert, popcounts summed over chunks: the counts, their
//             exclusive scan (the expert offsets), the absolute start of every
//             (chunk, expert) run, and the m-tile table of the grouped GEMM;
//   scatter - slot (n, j) with expert e lands at
//             start(chunk, e) + popcount(mask(chunk, e) below lane n%64).
#include "common.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(64) void moe_dispatch_mask(const int32_t* __restrict__ idx, int64_t N,
                                                        int k, int64_t E,
                                                        uint64_t* __restrict__ bits) {
  __shared__ unsigned long long m[1024];
  const int lane = threadIdx.x;
  for (int64_t e = lane; e < E; e += 64) m[e] = 0ull;
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 64 + lane;
  if (n < N) {
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[n * k + j];
      if (e >= 0 && e < E) atomicOr(&m[e], 1ull << lane);
    }
  }
  __syncthreads();
  uint64_t* out = bits + (int64_t)blockIdx.x * E;
  for (int64_t e = lane; e < E; e += 64) out[e] = m[e];
}

// Block-wide exclusive scan of one value per thread (1024 threads), fixed order.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t add = t >= off ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  const int32_t incl = sh[t];
  *total = sh[kScanThreads - 1];
  __syncthreads();
  return incl - v;
}

// Splits the segments (in id order, so each XCD gets a contiguous run) into 8
// runs of about equal estimated cost, one per XCD, and writes the run
// boundaries xcd_seg[0..8] (xcd_seg[0] = 0; xcd_seg[x] for x = 1..7 is the
// first segment whose cost-prefix reaches x/8 of the total, E if none).  A
// segment's cost: kTileCost per m-tile (streaming its weights) plus one per
// 32-row block (its MFMA work).  Thread e owns segment e; every thread calls.
constexpr int32_t kTileCost = 4;
__device__ void xcd_split(int64_t E, int32_t cnt, int32_t mt, int32_t* sh,
                          int32_t* __restrict__ xcd_seg) {
  const int e = threadIdx.x;
  const int32_t cost = e < E ? mt * kTileCost + (cnt + 31) / 32 : 0;
  int32_t total;
  block_exclusive_scan(cost, sh, &total);  // leaves the inclusive prefix in sh
  if (e < 9) xcd_seg[e] = e == 0 ? 0 : (int32_t)E;
  __syncthreads();
  if (e < E) {
    const int64_t start = e == 0 ? 0 : sh[e - 1];
    const int64_t prev_start = e >= 2 ? sh[e - 2] : 0;
    for (int x = 1; x < 8; ++x) {
      const int64_t mark = ((int64_t)total * x + 7) / 8;
      if (start >= mark && (e == 0 || prev_start < mark)) xcd_seg[x] = e;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void moe_dispatch_scan(
    const uint64_t* __restrict__ bits, int64_t n_chunks, int64_t E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ base, int rows_per_tile,
    int32_t* __restrict__ mt_off, int32_t* __restrict__ tile_seg, int64_t tile_cap) {
  __shared__ int32_t sh[kScanThreads];
  const int e = threadIdx.x;  // E <= 1024
  int32_t cnt = 0;
  if (e < E) {
    int64_t c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      uint64_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = bits[(c + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) cnt += __popcll(w[q]);
    }
    for (; c < n_chunks; ++c) cnt += __popcll(bits[c * E + e]);
  }
  int32_t total;
  const int32_t off = block_exclusive_scan(e < E ? cnt : 0, sh, &total);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    int32_t run = off;
    int64_t c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      uint64_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) w[q] = bits[(c + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        base[(c + q) * E + e] = run;
        run += __popcll(w[q]);
      }
    }
    for (; c < n_chunks; ++c) {
      base[c * E + e] = run;
      run += __popcll(bits[c * E + e]);
    }
  }
  if (e == 0) offsets[E] = total;
  if (rows_per_tile > 0) {
    const int32_t mt = e < E ? (cnt + rows_per_tile - 1) / rows_per_tile : 0;
    int32_t mt_total;
    const int32_t mb = block_exclusive_scan(mt, sh, &mt_total);
    if (e < E) {
      mt_off[e] = mb;
      for (int32_t u = mb; u < mb + mt && u < tile_cap; ++u) tile_seg[u] = e;
    }
    if (e == 0) mt_off[E] = mt_total;
    for (int64_t u = (int64_t)mt_total + e; u < tile_cap; u += kScanThreads) tile_seg[u] = -1;
    xcd_split(E, cnt, mt, sh, mt_off + E + 1);
  }
}

__global__ __launch_bounds__(64) void moe_dispatch_scatter(
    const int32_t* __restrict__ idx, int64_t N, int k, int64_t E, const uint64_t* __restrict__ bits,
    const int32_t* __restrict__ base, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  const int lane = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  const int64_t n = chunk * 64 + lane;
  if (n >= N) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int64_t slot = n * k + j;
    const int32_t e = idx[slot];
    if (e < 0 || e >= E) {
      inv_perm[slot] = -1;
      continue;
    }
    const int64_t pos = base[chunk * E + e] + __popcll(bits[chunk * E + e] & below);
    perm[pos] = (int32_t)slot;
    inv_perm[slot] = (int32_t)pos;
  }
}

// x_sorted[p] = x[perm[p] / k]: one row per work-group iteration, 16 B per thread.
__global__ __launch_bounds__(256) void moe_gather_rows(const uint8_t* __restrict__ x, int64_t N,
                                                       int64_t row_bytes,
                                                       const int32_t* __restrict__ perm, int k,
                                                       int64_t rows, uint8_t* __restrict__ out) {
  for (int64_t p = blockIdx.x; p < rows; p += gridDim.x) {
    int64_t src = perm[p] / k;
    src = src < 0 ? 0 : (src >= N ? N - 1 : src);
    const uint8_t* s = x + src * row_bytes;
    uint8_t* d = out + p * row_bytes;
    for (int64_t b = (int64_t)threadIdx.x * 16; b < row_bytes; b += 256 * 16) {
      *reinterpret_cast<u32x4*>(d + b) = *reinterpret_cast<const u32x4*>(s + b);
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void moe_tiles_from_offsets(
    const int32_t* __restrict__ offsets, int64_t E, int rows_per_tile, int32_t* __restrict__ mt_off,
    int32_t* __restrict__ tile_seg, int64_t tile_cap) {
  __shared__ int32_t sh[kScanThreads];
  const int e = threadIdx.x;
  int32_t cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  if (cnt < 0) cnt = 0;
  const int32_t mt = (cnt + rows_per_tile - 1) / rows_per_tile;
  int32_t mt_total;
  const int32_t mb = block_exclusive_scan(mt, sh, &mt_total);
  if (e < E) {
    mt_off[e] = mb;
    for (int32_t u = mb; u < mb + mt && u < tile_cap; ++u) tile_seg[u] = e;
  }
  if (e == 0) mt_off[E] = mt_total;
  for (int64_t u = (int64_t)mt_total + e; u < tile_cap; u += kScanThreads) tile_seg[u] = -1;
  xcd_split(E, cnt, mt, sh, mt_off + E + 1);
}

}  // namespace

hipError_t launch_dispatch_mask(const int32_t* topk_idx, int64_t N, int k, int64_t E,
                                uint64_t* bits, hipStream_t s) {
  const int64_t chunks = (N + 63) / 64;
  if (chunks == 0) return hipSuccess;
  moe_dispatch_mask<<<dim3((unsigned)chunks), dim3(64), 0, s>>>(topk_idx, N, k, E, bits);
  return hipGetLastError();
}

hipError_t launch_dispatch_scan(const uint64_t* bits, int64_t n_chunks, int64_t E, int32_t* counts,
                                int32_t* offsets, int32_t* base, int rows_per_tile,
                                int32_t* mt_off, int32_t* tile_seg, int64_t tile_cap,
                                hipStream_t s) {
  moe_dispatch_scan<<<dim3(1), dim3(kScanThreads), 0, s>>>(bits, n_chunks, E, counts, offsets, base,
                                                           rows_per_tile, mt_off, tile_seg, tile_cap);
  return hipGetLastError();
}

hipError_t launch_dispatch_scatter(const int32_t* topk_idx, int64_t N, int k, int64_t E,
                                   const uint64_t* bits, const int32_t* base, int32_t* perm,
                                   int32_t* inv_perm, hipStream_t s) {
  const int64_t chunks = (N + 63) / 64;
  if (chunks == 0) return hipSuccess;
  moe_dispatch_scatter<<<dim3((unsigned)chunks), dim3(64), 0, s>>>(topk_idx, N, k, E, bits, base,
                                                                   perm, inv_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, int64_t N, int64_t width, int elem_bytes,
                              const int32_t* perm, int k, int64_t rows, void* x_sorted,
                              hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int64_t grid = rows < 65536 ? rows : 65536;
  moe_gather_rows<<<dim3((unsigned)grid), dim3(256), 0, s>>>(
      static_cast<const uint8_t*>(x), N, width * elem_bytes, perm, k, rows,
      static_cast<uint8_t*>(x_sorted));
  return hipGetLastError();
}

hipError_t launch_tiles_from_offsets(const int32_t* offsets, int64_t E, int rows_per_tile,
                                     int32_t* mt_off, int32_t* tile_seg, int64_t tile_cap,
                                     hipStream_t s) {
  moe_tiles_from_offsets<<<dim3(1), dim3(kScanThreads), 0, s>>>(offsets, E, rows_per_tile, mt_off,
                                                                tile_seg, tile_cap);
  return hipGetLastError();
}

}  // namespace moe
