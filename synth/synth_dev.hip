// synth_dev.hip - device filler for the seeded synthetic inputs (libsynth_dev.so).
//
// The same element definition as synth_host.c, compiled for the GPU from the one
// header synth_core.h, so that large tensors are filled in place in HBM rather than
// generated on the host and copied.  Built with contraction off; a GPU test checks
// these bits against the host filler's.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang force_cuda_host_device begin
#include "synth_core.h"
#pragma clang force_cuda_host_device end

namespace {

constexpr int kThreads = 256;

// Thread t serves block q = q0 + t (elements 4q .. 4q+3) and writes the ones that
// fall inside [first, first + count).
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void fill_normal_kernel(void* out, int64_t count,
                                                               uint64_t first, uint64_t seed,
                                                               uint32_t tid, double stdev,
                                                               uint64_t q_begin, uint64_t n_blocks) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t b = (uint64_t)blockIdx.x * kThreads + threadIdx.x; b < n_blocks; b += stride) {
    const uint64_t q = q_begin + b;
    const synth_u32x4 w = synth_block_bits(seed, tid, q);
    double z[4];
    synth_box_muller(w.v[0], w.v[1], &z[0], &z[1]);
    synth_box_muller(w.v[2], w.v[3], &z[2], &z[3]);
#pragma unroll
    for (int lane = 0; lane < 4; ++lane) {
      const uint64_t i = q * 4u + (uint64_t)lane;
      if (i < first || i >= first + (uint64_t)count) continue;
      const float f = (float)(z[lane] * stdev);
      if (kBf16) {
        static_cast<uint16_t*>(out)[i - first] = synth_f32_to_bf16(f);
      } else {
        static_cast<float*>(out)[i - first] = f;
      }
    }
  }
}

}  // namespace

extern "C" int synth_dev_fill_normal(void* out, int dtype, int64_t count, uint64_t first,
                                     uint64_t seed, uint32_t tid, double stdev, void* stream) {
  if (count < 0 || (count > 0 && out == nullptr)) return 1;
  if (dtype != 0 && dtype != 1) return 1;
  if (count == 0) return 0;
  const uint64_t q_begin = first >> 2;
  const uint64_t q_end = (first + (uint64_t)count + 3u) >> 2;
  const uint64_t n_blocks = q_end - q_begin;
  uint64_t grid = (n_blocks + kThreads - 1) / kThreads;
  if (grid > 65536) grid = 65536;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == 1) {
    fill_normal_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(
        out, count, first, seed, tid, stdev, q_begin, n_blocks);
  } else {
    fill_normal_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(
        out, count, first, seed, tid, stdev, q_begin, n_blocks);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
