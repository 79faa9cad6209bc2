// gemm_lds.h - device helpers shared by the bf16 MFMA GEMM kernels: the
// HBM->LDS copies of the load units, the swizzled LDS row layout, and the
// explicit waits and barriers of their software pipelines.
#pragma once

#include "gemm_common.h"
#include "gemm_plan.h"

namespace moe {
namespace lds {

// One wave-wide HBM->LDS copy: lane l's 16 bytes at `src` land at LDS byte
// address m0 + 16 l (m0 = `lds`, uniform).  Written as inline asm on purpose:
// the instruction has no register results (nothing for the compiler to track),
// and the compiler, seeing an LDS-DMA load in flight, would otherwise treat
// every LDS read as unordered and wait for all of them before each MFMA.  The
// loads are counted by the explicit vmcnt waits of the pipelines using it.  An
// LDS-DMA load must not directly follow the scalar write of m0 (one wait
// state), hence the s_nop.
template <bool NT>
__device__ __forceinline__ void dma16(const void* src, const uint8_t* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>(lds));
  if (NT) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src), "s"(m0) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0) : "memory", "m0");
  }
}

using plan::kRowBytes;

// Byte offset of 16-byte chunk `c` of row `r` in a swizzled 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) {
  return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4);
}

// Compiler-level fence: no memory access moves across it (IR or scheduler).
__device__ __forceinline__ void code_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt on the vector-memory counter only (lgkm and exp left free).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  code_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  code_fence();
}
__device__ __forceinline__ void wait_lgkm0() {
  code_fence();
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  code_fence();
}
// Work-group barrier without the memory fence of __syncthreads (whose release
// semantics would wait for every load in flight, including the prefetches).
// LDS visibility is arranged by the explicit waits before it.
__device__ __forceinline__ void wg_barrier() {
  code_fence();
  __builtin_amdgcn_s_barrier();
  code_fence();
}

}  // namespace lds
}  // namespace moe
