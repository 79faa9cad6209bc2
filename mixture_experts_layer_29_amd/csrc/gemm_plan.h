// gemm_plan.h - the streaming plan of the grouped bf16 GEMM (gemm_bf16.hip):
// LDS stages per tile height and the vmcnt counts of its pipeline.  Plain
// C++ (compile-time only), so the host tests can check the counts against a
// simulation of the kernel's issue order.
#pragma once

namespace moe {
namespace plan {

constexpr int kPairs = 4;                           // column pairs (32+32 columns) per tile
constexpr int kRowBytes = 128;                      // one 64-element K block of a bf16 row
constexpr int kBRows = 32;                          // weight rows of a column pair per sub-block
constexpr int kBPair = kBRows * kRowBytes;          // 4 KB
constexpr int kBStage = kPairs * kBPair;            // 16 KB
constexpr int kLdsMax = 160 * 1024;                 // LDS of one CU
constexpr int kLdsHalf = 80 * 1024;                 // half of it: two work-groups per CU

// LDS plan of a tile with NR row blocks in an LDS budget of LDS bytes: NA
// activation stages of NR x 4 KB, then as many 16 KB weight stages as fit (at
// most 9).  Loads complete in issue order, so waiting for the activations of
// a K block also waits for every weight load issued before them: the
// activations are issued NA - 1 K blocks (2 (NA - 1) sub-iterations) ahead,
// far enough that the wait for them does not drain the weight loads in
// flight.  With the whole CU, short tiles afford four activation stages, tall
// ones three.  With half of it (two work-groups per CU, each covering the
// other's tile start and end) the rings are shallower: 4, 3 or 2 activation
// stages for 1, 2 or more row blocks, and 3 or 4 weight stages.
template <int NR, int LDS = kLdsMax>
struct Ring {
  static constexpr int kATile = NR * 32 * kRowBytes;
  static constexpr int kNA = LDS == kLdsMax ? (NR <= 5 ? 4 : 3) : (NR <= 1 ? 4 : NR == 2 ? 3 : 2);
  static constexpr int kFit = (LDS - kNA * kATile) / kBStage;
  static constexpr int kNB = kFit > 9 ? 9 : kFit;
  static constexpr int kBytes = kNA * kATile + kNB * kBStage;
  static_assert(kNB >= 3 && kBytes <= LDS, "LDS plan");
};
// vmcnt for the wait of sub-iteration u (even or odd, away from the start).
// vmcnt counts a wave's loads in issue order, so the wait lets through the
// loads issued after the newest one that u needs: sub-block u, issued at
// u - (NB - 1), and for even u the activations of its K block, issued at
// u - 2 (NA - 1).  Issue points (key 2 s + phase, in program order): with
// W = 4, sub-iteration s issues its weights before its wait (phase 0) and,
// for even s, its activations after its barrier (phase 1); with W = 8 both
// come after the barrier, activations first (phase 0), and nothing of s is
// issued before its wait.
template <int W, int NA, int NB, int NRH, int KBL>
constexpr int wait_count(bool even) {
  const int u = even ? 64 : 65;
  const int pa = W == 4 ? 1 : 0, pb = W == 4 ? 0 : 1;
  int newest = 2 * (u - (NB - 1)) + pb;
  if (even) {
    const int ka = 2 * (u - 2 * (NA - 1)) + pa;
    if (ka > newest) newest = ka;
  }
  const int last = W == 4 ? 2 * u + pb : 2 * u - 1;
  int n = 0;
  for (int key = newest + 1; key <= last; ++key) {
    if ((key & 1) == pb) n += KBL;
    if ((key & 1) == pa && ((key >> 1) & 1) == 0) n += NRH;
  }
  return n;
}

}  // namespace plan
}  // namespace moe
