/*
 * synth_host.c - host filler for the seeded synthetic inputs (libsynth_host.so).
 *
 * Element i of tensor (seed, tid) is std * N_i where N_i is the standard normal
 * defined in synth_core.h; it is rounded once to the destination type.  The
 * elements [first, first + count) are written to out[0 .. count).  The same
 * definitions run on the GPU in synth_dev.hip; both must give the same bits.
 */
#include <stdint.h>
#include <stddef.h>

#include "synth_core.h"

#define SYNTH_DTYPE_F32 0
#define SYNTH_DTYPE_BF16 1

int synth_fill_normal(void* out, int dtype, int64_t count, uint64_t first, uint64_t seed,
                      uint32_t tid, double std) {
  if (count < 0 || (count > 0 && out == NULL)) return 1;
  if (dtype != SYNTH_DTYPE_F32 && dtype != SYNTH_DTYPE_BF16) return 1;
  if (count == 0) return 0;
  const uint64_t end = first + (uint64_t)count;
  const int64_t q_begin = (int64_t)(first >> 2), q_end = (int64_t)((end + 3u) >> 2);
  /* One Philox call and two Box-Muller pairs per block of four elements. */
#pragma omp parallel for schedule(static)
  for (int64_t q = q_begin; q < q_end; ++q) {
    const synth_u32x4 w = synth_block_bits(seed, tid, (uint64_t)q);
    double z[4];
    synth_box_muller(w.v[0], w.v[1], &z[0], &z[1]);
    synth_box_muller(w.v[2], w.v[3], &z[2], &z[3]);
    for (int lane = 0; lane < 4; ++lane) {
      const uint64_t i = (uint64_t)q * 4u + (uint64_t)lane;
      if (i < first || i >= end) continue;
      const float f = (float)(z[lane] * std);
      if (dtype == SYNTH_DTYPE_F32) {
        ((float*)out)[i - first] = f;
      } else {
        ((uint16_t*)out)[i - first] = synth_f32_to_bf16(f);
      }
    }
  }
  return 0;
}

/* Raw 32-bit words: word i is output i%4 of block i/4. */
int synth_fill_u32(uint32_t* out, int64_t count, uint64_t first, uint64_t seed, uint32_t tid) {
  if (count < 0 || (count > 0 && out == NULL)) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    const uint64_t i = first + (uint64_t)j;
    out[j] = synth_block_bits(seed, tid, i >> 2).v[i & 3u];
  }
  return 0;
}

/* Philox4x32-10 on one explicit counter and key (known-answer checks). */
void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const synth_u32x4 w = synth_philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = w.v[i];
}

/* The transform pieces, exposed so that tests can check them on their own. */
double synth_log_u1_host(uint32_t a) { return synth_log_u1(a); }
double synth_sqrt_host(double v) { return synth_sqrt(v); }
void synth_box_muller_host(uint32_t a, uint32_t b, double* z0, double* z1) {
  synth_box_muller(a, b, z0, z1);
}
