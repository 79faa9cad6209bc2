/*
 * synth_core.h - the seeded synthetic-input generator, as plain inline C.
 *
 * This header is the whole definition of the generator.  It holds no step of
 * the mixture-of-experts method: it only turns (seed, tensor id, element index)
 * into a number.  It is compiled twice from this one text: by gcc into the host
 * filler (synth_host.c) and by hipcc into the device filler (synth_dev.hip), so
 * that a tensor filled on the GPU and the same tensor filled on the host are
 * bit-identical.  To keep them identical the code uses only integer arithmetic
 * and IEEE-754 double +, -, *, / (correctly rounded on both processors), with
 * floating-point contraction switched off by both builds; no libm call appears.
 *
 * Uniform bits: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten
 * rounds of two 32x32->64-bit multiplies with the published multipliers and
 * Weyl key increments.
 *
 * Normals: the Box-Muller transform (Box and Muller, 1958): from uniforms
 * u1 in (0,1] and u2 in [0,1), rho = sqrt(-2 ln u1) and theta = 2 pi u2 give
 * the independent standard normals rho cos(theta) and rho sin(theta).  The log
 * is an atanh series after an exact power-of-two split, the square root is
 * Newton's iteration, sin and cos are Taylor series after an exact quadrant
 * split of the 32-bit integer that defines u2.
 *
 * Element i of a tensor draws counter (i/4 low, i/4 high, tensor id, SALT) under
 * key (seed low, seed high); the four 32-bit outputs give two Box-Muller pairs,
 * i.e. four normals, and element i takes normal number i%4.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#define SYNTH_SALT 0x5EED0A11u

typedef struct {
  uint32_t v[4];
} synth_u32x4;

/* Philox4x32 with 10 rounds (Salmon et al., SC'11, section 3.3). */
static inline synth_u32x4 synth_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                              uint32_t c3, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  synth_u32x4 out;
  out.v[0] = c0;
  out.v[1] = c1;
  out.v[2] = c2;
  out.v[3] = c3;
  return out;
}

/* The four raw 32-bit words that serve elements 4q .. 4q+3 of tensor `tid`. */
static inline synth_u32x4 synth_block_bits(uint64_t seed, uint32_t tid, uint64_t q) {
  return synth_philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), tid, SYNTH_SALT,
                             (uint32_t)seed, (uint32_t)(seed >> 32));
}

static inline double synth_bits_to_double(uint64_t b) {
  union {
    uint64_t u;
    double d;
  } c;
  c.u = b;
  return c.d;
}

static inline uint64_t synth_double_to_bits(double d) {
  union {
    uint64_t u;
    double d;
  } c;
  c.d = d;
  return c.u;
}

/* ln(u1) for u1 = (a + 1) * 2^-32, a in [0, 2^32).  m = a + 1 = 2^e * f exactly,
 * f folded into [sqrt(1/2), sqrt(2)); ln f = 2 atanh(s) with s = (f-1)/(f+1),
 * |s| < 0.1716, summed to s^29 (truncation below 1e-23 relative). */
static inline double synth_log_u1(uint32_t a) {
  const uint64_t m = (uint64_t)a + 1u;
  int e = 63 - __builtin_clzll(m);
  /* f = m / 2^e, exact: build 2^-e from its exponent bits. */
  double f = (double)m * synth_bits_to_double((uint64_t)(1023 - e) << 52);
  if (f > 1.4142135623730951) {
    f = f * 0.5;
    e = e + 1;
  }
  const double s = (f - 1.0) / (f + 1.0);
  const double z = s * s;
  double p = 1.0 / 29.0;
  p = p * z + 1.0 / 27.0;
  p = p * z + 1.0 / 25.0;
  p = p * z + 1.0 / 23.0;
  p = p * z + 1.0 / 21.0;
  p = p * z + 1.0 / 19.0;
  p = p * z + 1.0 / 17.0;
  p = p * z + 1.0 / 15.0;
  p = p * z + 1.0 / 13.0;
  p = p * z + 1.0 / 11.0;
  p = p * z + 1.0 / 9.0;
  p = p * z + 1.0 / 7.0;
  p = p * z + 1.0 / 5.0;
  p = p * z + 1.0 / 3.0;
  p = p * z + 1.0;
  const double lnf = 2.0 * s * p;
  const double ln2 = 0.6931471805599453;
  return (double)(e - 32) * ln2 + lnf;
}

/* sqrt(v), v >= 0, by Newton's iteration y <- (y + v/y)/2 from a guess that
 * halves the exponent; seven steps reach the fixed point from any guess
 * within a factor of two. */
static inline double synth_sqrt(double v) {
  if (v <= 0.0) return 0.0;
  double y = synth_bits_to_double((synth_double_to_bits(v) >> 1) + 0x1FF8000000000000ull);
  for (int i = 0; i < 7; ++i) y = 0.5 * (y + v / y);
  return y;
}

/* sin and cos of phi in [0, pi/2) by their Taylor series in nested form,
 * to phi^27 / phi^26 (truncation below 1e-22). */
static inline double synth_sin_q(double x) {
  const double z = x * x;
  double p = 1.0 - z / (26.0 * 27.0);
  p = 1.0 - z / (24.0 * 25.0) * p;
  p = 1.0 - z / (22.0 * 23.0) * p;
  p = 1.0 - z / (20.0 * 21.0) * p;
  p = 1.0 - z / (18.0 * 19.0) * p;
  p = 1.0 - z / (16.0 * 17.0) * p;
  p = 1.0 - z / (14.0 * 15.0) * p;
  p = 1.0 - z / (12.0 * 13.0) * p;
  p = 1.0 - z / (10.0 * 11.0) * p;
  p = 1.0 - z / (8.0 * 9.0) * p;
  p = 1.0 - z / (6.0 * 7.0) * p;
  p = 1.0 - z / (4.0 * 5.0) * p;
  p = 1.0 - z / (2.0 * 3.0) * p;
  return x * p;
}

static inline double synth_cos_q(double x) {
  const double z = x * x;
  double p = 1.0 - z / (25.0 * 26.0);
  p = 1.0 - z / (23.0 * 24.0) * p;
  p = 1.0 - z / (21.0 * 22.0) * p;
  p = 1.0 - z / (19.0 * 20.0) * p;
  p = 1.0 - z / (17.0 * 18.0) * p;
  p = 1.0 - z / (15.0 * 16.0) * p;
  p = 1.0 - z / (13.0 * 14.0) * p;
  p = 1.0 - z / (11.0 * 12.0) * p;
  p = 1.0 - z / (9.0 * 10.0) * p;
  p = 1.0 - z / (7.0 * 8.0) * p;
  p = 1.0 - z / (5.0 * 6.0) * p;
  p = 1.0 - z / (3.0 * 4.0) * p;
  p = 1.0 - z / (1.0 * 2.0) * p;
  return p;
}

/* One Box-Muller pair from the words (a, b): u1 = (a+1)/2^32, u2 = b/2^32.
 * theta = 2 pi u2 = quadrant * pi/2 + phi with quadrant = b >> 30 exactly. */
static inline void synth_box_muller(uint32_t a, uint32_t b, double* z0, double* z1) {
  const double rho = synth_sqrt(-2.0 * synth_log_u1(a));
  const uint32_t quad = b >> 30;
  /* (pi/2) * 2^-30 */
  const double phi = (double)(b & 0x3FFFFFFFu) * 1.4629180792671596e-09;
  const double s = synth_sin_q(phi), c = synth_cos_q(phi);
  double cs, sn;
  if (quad == 0u) {
    cs = c;
    sn = s;
  } else if (quad == 1u) {
    cs = -s;
    sn = c;
  } else if (quad == 2u) {
    cs = -c;
    sn = -s;
  } else {
    cs = s;
    sn = -c;
  }
  *z0 = rho * cs;
  *z1 = rho * sn;
}

/* Standard normal number `lane` (0..3) of block q. */
static inline double synth_normal_in_block(synth_u32x4 w, int lane) {
  double z0, z1;
  if (lane < 2) {
    synth_box_muller(w.v[0], w.v[1], &z0, &z1);
  } else {
    synth_box_muller(w.v[2], w.v[3], &z0, &z1);
  }
  return (lane & 1) ? z1 : z0;
}

/* float -> bfloat16 bits, round to nearest even (inputs here are finite). */
static inline uint16_t synth_f32_to_bf16(float f) {
  union {
    uint32_t u;
    float f;
  } c;
  c.f = f;
  const uint32_t u = c.u + 0x7FFFu + ((c.u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* SYNTH_CORE_H */
