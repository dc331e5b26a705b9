/* Seeded synthetic inputs: Philox4x32-10 counter-based generator.
 *
 * Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3" (SC'11): a 4x32-bit counter, a 2x32-bit
 * key, ten rounds of two 32x32->64 multiplies with key bumps in between.
 *
 * On top of it, one value per counter: an approximately standard normal
 * variate built from the eight 16-bit halves of the block (Irwin-Hall sum of
 * eight uniforms, centred and scaled to unit variance).  Every step is exact
 * integer arithmetic or one IEEE-754 operation, so host and device produce the
 * same bits.  This header holds no arithmetic of the MoE layer itself; it is
 * included by the host generator (gcc) and by the device generator (hipcc).
 */
#ifndef MOEGEN_PHILOX4X32_H
#define MOEGEN_PHILOX4X32_H

#include <stdint.h>

#ifdef __HIPCC__
#define MOEGEN_FN __host__ __device__ static inline
#else
#define MOEGEN_FN static inline
#endif

typedef struct { uint32_t v[4]; } moegen_u32x4;

MOEGEN_FN moegen_u32x4 moegen_philox4x32_10(moegen_u32x4 ctr, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)M0 * ctr.v[0];
    uint64_t p1 = (uint64_t)M1 * ctr.v[2];
    moegen_u32x4 n;
    n.v[0] = (uint32_t)(p1 >> 32) ^ ctr.v[1] ^ k0;
    n.v[1] = (uint32_t)p1;
    n.v[2] = (uint32_t)(p0 >> 32) ^ ctr.v[3] ^ k1;
    n.v[3] = (uint32_t)p0;
    ctr = n;
    k0 += W0;
    k1 += W1;
  }
  return ctr;
}

/* Approximately N(0,1): z = (sum_i (2 u_i + 1) - 8*65536) / 131072 over the
 * eight 16-bit halves u_i of Philox(counter = (n_lo, n_hi, 0, 0), key =
 * (seed, stream)).  The sum of eight U(0,1) has variance 8/12; the caller's
 * fp64 scale folds in sqrt(12/8) and the target standard deviation.  The
 * numerator is an integer below 2^20 in magnitude, so z is exact in fp64. */
MOEGEN_FN double moegen_irwin_hall8(uint64_t n, uint32_t seed, uint32_t stream) {
  moegen_u32x4 c;
  c.v[0] = (uint32_t)n;
  c.v[1] = (uint32_t)(n >> 32);
  c.v[2] = 0;
  c.v[3] = 0;
  moegen_u32x4 r = moegen_philox4x32_10(c, seed, stream);
  int32_t s = 0;
  for (int i = 0; i < 4; ++i) {
    s += 2 * (int32_t)(r.v[i] & 0xFFFFu) + 1;
    s += 2 * (int32_t)(r.v[i] >> 16) + 1;
  }
  s -= 8 * 65536;
  return (double)s * (1.0 / 131072.0);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs only). */
MOEGEN_FN uint16_t moegen_f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } b;
  b.f = f;
  uint32_t lsb = (b.u >> 16) & 1u;
  return (uint16_t)((b.u + 0x7FFFu + lsb) >> 16);
}

/* One generated element: fp64 product z*scale rounded once to fp32. */
MOEGEN_FN float moegen_value_f32(uint64_t n, uint32_t seed, uint32_t stream, double scale) {
  double z = moegen_irwin_hall8(n, seed, stream);
  return (float)(z * scale);
}

#endif
