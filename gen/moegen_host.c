/* Host side of the seeded synthetic input generator (plain C, OpenMP).
 * Fills flat index ranges [start, start+count) of a tensor stream, so any
 * slice of a tensor can be regenerated without materialising the rest. */
#include <stdint.h>
#include <stddef.h>
#include "philox4x32.h"

void moegen_philox(const uint32_t ctr[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
  moegen_u32x4 c;
  for (int i = 0; i < 4; ++i) c.v[i] = ctr[i];
  moegen_u32x4 r = moegen_philox4x32_10(c, k0, k1);
  for (int i = 0; i < 4; ++i) out[i] = r.v[i];
}

void moegen_fill_f32(float* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream, double scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = moegen_value_f32(start + (uint64_t)i, seed, stream, scale);
}

void moegen_fill_bf16(uint16_t* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream, double scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = moegen_f32_to_bf16_rne(moegen_value_f32(start + (uint64_t)i, seed, stream, scale));
}

/* First 32-bit word of each Philox block: uniform integers for host-side draws. */
void moegen_fill_u32(uint32_t* out, uint64_t start, int64_t count, uint32_t seed, uint32_t stream) {
  for (int64_t i = 0; i < count; ++i) {
    uint64_t n = start + (uint64_t)i;
    moegen_u32x4 c;
    c.v[0] = (uint32_t)n; c.v[1] = (uint32_t)(n >> 32); c.v[2] = 0; c.v[3] = 0;
    out[i] = moegen_philox4x32_10(c, seed, stream).v[0];
  }
}
