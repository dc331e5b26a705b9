// The matrix-core operations under the grouped GEMMs and the router GEMM,
// one per tile, so that the instructions' own arithmetic, which every GEMM
// here inherits, can be measured and tested on the device.
//
// MXFP8 (Mixture-of-Kittens blog post, "Other features / MXFP8 support": the
// routed experts' GEMMs take E4M3 operands with one E8M0 scale per 32
// elements along K, OCP MX v1.0): one v_mfma_scale_f32_32x32x64_f8f6f4 per
// 32x32x64 tile, placed as csrc/gemm_mxfp8.hip places it: lane l = 32 g + r
// feeds row r of A (and of B) with K[16g, 16g+16) in its low 16 bytes and
// K[32+16g, 32+16g+16) in its high 16 bytes, and the scale of row r's K
// block g.
//
// bf16 (the grouped GEMMs and the router logits of csrc/gemm_bf16.hip): one
// v_mfma_f32_32x32x16_bf16 per 32x32x16 tile; lane l = 32 g + r feeds row r
// with K[8g, 8g+8).
//
// In both, accumulator element v of lane l is row 4g + 8(v/4) + v%4, column
// r of the 32x32 result.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(64) void mx_mma_tiles_kernel(const uint8_t* __restrict__ a,
                                                          const uint8_t* __restrict__ a_scale,
                                                          const uint8_t* __restrict__ b,
                                                          const uint8_t* __restrict__ b_scale,
                                                          const float* __restrict__ c, float* __restrict__ d) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
  const uint8_t* ar = a + (t * 32 + r) * 64;
  const uint8_t* br = b + (t * 32 + r) * 64;
  const u32x4 alo = *reinterpret_cast<const u32x4*>(ar + 16 * g);
  const u32x4 ahi = *reinterpret_cast<const u32x4*>(ar + 32 + 16 * g);
  const u32x4 blo = *reinterpret_cast<const u32x4*>(br + 16 * g);
  const u32x4 bhi = *reinterpret_cast<const u32x4*>(br + 32 + 16 * g);
  const i32x8 fa{(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
  const i32x8 fb{(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3], (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
  const float* ct = c + t * 1024 + (4 * g) * 32 + r;
  float* dt = d + t * 1024 + (4 * g) * 32 + r;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = ct[(8 * (v >> 2) + (v & 3)) * 32];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, a_scale[(t * 32 + r) * 2 + g], 0,
                                                        b_scale[(t * 32 + r) * 2 + g]);
#pragma unroll
  for (int v = 0; v < 16; ++v) dt[(8 * (v >> 2) + (v & 3)) * 32] = acc[v];
}

__global__ __launch_bounds__(64) void bf16_mma_tiles_kernel(const bf16_t* __restrict__ a,
                                                            const bf16_t* __restrict__ b,
                                                            const float* __restrict__ c, float* __restrict__ d) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
  const bf16x8 fa = *reinterpret_cast<const bf16x8*>(a + (t * 32 + r) * 16 + 8 * g);
  const bf16x8 fb = *reinterpret_cast<const bf16x8*>(b + (t * 32 + r) * 16 + 8 * g);
  const float* ct = c + t * 1024 + (4 * g) * 32 + r;
  float* dt = d + t * 1024 + (4 * g) * 32 + r;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = ct[(8 * (v >> 2) + (v & 3)) * 32];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
#pragma unroll
  for (int v = 0; v < 16; ++v) dt[(8 * (v >> 2) + (v & 3)) * 32] = acc[v];
}

}  // namespace

hipError_t launch_bf16_mma_tiles(const bf16_t* a, const bf16_t* b, const float* c, float* d, int64_t n,
                                 hipStream_t s) {
  if (n < 0 || n > INT32_MAX) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  bf16_mma_tiles_kernel<<<(unsigned)n, 64, 0, s>>>(a, b, c, d);
  return hipGetLastError();
}

hipError_t launch_mx_mma_tiles(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, const uint8_t* b_scale,
                               const float* c, float* d, int64_t n, hipStream_t s) {
  if (n < 0 || n > INT32_MAX) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  mx_mma_tiles_kernel<<<(unsigned)n, 64, 0, s>>>(a, a_scale, b, b_scale, c, d);
  return hipGetLastError();
}

}  // namespace moe
