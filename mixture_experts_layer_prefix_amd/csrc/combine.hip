// Weighted sum of the expert outputs back to token order.
//
// Mixture-of-Kittens blog post (footnote to "Overlapping computation and
// communication in MoE"): after the combine, a weighted reduction of the
// expert outputs with the router weights finishes the layer; the shared
// expert's output is added (paper summary, section 2.1).  Blog post,
// "Determinism": the floating-point order is fixed, so the result is
// bitwise reproducible.
//
// y[t] = sum_{j = 0..k-1} w[t][j] * o_perm[token_row[t][j]] + y_shared[t].
// The token's experts are stored in ascending id, so j ascending is the
// ascending-expert order.  fp32 accumulation, one rounding at the end.
// Each thread owns 8 consecutive output elements (one 16-byte bf16 vector)
// of one token and keeps its k row reads in flight; rows are read and
// written with 16-byte accesses.
#include "common.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;

template <bool F32>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ o_perm, const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w, const void* __restrict__ y_shared,
                                                      void* __restrict__ y, int64_t T, int d, int k) {
  const int vpr = d / 8;  // 8-element vectors per row
  const int64_t nvec = T * vpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t t = v / vpr;
    const int c = (int)(v - t * vpr) * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int64_t row = token_row[t * k + j];
      const float g = topk_w[t * k + j];
      if (F32) {
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(o_perm) + row * d + c);
        f32x4 a = src[0], b = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = fmaf(g, a[i], acc[i]);
          acc[4 + i] = fmaf(g, b[i], acc[4 + i]);
        }
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(o_perm) + row * d + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(g, __uint_as_float(w[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(g, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    }
    if (F32) {
      float* out = static_cast<float*>(y) + t * d + c;
      if (y_shared) {
        const f32x4* ys = reinterpret_cast<const f32x4*>(static_cast<const float*>(y_shared) + t * d + c);
        f32x4 a = ys[0], b = ys[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += a[i];
          acc[4 + i] += b[i];
        }
      }
      reinterpret_cast<f32x4*>(out)[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      reinterpret_cast<f32x4*>(out)[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      if (y_shared) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(y_shared) + t * d + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += __uint_as_float(w[i] << 16);
          acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
        }
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(y) + t * d + c) = o;
    }
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(u32x4* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = u32x4{0, 0, 0, 0};
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  if (p == nullptr) return hipErrorInvalidValue;
  int64_t g = (n + 255) / 256;
  if (g > 8192) g = 8192;
  fill_zero_kernel<<<(unsigned)g, 256, 0, s>>>(static_cast<u32x4*>(p), n);
  return hipGetLastError();
}

hipError_t launch_combine(bool act_f32, const void* o_perm, const int32_t* token_row, const float* topk_w,
                          const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t nvec = T * (d / 8);
  int64_t g = (nvec + 255) / 256;
  if (g > 16384) g = 16384;
  if (act_f32)
    combine_kernel<true><<<(unsigned)g, 256, 0, s>>>(o_perm, token_row, topk_w, y_shared, y, T, d, k);
  else
    combine_kernel<false><<<(unsigned)g, 256, 0, s>>>(o_perm, token_row, topk_w, y_shared, y, T, d, k);
  return hipGetLastError();
}

}  // namespace moe
