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
// One workgroup per token; each thread owns 16-byte vectors (8 bf16 or 4
// fp32 outputs) of the token's row and keeps their k row reads in flight;
// rows are read and written with 16-byte accesses.
#include <limits.h>

#include "common.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;

// One workgroup per token, sized so that each thread owns two 16-byte
// vectors of the row (the whole row for rows up to 2048 vectors; one vector
// for K > 12, whose 2K rows would spill): the token's K rows and router
// weights are workgroup-uniform (scalar loads, no per-thread index
// arithmetic) and 2K row loads are in flight per thread (K a template
// parameter: registers for exactly the token's routes).
template <bool F32, int K>
__global__ void __launch_bounds__(1024) combine_kernel(const void* __restrict__ o_perm, const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w, const void* __restrict__ y_shared,
                                                      void* __restrict__ y, int d) {
  constexpr int k = K;
  constexpr bool TWO = K <= 12;     // two vectors per thread while 2K rows fit in registers
  constexpr int EPV = F32 ? 4 : 8;  // elements per 16-byte vector
  const int vpr = d / EPV;
  const int64_t t = blockIdx.x;
  int64_t rows[K];
  float g[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = (int64_t)token_row[t * k + j] * vpr;
    g[j] = topk_w[t * k + j];
  }
  const u32x4* O = static_cast<const u32x4*>(o_perm);
  const u32x4* YS = y_shared ? static_cast<const u32x4*>(y_shared) + t * vpr : nullptr;
  u32x4* Y = static_cast<u32x4*>(y) + t * vpr;
  for (int v0 = threadIdx.x; v0 < vpr; v0 += (TWO ? 2 : 1) * blockDim.x) {
    const int v1 = v0 + blockDim.x;
    const bool two = TWO && v1 < vpr;
    float a0[8], a1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a0[i] = a1[i] = 0.0f;
    u32x4 w0[K], w1[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      w0[j] = __builtin_nontemporal_load(O + rows[j] + v0);
      w1[j] = two ? __builtin_nontemporal_load(O + rows[j] + v1) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[i] = fmaf(g[j], __uint_as_float(w0[j][i]), a0[i]);
          a1[i] = fmaf(g[j], __uint_as_float(w1[j][i]), a1[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[2 * i] = fmaf(g[j], __uint_as_float(w0[j][i] << 16), a0[2 * i]);
          a0[2 * i + 1] = fmaf(g[j], __uint_as_float(w0[j][i] & 0xFFFF0000u), a0[2 * i + 1]);
          a1[2 * i] = fmaf(g[j], __uint_as_float(w1[j][i] << 16), a1[2 * i]);
          a1[2 * i + 1] = fmaf(g[j], __uint_as_float(w1[j][i] & 0xFFFF0000u), a1[2 * i + 1]);
        }
      }
    }
    auto finish = [&](float (&a)[8], int v) {
      u32x4 o;
      if (F32) {
        if (YS) {
          const u32x4 ys = __builtin_nontemporal_load(YS + v);
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] += __uint_as_float(ys[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(a[i]);
      } else {
        if (YS) {
          const u32x4 ys = __builtin_nontemporal_load(YS + v);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[2 * i] += __uint_as_float(ys[i] << 16);
            a[2 * i + 1] += __uint_as_float(ys[i] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
      }
      __builtin_nontemporal_store(o, Y + v);
    };
    finish(a0, v0);
    if (two) finish(a1, v1);
  }
}

__global__ void __launch_bounds__(256) fill_zero_kernel(u32x4* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = u32x4{0, 0, 0, 0};
}

// The instantiation for the runtime k (1..kMaxK).
template <int K>
void launch_combine_k(bool act_f32, int k, const void* o_perm, const int32_t* token_row, const float* topk_w,
                      const void* y_shared, void* y, int64_t T, int d, hipStream_t s) {
  if constexpr (K <= kMaxK) {
    if (k != K) return launch_combine_k<K + 1>(act_f32, k, o_perm, token_row, topk_w, y_shared, y, T, d, s);
    const int vpr = d / (act_f32 ? 4 : 8), vpt = K <= 12 ? 2 : 1;
    int th = ((vpr + vpt - 1) / vpt + 63) / 64 * 64;
    th = th > 1024 ? 1024 : th;
    if (act_f32)
      combine_kernel<true, K><<<(unsigned)T, (unsigned)th, 0, s>>>(o_perm, token_row, topk_w, y_shared, y, d);
    else
      combine_kernel<false, K><<<(unsigned)T, (unsigned)th, 0, s>>>(o_perm, token_row, topk_w, y_shared, y, d);
  }
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
  if (d % (act_f32 ? 4 : 8) || k > kMaxK || T > INT32_MAX) return hipErrorInvalidValue;
  launch_combine_k<1>(act_f32, k, o_perm, token_row, topk_w, y_shared, y, T, d, s);
  return hipGetLastError();
}

}  // namespace moe
