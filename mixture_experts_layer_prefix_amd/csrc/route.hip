// Router: projection logits, top-k selection with normalized weights.
//
// Mixture-of-Kittens blog post, "Overlapping computation and communication
// in MoE": a router projection selects the top-k routed experts of a token
// and a router weight for each; paper summary section 2.1: the weights are
// normalized over the selected experts (softmax of the selected logits).
//
// The logits are a GEMM with fp32 accumulation (MFMA in bf16, FMA in fp32)
// followed by the top-k kernel: one wavefront per token, ceil(E/64) logits
// per lane, rounds of a wave-wide arg-max (larger value, then smaller id).
//
// Exact selection.  Each logit is an fp64 sum, in K order, of fp32 partial
// sums of c consecutive products (c = 64 on the bf16 path, the K slab of the
// matrix-core GEMM; 16 on the fp32 path), rounded once to fp32, plus the
// fp32 bias.  A partial of c products accumulated in fp32 lies within
// gamma_c * sum |x_i w_i| of its exact value, gamma_c = c u / (1 - c u),
// u = 2^-24 (Higham, "Accuracy and Stability of Numerical Algorithms", 2nd
// ed., section 3.1), taken twice over.  The bf16 matrix cores are not plain
// fp32 adders: each half of a v_mfma_f32_32x32x16_bf16 aligns its accumulator
// and eight products to the largest of them, cuts each at 2^-24 of it toward
// zero and rounds the step to fp32 (measured on the device, where the tile
// tests hold it), so a step errs by at most 9u of its largest term plus u of
// its sum: at most 80u sum |x_i w_i| over a 64-product partial, inside the
// 2 gamma_64 sum |x_i w_i| allowed.  The fp64 sum of the partials, and the
// fp64 recomputation below, add at most 4 d 2^-53 sum |x_i w_i|.  The logits
// GEMM also accumulates sum_i |x_i||w_i| in the matrix cores and keeps, per
// token, its largest value A over the experts (non-negative terms, so each
// step underestimates by at most 10u of the running sum: the true maximum is
// at most A / (1 - 2 gamma_d), d/8 steps of 10u being within 2 gamma_d).
// With the two fp32 roundings (before and after the
// bias) on either side, every GPU logit lies within
//   delta = gamma A + 4u (|l_k| + |l_k+1|) + eta
// of the logit recomputed in fp64, gamma = (2 gamma_c + 2u + 4 d 2^-53) /
// (1 - 2 gamma_d) and eta = d 2^-124 for products below the fp32 normal
// range that may be flushed (operands in the bf16 subnormal range are
// outside this statement).  When the k-th and (k+1)-th GPU logits are more
// than 2 delta apart, the selection is the one on the recomputed logits.
// Otherwise every expert whose GPU logit lies in [l_k+1 - 2 delta, l_k +
// 2 delta] gets its logit recomputed as an fp64 dot product rounded once to
// fp32 (plus the fp32 bias) and the selection is redone: experts above that
// window are in the top-k and experts below it are out under any error of
// that size.  The fp64 recomputation is the oracle's definition of a logit
// (an fp64 product rounded to fp32, plus the bias) up to the order of the
// fp64 additions.
#include <math.h>

#include "common.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;

__device__ __forceinline__ void better(float& bv, int& bid, float ov, int oid) {
  if (ov > bv || (ov == bv && oid < bid)) {
    bv = ov;
    bid = oid;
  }
}

// Key whose unsigned order is the order of the (finite) logits; -0 and +0
// share a key so that, as in a float comparison, they tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// `rounds` rounds of a wave-wide arg-max over the not yet taken logits:
// each lane's best candidate (larger value, then smaller id), the wave
// maximum of their keys in DPP steps, then among the lanes holding that
// value the smallest id (the lane of an id is id mod 64).
template <int PER_LANE>
__device__ __forceinline__ void select_rounds(const float (&v)[PER_LANE], int E, int rounds, int lane, float (&sel_v)[kMaxK + 1],
                                              int (&sel_id)[kMaxK + 1]) {
  uint32_t taken = 0;
#pragma unroll
  for (int r = 0; r < kMaxK + 1; ++r) {
    if (r >= rounds) continue;  // (not break: the loop unrolls, sel_v and sel_id stay in registers)
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) better(bv, bid, v[i], e);
    }
    const bool has = bid != 0x7fffffff;
    const uint32_t key = has ? order_key(bv) : 0u;
    const uint32_t h = half_max32_u(key);
    const uint32_t m = max((uint32_t)__builtin_amdgcn_readlane((int)h, 0), (uint32_t)__builtin_amdgcn_readlane((int)h, 32));
    uint64_t tie = __ballot(has && key == m);
    int id = __builtin_amdgcn_readlane(bid, __ffsll((unsigned long long)tie) - 1);
    tie &= tie - 1;
    while (tie) {  // equal values in several lanes: the smallest id
      id = min(id, __builtin_amdgcn_readlane(bid, __ffsll((unsigned long long)tie) - 1));
      tie &= tie - 1;
    }
    sel_v[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), id & 63));
    sel_id[r] = id;
    if ((id & 63) == lane) taken |= 1u << (id >> 6);
  }
}

// Eight consecutive elements starting at i (i a multiple of 8), widened to fp64.
__device__ __forceinline__ void load8_f64(const void* p, int64_t i, bool f32, double (&v)[8]) {
  if (f32) {
    const f32x4* q = reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    f32x4 a = q[0], b = q[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  } else {
    u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(p) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <int PER_LANE>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, const void* __restrict__ x,
                                                   const void* __restrict__ wr, const float* __restrict__ bias,
                                                   bool act_f32, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, int64_t T, int d, int E, int k,
                                                   float gamma, float eta) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront leaves; no block barrier below
  // max_e sum_i |x_ti| |W_r[e][i]| left by the logits kernel in this token's
  // first topk_w slot (read before this wave writes its weights there)
  const float abs_sum = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                      __builtin_bit_cast(int, topk_w[t * k])));
  float v[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? logits[t * E + e] : -INFINITY;
  }
  const int rounds = k < E ? k + 1 : k;
  float lv[kMaxK + 1];
  int lid[kMaxK + 1];
  select_rounds<PER_LANE>(v, E, rounds, lane, lv, lid);
  constexpr float u = 5.9604645e-8f;  // 2^-24
  // (1 + 2^-20): the few fp32 roundings of this expression
  const float delta = (gamma * abs_sum + 4.0f * u * (fabsf(lv[k - 1]) + (k < E ? fabsf(lv[k]) : 0.0f)) + eta) *
                      (1.0f + 9.5367432e-7f);
  if (k < E && lv[k - 1] - lv[k] <= 2.0f * delta) {
    // Near tie at the selection boundary.  Experts above hi are in the top-k
    // under any logit error up to delta (fewer than k GPU logits exceed the
    // k-th largest); experts below lo are out (at least k+1 lie above them).
    // Only the ones in between get exact logits before the selection is
    // redone.
    const float lo = lv[k] - 2.0f * delta, hi = lv[k - 1] + 2.0f * delta;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      int e0 = 64 * i;
      uint64_t mask = __ballot(lane + e0 < E && v[i] >= lo && v[i] <= hi);
      while (mask) {
        int b = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        int e = e0 + b;
        double acc = 0.0;
        // 8 consecutive elements per lane per step (d is a multiple of 8),
        // added in ascending order; bf16 rows: four steps' loads in flight.
        if (act_f32) {
#pragma unroll 1
          for (int c = lane * 8; c < d; c += 512) {
            double xv[8], wv[8];
            load8_f64(x, t * (int64_t)d + c, true, xv);
            load8_f64(wr, (int64_t)e * d + c, true, wv);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += xv[q] * wv[q];
          }
        } else {
          constexpr int U = 4;
          const bf16_t* xb = static_cast<const bf16_t*>(x) + t * (int64_t)d;
          const bf16_t* wb = static_cast<const bf16_t*>(wr) + (int64_t)e * d;
#pragma unroll 1
          for (int c0 = lane * 8; c0 < d; c0 += U * 512) {
            u32x4 xr[U], wq[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const int c = c0 + u * 512;
              if (c < d) {
                xr[u] = *reinterpret_cast<const u32x4*>(xb + c);
                wq[u] = *reinterpret_cast<const u32x4*>(wb + c);
              }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
              if (c0 + u * 512 >= d) break;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                acc += (double)__uint_as_float(xr[u][j] << 16) * (double)__uint_as_float(wq[u][j] << 16);
                acc += (double)__uint_as_float(xr[u][j] & 0xFFFF0000u) * (double)__uint_as_float(wq[u][j] & 0xFFFF0000u);
              }
            }
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        float ex = (float)acc;
        if (bias) ex = ex + bias[e];
        if (lane == b) v[i] = ex;
      }
    }
    select_rounds<PER_LANE>(v, E, k, lane, lv, lid);
  }
  // Normalized weights over the selected logits, summed in selection order.
  const float m = lv[0];
  float ex[kMaxK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      ex[j] = expf(lv[j] - m);
      sum += ex[j];
    }
  }
  // Lane j writes the j-th selected expert at its ascending-id position.
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k && lane == j) {
      int rank = 0;
#pragma unroll
      for (int q = 0; q < kMaxK; ++q)
        if (q < k && lid[q] < lid[j]) ++rank;
      topk_idx[t * k + rank] = lid[j];
      topk_w[t * k + rank] = ex[j] / sum;
    }
  }
}

}  // namespace

namespace {
// topk_w[t * k] = 0 for every token: the slot the logits kernel's |x||w|
// maximum accumulates into.
__global__ void __launch_bounds__(256) zero_slot_kernel(float* __restrict__ p, int64_t T, int k) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < T) p[t * k] = 0.0f;
}
}  // namespace

hipError_t launch_router_logits(bool act_f32, const void* x, const void* w_router, const float* bias,
                                float* logits, float* topk_w, int64_t T, int d, int E, int k, hipStream_t s) {
  GemmProblem q = {};
  q.mode = act_f32 ? GEMM_DOWN : GEMM_PLAIN_F32OUT;
  q.A = x;
  q.lda = d;
  q.M = T;
  q.G = 1;
  q.B0 = w_router;
  q.N = E;
  q.K = d;
  q.C = logits;
  q.ldc = E;
  q.bias = bias;
  q.rowabs = topk_w;
  q.rowabs_stride = k;
  if (T == 0) return hipSuccess;
  zero_slot_kernel<<<(unsigned)((T + 255) / 256), 256, 0, s>>>(topk_w, T, k);
  return act_f32 ? launch_gemm_f32(q, s) : launch_gemm_bf16(q, s);
}

hipError_t launch_topk(bool act_f32, const float* logits, const void* x, const void* w_router, const float* bias,
                       int32_t* topk_idx, float* topk_w, int64_t T, int d, int E, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4));
  const int per_lane = (E + 63) / 64;
  // the bound's coefficients (see the top of this file), rounded up
  const double u = 5.9604644775390625e-8, c = act_f32 ? kLogitChunkF32 : kLogitChunkBf16;
  const double gamma_c = c * u / (1.0 - c * u), gamma_d = d * u / (1.0 - d * u);
  const float gamma = (float)((2.0 * gamma_c + 2.0 * u + 4.0 * d * 0x1p-53) / (1.0 - 2.0 * gamma_d) * (1.0 + 0x1p-20));
  const float eta = (float)(d * 0x1p-124);
#define MOE_TOPK(P)                                                                                                \
  topk_kernel<P><<<grid, 256, 0, s>>>(logits, x, w_router, bias, act_f32, topk_idx, topk_w, T, d, E, k, gamma, eta); \
  break;
  switch (per_lane) {
    case 1: MOE_TOPK(1)
    case 2: MOE_TOPK(2)
    case 3: case 4: MOE_TOPK(4)
    case 5: case 6: case 7: case 8: MOE_TOPK(8)
    default: MOE_TOPK(16)
  }
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
