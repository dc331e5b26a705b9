// Expert-grouped fp32 GEMMs on the vector ALUs (the MOE_F32 mode, used for
// small reference-precision layers).  Same contract as the bf16 kernels:
// C[rows of group g] = A[rows of g] . B[g]^T with K-contiguous operands, any
// N and K (edges masked).  64x64 tiles, each of the 256 threads computes a
// 4x4 patch; K streamed through LDS 16 at a time.  In gate/up mode a thread
// keeps the gate and the up patch of the same outputs and stores
// h = SiLU(G) * U.
#include "common.h"

namespace moe {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__global__ void __launch_bounds__(1024) f32_tile_prefix(const int32_t* __restrict__ row_off, int64_t M, int G,
                                                         int32_t* __restrict__ prefix) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int acc = 0;
    prefix[0] = 0;
    for (int g = 0; g < G; ++g) {
      int64_t rows = row_off ? (int64_t)(row_off[g + 1] - row_off[g]) : M;
      acc += (int)((rows + TM - 1) / TM);
      prefix[g + 1] = acc;
    }
  }
}

// ABS (router logits): each K step's 16 products are summed by fmaf into a
// fresh fp32 partial and the partials added in fp64 in K order; also the
// largest sum of |a_k| |b_k| of each row over the tile's columns, into
// rowabs[row * rowabs_stride] by atomic maximum.
template <int MODE, bool ABS = false>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const int32_t* __restrict__ a_rows,
                                                       int64_t lda, const int32_t* __restrict__ row_off, int64_t M,
                                                       int G, const float* __restrict__ B0,
                                                       const float* __restrict__ B1, int64_t bstride, int N, int K,
                                                       float* __restrict__ C, int64_t ldc,
                                                       const float* __restrict__ bias,
                                                       const int32_t* __restrict__ prefix, float* rowabs = nullptr,
                                                       int rowabs_stride = 0) {
  constexpr bool GU = MODE == GEMM_GATEUP;
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[GU ? 2 : 1][TK][TN + 1];
  const int mt = blockIdx.x;
  if (prefix && mt >= prefix[G]) return;
  int lo = 0, hi = G;
  if (prefix) {
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (prefix[mid] <= mt) lo = mid; else hi = mid;
    }
  }
  const int g = lo;
  const int64_t row_begin = prefix ? row_off[g] : 0;
  const int64_t n_g = prefix ? (int64_t)(row_off[g + 1] - row_off[g]) : M;
  const int64_t m0 = (int64_t)(mt - (prefix ? prefix[g] : 0)) * TM;
  const int n0 = blockIdx.y * TN;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[2][4][4] = {};
  float aab[4][4] = {};
  double acc64[ABS ? 4 : 1][4] = {};
  static_assert(TK == kLogitChunkF32, "logit chunk = K step");
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int i = threadIdx.x; i < TM * TK; i += 256) {
      int r = i / TK, kk = i % TK;
      int64_t lr = m0 + r;
      float v = 0.0f;
      if (lr < n_g && k0 + kk < K) {
        int64_t grow = row_begin + lr;
        int64_t src = a_rows ? (int64_t)a_rows[grow] : grow;
        v = A[src * lda + k0 + kk];
      }
      As[kk][r] = v;
    }
    for (int m = 0; m < (GU ? 2 : 1); ++m) {
      const float* Bm = (m == 0 ? B0 : B1) + (int64_t)g * bstride;
      for (int i = threadIdx.x; i < TN * TK; i += 256) {
        int n = i / TK, kk = i % TK;
        float v = 0.0f;
        if (n0 + n < N && k0 + kk < K) v = Bm[(int64_t)(n0 + n) * K + k0 + kk];
        Bs[m][kk][n] = v;
      }
    }
    __syncthreads();
    for (int kk = 0; kk < TK; ++kk) {
      float a[4];
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      for (int m = 0; m < (GU ? 2 : 1); ++m)
        for (int j = 0; j < 4; ++j) {
          float b = Bs[m][kk][tx * 4 + j];
          for (int i = 0; i < 4; ++i) acc[m][i][j] = fmaf(a[i], b, acc[m][i][j]);
          if (ABS)
            for (int i = 0; i < 4; ++i) aab[i][j] = fmaf(fabsf(a[i]), fabsf(b), aab[i][j]);
        }
    }
    if constexpr (ABS)
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
          acc64[i][j] += (double)acc[0][i][j];
          acc[0][i][j] = 0.0f;
        }
    __syncthreads();
  }
  if constexpr (ABS)
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j) acc[0][i][j] = (float)acc64[i][j];
  for (int i = 0; i < 4; ++i) {
    int64_t lr = m0 + ty * 4 + i;
    if (lr >= n_g) continue;
    int64_t grow = row_begin + lr;
    for (int j = 0; j < 4; ++j) {
      int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float v;
      if (GU) v = silu_f32(acc[0][i][j]) * acc[1][i][j];
      else v = acc[0][i][j] + (bias ? bias[col] : 0.0f);
      C[grow * ldc + col] = v;
    }
  }
  if (ABS) {
    for (int i = 0; i < 4; ++i) {
      int64_t lr = m0 + ty * 4 + i;
      if (lr >= n_g) continue;
      float mx = 0.0f;
      for (int j = 0; j < 4; ++j)
        if (n0 + tx * 4 + j < N) mx = fmaxf(mx, aab[i][j]);
      atomicMax(reinterpret_cast<unsigned int*>(rowabs + (row_begin + lr) * rowabs_stride), __float_as_uint(mx));
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmProblem& q, hipStream_t s) {
  // Upper bound of M tiles: ceil(total_rows / TM) + G (one partial tile per group).
  int64_t mt_ub = (q.M + TM - 1) / TM + (q.row_off ? q.G : 0);
  const int32_t* prefix = nullptr;
  if (q.row_off) {
    f32_tile_prefix<<<1, 64, 0, s>>>(q.row_off, q.M, q.G, q.tile_prefix);
    prefix = q.tile_prefix;
  }
  dim3 grid((unsigned)mt_ub, (unsigned)((q.N + TN - 1) / TN));
  const float* A = static_cast<const float*>(q.A);
  const float* B0 = static_cast<const float*>(q.B0);
  const float* B1 = static_cast<const float*>(q.B1);
  float* C = static_cast<float*>(q.C);
  if (mt_ub == 0) return hipGetLastError();
  if (q.mode == GEMM_GATEUP)
    gemm_f32_kernel<GEMM_GATEUP><<<grid, 256, 0, s>>>(A, q.a_rows, q.lda, q.row_off, q.M, q.G, B0, B1,
                                                      q.b_group_stride, q.N, q.K, C, q.ldc, q.bias, prefix);
  else if (q.rowabs)
    gemm_f32_kernel<GEMM_DOWN, true><<<grid, 256, 0, s>>>(A, q.a_rows, q.lda, q.row_off, q.M, q.G, B0, B1,
                                                          q.b_group_stride, q.N, q.K, C, q.ldc, q.bias, prefix,
                                                          q.rowabs, q.rowabs_stride);
  else
    gemm_f32_kernel<GEMM_DOWN><<<grid, 256, 0, s>>>(A, q.a_rows, q.lda, q.row_off, q.M, q.G, B0, B1,
                                                    q.b_group_stride, q.N, q.K, C, q.ldc, q.bias, prefix);
  return hipGetLastError();
}

}  // namespace moe
