// Expert-grouped bf16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// C[rows of group g][N] = A[rows of g][K] . B[g][N][K]^T, fp32 accumulation.
// Both operands are K-contiguous ("NT"), which is the layout of the token
// rows and of nn.Linear-style [out][in] weights.  The grouping follows the
// expert-contiguous rows of the schedule (Mixture-of-Kittens blog post,
// "Scheduling": tokens of an expert land in contiguous rows so the
// expert-grouped GEMMs start without reordering).
//
// Structure (one persistent grid, every workgroup loops over output tiles):
//  * Tiles are BM x BN; 4 waves of 64 lanes split the tile 2 x 2, each wave
//    owns (BM/2) x (BN/2) as a grid of 32x32 MFMA blocks.
//  * K is consumed BK at a time through two LDS buffers; the next slab is
//    fetched from global memory into registers while the MFMAs run on the
//    current one (one barrier per slab).  LDS rows are padded by 16 bytes so
//    the 16-byte fragment reads of 32 consecutive rows hit distinct banks.
//  * Tile order: an M-tile prefix over the groups (experts) is computed on
//    the device, so empty experts cost nothing and the host never learns the
//    counts.  Logical tiles are handed out so that each XCD (workgroup id
//    mod 8) owns a contiguous run, and runs walk GN N-tiles of one M-tile
//    before the next M-tile: neighbouring workgroups of an XCD share A and B
//    slabs in that XCD's L2.
//  * Gate/up mode: the B tile interleaves 32-row blocks of W_gate and W_up
//    for the same output columns, so a wave holds G and U of the same
//    elements and applies SwiGLU, h = SiLU(G) * U, in registers (blog post,
//    "Scheduling the overlaps": SwiGLU runs with the grouped GEMMs).
#include "common.h"

namespace moe {

namespace {

constexpr int kPad = 8;  // bf16 elements of padding per LDS row (16 bytes)

__global__ void __launch_bounds__(1024) tile_prefix_kernel(const int32_t* __restrict__ row_off, int64_t M, int G,
                                                            int BM, int32_t* __restrict__ prefix) {
  __shared__ int32_t s[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) {
    carry = 0;
    prefix[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < G; base += 1024) {
    int g = base + threadIdx.x;
    int n = 0;
    if (g < G) {
      int64_t rows = row_off ? (int64_t)(row_off[g + 1] - row_off[g]) : M;
      n = (int)((rows + BM - 1) / BM);
    }
    s[threadIdx.x] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int v = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
      __syncthreads();
      s[threadIdx.x] += v;
      __syncthreads();
    }
    if (g < G) prefix[g + 1] = carry + s[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 1023) carry += s[1023];
    __syncthreads();
  }
}

struct KArgs {
  const bf16_t* A;
  const int32_t* a_rows;
  int64_t lda;
  const int32_t* row_off;
  int64_t M;
  int G;
  const bf16_t* B0;
  const bf16_t* B1;
  int64_t b_group_stride;
  int N;
  int K;
  int ntiles;
  void* C;
  int64_t ldc;
  const float* bias;
  const int32_t* prefix;  // M-tile prefix per group, or nullptr: one group
  int single_mt;          // M tiles of the single group when prefix == nullptr
};

template <int BM, int BN, int BK, int MODE, int GN>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(KArgs p) {
  constexpr int NT = 256;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int LDS_K = BK + kPad;
  constexpr int KV = BK / 8;  // 16-byte vectors per row slab
  constexpr int A_VECS = BM * KV / NT;
  constexpr int B_VECS = BN * KV / NT;
  static_assert(A_VECS * NT == BM * KV && B_VECS * NT == BN * KV, "tile/thread mismatch");
  static_assert(MODE != GEMM_GATEUP || FN % 2 == 0, "gate/up needs G,U block pairs per wave");

  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM][LDS_K];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN][LDS_K];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int total_m = p.prefix ? p.prefix[p.G] : p.single_mt;
  const int total = total_m * p.ntiles;
  const int nwg = gridDim.x;
  const int per_xcd = nwg >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int KT = p.K / BK;

  for (int it = 0;; ++it) {
    const int L = it * nwg + xcd * per_xcd + slot;
    if (L >= total) break;
    // ---- decode the logical tile ----------------------------------------
    const int ng = L / (total_m * GN);
    const int r0 = L - ng * total_m * GN;
    const int gn = min(GN, p.ntiles - ng * GN);
    const int mt = r0 / gn;
    const int ntile = ng * GN + (r0 - mt * gn);
    int lo = 0, hi = p.G;  // largest g with prefix[g] <= mt
    if (p.prefix) {
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (p.prefix[mid] <= mt) lo = mid; else hi = mid;
      }
    }
    const int g = lo;
    const int64_t row_begin = p.prefix ? p.row_off[g] : 0;
    const int64_t n_g = p.prefix ? (int64_t)(p.row_off[g + 1] - p.row_off[g]) : p.M;
    const int64_t m0 = (int64_t)(mt - (p.prefix ? p.prefix[g] : 0)) * BM;

    // ---- per-thread global source pointers --------------------------------
    const bf16_t* pa[A_VECS];
    const bf16_t* pb[B_VECS];
#pragma unroll
    for (int i = 0; i < A_VECS; ++i) {
      int v = tid + i * NT;
      int row = v / KV, kc = (v % KV) * 8;
      int64_t lr = m0 + row;
      int64_t grow = row_begin + (lr < n_g ? lr : 0);
      int64_t src = p.a_rows ? (int64_t)p.a_rows[grow] : grow;
      pa[i] = p.A + src * p.lda + kc;
    }
#pragma unroll
    for (int i = 0; i < B_VECS; ++i) {
      int v = tid + i * NT;
      int n = v / KV, kc = (v % KV) * 8;
      const bf16_t* mat;
      int srow;
      if (MODE == GEMM_GATEUP) {
        int blk = n >> 5;
        mat = (blk & 1) ? p.B1 : p.B0;
        srow = ntile * (BN / 2) + (blk >> 1) * 32 + (n & 31);
      } else {
        mat = p.B0;
        srow = min(ntile * BN + n, p.N - 1);
      }
      pb[i] = mat + (int64_t)g * p.b_group_stride + (int64_t)srow * p.K + kc;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    u32x4 ra[A_VECS], rb[B_VECS];
    auto load_global = [&](int k0) {
#pragma unroll
      for (int i = 0; i < A_VECS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + k0);
#pragma unroll
      for (int i = 0; i < B_VECS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + k0);
    };
    auto store_lds = [&](int buf) {
#pragma unroll
      for (int i = 0; i < A_VECS; ++i) {
        int v = tid + i * NT;
        *reinterpret_cast<u32x4*>(&As[buf][v / KV][(v % KV) * 8]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_VECS; ++i) {
        int v = tid + i * NT;
        *reinterpret_cast<u32x4*>(&Bs[buf][v / KV][(v % KV) * 8]) = rb[i];
      }
    };

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) load_global((kt + 1) * BK);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[FM], bfr[FN];
        const int kof = kk * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * WM + i * 32 + (lane & 31)][kof]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * WN + j * 32 + (lane & 31)][kof]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) store_lds(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    // 32x32 block layout: lane holds column (lane & 31) and rows
    // 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t lr = m0 + rl;
        if (lr >= n_g) continue;
        const int64_t grow = row_begin + lr;
        if (MODE == GEMM_GATEUP) {
          bf16_t* C = static_cast<bf16_t*>(p.C);
#pragma unroll
          for (int q = 0; q < FN / 2; ++q) {
            float gv = acc[i][2 * q][v], uv = acc[i][2 * q + 1][v];
            int col = ntile * (BN / 2) + (wn * (FN / 2) + q) * 32 + (lane & 31);
            C[grow * p.ldc + col] = f32_to_bf16(silu_f32(gv) * uv);
          }
        } else if (MODE == GEMM_DOWN) {
          bf16_t* C = static_cast<bf16_t*>(p.C);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            int col = ntile * BN + wn * WN + j * 32 + (lane & 31);
            if (col < p.N) C[grow * p.ldc + col] = f32_to_bf16(acc[i][j][v]);
          }
        } else {
          float* C = static_cast<float*>(p.C);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            int col = ntile * BN + wn * WN + j * 32 + (lane & 31);
            if (col < p.N) C[grow * p.ldc + col] = acc[i][j][v] + (p.bias ? p.bias[col] : 0.0f);
          }
        }
      }
    }
  }
}

int num_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

template <int BM, int BN, int BK, int MODE, int GN>
hipError_t run(const GemmProblem& q, int occupancy, hipStream_t s) {
  KArgs a;
  a.A = static_cast<const bf16_t*>(q.A);
  a.a_rows = q.a_rows;
  a.lda = q.lda;
  a.row_off = q.row_off;
  a.M = q.M;
  a.G = q.G;
  a.B0 = static_cast<const bf16_t*>(q.B0);
  a.B1 = static_cast<const bf16_t*>(q.B1);
  a.b_group_stride = q.b_group_stride;
  a.N = q.N;
  a.K = q.K;
  a.ntiles = MODE == GEMM_GATEUP ? q.N / (BN / 2) : (q.N + BN - 1) / BN;
  a.C = q.C;
  a.ldc = q.ldc;
  a.bias = q.bias;
  if (q.row_off) {
    a.prefix = q.tile_prefix;
    a.single_mt = 0;
    tile_prefix_kernel<<<1, 1024, 0, s>>>(q.row_off, q.M, q.G, BM, q.tile_prefix);
  } else {
    a.prefix = nullptr;
    a.G = 1;
    a.single_mt = (int)((q.M + BM - 1) / BM);
  }
  int64_t wg = (int64_t)num_cus() * occupancy;
  wg = (wg + 7) / 8 * 8;
  gemm_bf16_kernel<BM, BN, BK, MODE, GN><<<(unsigned)wg, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmProblem& q, hipStream_t s) {
  if (q.K % 64 != 0) return hipErrorInvalidValue;
  switch (q.mode) {
    case GEMM_GATEUP:
      if (q.N % 64 != 0) return hipErrorInvalidValue;
      return run<128, 128, 64, GEMM_GATEUP, 4>(q, 2, s);
    case GEMM_DOWN:
      if (q.N % 8 != 0) return hipErrorInvalidValue;
      return run<128, 128, 64, GEMM_DOWN, 4>(q, 2, s);
    default:
      return run<64, 64, 64, GEMM_PLAIN_F32OUT, 4>(q, 4, s);
  }
}

}  // namespace moe
