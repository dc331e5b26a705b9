// Memory-bound kernels of the layer backward.
//
// Mixture-of-Kittens blog post, "Scheduling overlap" (backward ordering):
// the output gradient is gathered back to the expert rows (reverse combine),
// the input-gradient GEMMs and the SwiGLU backward run per expert, the input
// gradients return to token order (reverse dispatch), and the weight
// gradients run last, each accumulated over an expert's whole token range.
// Blog post, "Router weight gradient computation": the gradient of a route's
// router weight is the inner product of the SwiGLU activation with the down
// projection's input gradient, taken inside the SwiGLU backward (the GEMM
// epilogue writes per-32-column partials; dg_kernel sums them).
//
// Kernels here:
//  - pad_offsets_kernel: expert K ranges of the weight-gradient GEMMs, each
//    expert's rows rounded up to a multiple of the K slab (64 rows in bf16,
//    128 in MXFP8; zero padded);
//  - row_weight_kernel: router weight of every routed row;
//  - dg_kernel: router-weight gradients, and the logit gradients through the
//    renormalized softmax when the router gradient is requested;
//  - transpose_rows_kernel: [rows][cols] -> [cols][padded rows], optionally
//    gathering rows (dispatch), in expert-padded column order;
//  - transpose_batched_kernel: weight transposes (prepared once per update);
//  - dx_kernel: token-order sum of the routed input gradients in ascending
//    expert order, plus the shared expert's and the router's terms;
//  - router_partial_kernel / router_reduce_kernel: W_router gradient as a
//    fixed-order two-level sum over each expert's rows.
//  - transpose_quant_kernel: the same transpose, quantized to MX along the
//    routed-row axis (the K axis of the MXFP8 weight-gradient GEMMs);
// Every reduction has a fixed order: results do not depend on scheduling.
#include "common.h"

namespace moe {

namespace {

constexpr int kMaxK = 16;
constexpr int kPadRows = 64;
constexpr int kTqChunks = 8;  // 64-column chunks per transpose-quantize workgroup
constexpr int kTrChunks = 8;  // 64-column chunks per bf16 transpose workgroup

__global__ void __launch_bounds__(1024) pad_offsets_kernel(const int32_t* __restrict__ counts, int E, int64_t T,
                                                           int pad, int32_t* __restrict__ pad_off,
                                                           int32_t* __restrict__ single_off) {
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  const int32_t c = e < E ? (counts[e] + pad - 1) / pad * pad : 0;
  s[e] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) pad_off[e + 1] = s[e];
  if (e == 0) {
    pad_off[0] = 0;
    single_off[0] = 0;
    single_off[1] = (int32_t)((T + pad - 1) / pad * pad);
    single_off[2] = 0;
    single_off[3] = (int32_t)T;
  }
}

__global__ void __launch_bounds__(256) row_weight_kernel(const int32_t* __restrict__ token_row,
                                                         const float* __restrict__ topk_w, int64_t R,
                                                         float* __restrict__ w_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < R) w_row[token_row[i]] = topk_w[i];
}

// One wave per token.  dg[t][j] = sum over the 32-column partials of the
// token's j-th row (lanes read partials, a fixed butterfly sums them).
// With the router gradient: dl_j = g_j (dg_j - sum_i g_i dg_i).
__global__ void __launch_bounds__(256) dg_kernel(const float* __restrict__ dg_part, int nparts,
                                                 const int32_t* __restrict__ token_row, const float* __restrict__ topk_w,
                                                 int64_t T, int k, float* __restrict__ dtopk_w, float* __restrict__ dl,
                                                 float* __restrict__ dl_row) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  float dg[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    dg[j] = 0.0f;
    if (j < k) {
      const int64_t row = token_row[t * k + j];
      float v = 0.0f;
      for (int c = lane; c < nparts; c += 64) v += dg_part[row * nparts + c];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      dg[j] = v;
    }
  }
  if (lane == 0) {
    float inner = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) {
        dtopk_w[t * k + j] = dg[j];
        inner = fmaf(topk_w[t * k + j], dg[j], inner);
      }
    if (dl) {
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) {
          const float v = topk_w[t * k + j] * (dg[j] - inner);
          dl[t * k + j] = v;
          dl_row[token_row[t * k + j]] = v;
        }
    }
  }
}

// Expert segment of padded column p0 (pad_off nondecreasing, p0 < pad_off[nseg]).
__device__ __forceinline__ int find_segment(const int32_t* pad_off, int nseg, int64_t p0) {
  int lo = 0, hi = nseg;  // invariant: pad_off[lo] <= p0 < pad_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pad_off[mid] <= p0) lo = mid; else hi = mid;
  }
  return lo;
}

// dst[c][p] = src[row(p)][c] for the 64x64 tile (p0.., c0..), where padded
// column p of segment e is row seg_off[e] + (p - pad_off[e]) (zero past the
// segment's rows) and row r reads source row gather[r] (or r).  The output is
// expert-blocked: segment e is a dense [cols][Kp_e] block at element
// pad_off[e] * cols, Kp_e = pad_off[e+1] - pad_off[e].
__global__ void __launch_bounds__(256) transpose_rows_kernel(const bf16_t* __restrict__ src, int64_t ld_src, int cols,
                                                             const int32_t* __restrict__ gather,
                                                             const int32_t* __restrict__ seg_off,
                                                             const int32_t* __restrict__ pad_off, int nseg,
                                                             bf16_t* __restrict__ dst) {
  __shared__ bf16_t tile[64][66];
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  if (p0 >= pad_off[nseg]) return;
  const int e = find_segment(pad_off, nseg, p0);
  const int64_t r0 = seg_off[e] + (p0 - pad_off[e]);
  const int64_t r_end = seg_off[e + 1];
  const int64_t kp = pad_off[e + 1] - pad_off[e];
  const int tid = threadIdx.x;
  const int ch = tid & 7;
  // This thread's two source rows, shared by the workgroup's column chunks.
  int64_t srow[2];
  bool rok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t r = r0 + (tid >> 3) + 32 * h;
    rok[h] = r < r_end;
    srow[h] = rok[h] ? (gather ? (int64_t)gather[r] : r) : 0;
  }
  auto load = [&](int cc0, u32x4 (&v)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v[h] = u32x4{0, 0, 0, 0};
      if (rok[h] && cc0 + ch * 8 < cols) v[h] = *reinterpret_cast<const u32x4*>(src + srow[h] * ld_src + cc0 + ch * 8);
    }
  };
  const int cbase = blockIdx.y * 64 * kTrChunks;
  u32x4 v[2];
  load(cbase, v);
  for (int k = 0; k < kTrChunks; ++k) {
    const int c0 = cbase + k * 64;
    if (c0 >= cols) break;
    if (k) __syncthreads();  // the previous chunk's columns have been read
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (tid >> 3) + 32 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        tile[i][ch * 8 + 2 * q] = (bf16_t)(v[h][q] & 0xFFFFu);
        tile[i][ch * 8 + 2 * q + 1] = (bf16_t)(v[h][q] >> 16);
      }
    }
    if (k + 1 < kTrChunks && c0 + 64 < cols) load(c0 + 64, v);  // the next chunk's rows in flight
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (tid >> 3) + 32 * h;
      if (c0 + c >= cols) continue;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)tile[ch * 8 + 2 * q][c] | ((uint32_t)tile[ch * 8 + 2 * q + 1][c] << 16);
      *reinterpret_cast<u32x4*>(dst + (int64_t)pad_off[e] * cols + (int64_t)(c0 + c) * kp + (p0 - pad_off[e]) +
                                ch * 8) = o;
    }
  }
}

// As transpose_rows_kernel, with the output quantized to MX E4M3 along its
// rows (blocks of 32 consecutive padded positions p, i.e. 32 consecutive
// routed rows of one expert; zero padding quantizes to zero codes), and
// stored expert-blocked: segment e is a dense [cols][Kp_e] block at byte
// pad_off[e] * cols (Kp_e = pad_off[e+1] - pad_off[e]).  Its scales are
// slab-major, a [Kp_e / 128][cols][4] block at pad_off[e] * cols / 32: the
// four E8M0 bytes of one column and one 128-position slab are one dword, and
// a slab's dwords are contiguous over the columns (the weight-gradient GEMM
// reads one slab's scales of 256 rows as 1 KB).  One workgroup
// transposes 128 positions x 64 columns (segments are whole multiples of 128
// positions); each thread quantizes one 32-position block of one column, and
// the codes go back through LDS so that every output row piece (one column's
// 128 positions, a whole cache line) leaves as 8 lanes x 16 bytes.
__global__ void __launch_bounds__(256) transpose_quant_kernel(const bf16_t* __restrict__ src, int64_t ld_src, int cols,
                                                              const int32_t* __restrict__ gather,
                                                              const int32_t* __restrict__ seg_off,
                                                              const int32_t* __restrict__ pad_off, int nseg,
                                                              uint8_t* __restrict__ dst,
                                                              uint8_t* __restrict__ dst_scale) {
  constexpr int TP = 128, TC = 64, LDT = TC + 8;  // LDS rows of 144 bytes: 16-byte aligned
  __shared__ __attribute__((aligned(16))) bf16_t tile[TP][LDT];
  // After the quantization the same LDS holds the codes, [column][8 x 16 bytes],
  // and the scales, [column][4].
  u32x4(*codes)[8] = reinterpret_cast<u32x4(*)[8]>(&tile[0][0]);
  uint32_t* scales = reinterpret_cast<uint32_t*>(&tile[0][0]) + TC * 8 * 4;
  static_assert(TC * 8 * 16 + TC * 4 <= TP * LDT * 2, "codes fit the tile");
  const int64_t p0 = (int64_t)blockIdx.x * TP;
  if (p0 >= pad_off[nseg]) return;
  const int e = find_segment(pad_off, nseg, p0);
  const int64_t r0 = seg_off[e] + (p0 - pad_off[e]);
  const int64_t r_end = seg_off[e + 1];
  const int tid = threadIdx.x;
  const int ch = tid & 7;
  // This thread's four source rows, shared by the workgroup's column chunks.
  int64_t srow[TP / 32];
  bool rok[TP / 32];
#pragma unroll
  for (int h = 0; h < TP / 32; ++h) {
    const int64_t r = r0 + (tid >> 3) + 32 * h;
    rok[h] = r < r_end;
    srow[h] = rok[h] ? (gather ? (int64_t)gather[r] : r) : 0;
  }
  auto load = [&](int cc0, u32x4 (&v)[TP / 32]) {
#pragma unroll
    for (int h = 0; h < TP / 32; ++h) {
      v[h] = u32x4{0, 0, 0, 0};
      if (rok[h] && cc0 + ch * 8 < cols) v[h] = *reinterpret_cast<const u32x4*>(src + srow[h] * ld_src + cc0 + ch * 8);
    }
  };
  const int64_t kp = pad_off[e + 1] - pad_off[e];
  const int64_t base = (int64_t)pad_off[e] * cols + (p0 - pad_off[e]);
  uint32_t* sdst = reinterpret_cast<uint32_t*>(dst_scale + (int64_t)pad_off[e] * cols / 32) +
                   (p0 - pad_off[e]) / TP * cols;
  const int cbase = blockIdx.y * TC * kTqChunks;
  u32x4 v[TP / 32];
  load(cbase, v);
  for (int k = 0; k < kTqChunks; ++k) {
    const int c0 = cbase + k * TC;
    if (c0 >= cols) break;
    if (k) __syncthreads();  // the previous chunk's codes have left the LDS
#pragma unroll
    for (int h = 0; h < TP / 32; ++h) *reinterpret_cast<u32x4*>(&tile[(tid >> 3) + 32 * h][ch * 8]) = v[h];
    if (k + 1 < kTqChunks && c0 + TC < cols) load(c0 + TC, v);  // the next chunk's rows in flight
    __syncthreads();
    const int c = tid & (TC - 1), blk = tid / TC;
    float f[32];
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      f[q] = bf16_to_f32(tile[blk * 32 + q][c]);
      amax = fmaxf(amax, fabsf(f[q]));
    }
    const int ex = mx_block_exp(amax);
    const float inv = mx_inv_scale(ex);
    u32x4 w[2];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q >> 2][q & 3] = e4m3x4_rne_sat(f[4 * q] * inv, f[4 * q + 1] * inv, f[4 * q + 2] * inv, f[4 * q + 3] * inv);
    __syncthreads();  // every thread has read its tile column
    codes[c][blk * 2] = w[0];
    codes[c][blk * 2 + 1] = w[1];
    reinterpret_cast<uint8_t*>(scales)[c * 4 + blk] = (uint8_t)(ex + 127);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int q = tid + 256 * it, cc = q >> 3, part = q & 7;
      if (c0 + cc < cols) {
        const int64_t off = base + (int64_t)(c0 + cc) * kp;
        *reinterpret_cast<u32x4*>(dst + off + part * 16) = codes[cc][part];
      }
    }
    if (tid < TC && c0 + tid < cols) sdst[c0 + tid] = scales[tid];
  }
}

// dst[b][c][r] = src[b][r][c], element-wise bounds (any rows, cols).
__global__ void __launch_bounds__(256) transpose_batched_kernel(const bf16_t* __restrict__ src, int64_t rows,
                                                                int64_t cols, bf16_t* __restrict__ dst) {
  __shared__ bf16_t tile[64][65];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const bf16_t* s = src + b * rows * cols;
  bf16_t* d = dst + b * rows * cols;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = s[r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) d[c * rows + r] = tile[tx][i];
  }
}

// dx[t] = sum_j dA_perm[token_row[t][j]] + sum_j dl[t][j] W_r[idx[t][j]]
//         + dx_shared[t]
// (j ascending = ascending expert id), fp32 accumulation, one bf16 rounding.
// One workgroup per token, sized so that each thread owns two 16-byte
// vectors of the row (one for k > 8, whose rows and router rows would
// spill; the whole row for rows up to 1024 vectors): the token's k rows,
// expert ids and logit gradients are workgroup-uniform, and the 2k row
// reads of a thread are in flight together (k a template parameter).  Per
// element: the k dA_perm rows are added, then the k router terms
// (ROUTER), then the shared expert's dX.  The routed rows and the shared
// dX stream (nontemporal); W_router rows are reread by every token and
// stay cached.
// 16-byte vectors per thread: two while 2k rows stay in registers.
constexpr int dx_vectors_per_thread(int k) { return k <= 8 ? 2 : 1; }

template <int K, bool ROUTER>
__global__ void __launch_bounds__(512) dx_kernel(const bf16_t* __restrict__ da_perm, const int32_t* __restrict__ token_row,
                                                  const int32_t* __restrict__ topk_idx, const float* __restrict__ dl,
                                                  const bf16_t* __restrict__ w_router,
                                                  const bf16_t* __restrict__ dx_shared, bf16_t* __restrict__ dx, int d) {
  constexpr bool TWO = dx_vectors_per_thread(K) == 2;
  const int vpr = d / 8;
  const int64_t t = blockIdx.x;
  int64_t rows[K], er[K];
  float g[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = (int64_t)token_row[t * K + j] * vpr;
    er[j] = ROUTER ? (int64_t)topk_idx[t * K + j] * vpr : 0;
    g[j] = ROUTER ? dl[t * K + j] : 0.0f;
  }
  const u32x4* A = reinterpret_cast<const u32x4*>(da_perm);
  const u32x4* WR = reinterpret_cast<const u32x4*>(w_router);
  const u32x4* XS = dx_shared ? reinterpret_cast<const u32x4*>(dx_shared) + t * vpr : nullptr;
  u32x4* Y = reinterpret_cast<u32x4*>(dx) + t * vpr;
  auto add_bf16 = [](float (&a)[8], const u32x4& w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] += __uint_as_float(w[i] << 16);
      a[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  };
  auto fma_bf16 = [](float (&a)[8], float s, const u32x4& w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = fmaf(s, __uint_as_float(w[i] << 16), a[2 * i]);
      a[2 * i + 1] = fmaf(s, __uint_as_float(w[i] & 0xFFFF0000u), a[2 * i + 1]);
    }
  };
  for (int v0 = threadIdx.x; v0 < vpr; v0 += (TWO ? 2 : 1) * blockDim.x) {
    const int v1 = v0 + blockDim.x;
    const bool two = TWO && v1 < vpr;
    float a0[8], a1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a0[i] = a1[i] = 0.0f;
    u32x4 w0[K], w1[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      w0[j] = __builtin_nontemporal_load(A + rows[j] + v0);
      w1[j] = two ? __builtin_nontemporal_load(A + rows[j] + v1) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      add_bf16(a0, w0[j]);
      add_bf16(a1, w1[j]);
    }
    if (ROUTER) {
      // The router rows are loaded once the routed rows' registers are
      // free (the empty asm pins the sums above it and, as a memory
      // clobber, the router loads below it), so the two sets of 2k vectors
      // are never live together.
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(a0[i]), "+v"(a1[i])::"memory");
      u32x4 r0[K], r1[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        r0[j] = WR[er[j] + v0];
        r1[j] = two ? WR[er[j] + v1] : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        fma_bf16(a0, g[j], r0[j]);
        fma_bf16(a1, g[j], r1[j]);
      }
    }
    auto finish = [&](float (&a)[8], int v) {
      if (XS) add_bf16(a, __builtin_nontemporal_load(XS + v));
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
      __builtin_nontemporal_store(o, Y + v);
    };
    finish(a0, v0);
    if (two) finish(a1, v1);
  }
}

// The instantiation for the runtime k (1..kMaxK).
template <int K>
void launch_dx_k(int k, const bf16_t* da_perm, const int32_t* token_row, const int32_t* topk_idx, const float* dl,
                 const bf16_t* w_router, const bf16_t* dx_shared, bf16_t* dx, int64_t T, int d, hipStream_t s) {
  if constexpr (K <= kMaxK) {
    if (k != K) return launch_dx_k<K + 1>(k, da_perm, token_row, topk_idx, dl, w_router, dx_shared, dx, T, d, s);
    const int vpr = d / 8, vpt = dx_vectors_per_thread(K);
    int th = ((vpr + vpt - 1) / vpt + 63) / 64 * 64;
    th = th > 512 ? 512 : th;
    if (dl)
      dx_kernel<K, true><<<(unsigned)T, (unsigned)th, 0, s>>>(da_perm, token_row, topk_idx, dl, w_router, dx_shared,
                                                             dx, d);
    else
      dx_kernel<K, false><<<(unsigned)T, (unsigned)th, 0, s>>>(da_perm, token_row, topk_idx, dl, w_router,
                                                              dx_shared, dx, d);
  }
}

// partial[q][c] = sum over the rows of padded chunk q (64 positions inside
// one expert's padded range) of dl_row[r] * x[row_token[r]][c], rows ascending.
__global__ void __launch_bounds__(256) router_partial_kernel(const bf16_t* __restrict__ x,
                                                             const int32_t* __restrict__ row_token,
                                                             const float* __restrict__ dl_row,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ pad_off, int E, int d,
                                                             float* __restrict__ partial) {
  const int64_t q = blockIdx.x;
  const int64_t p0 = q * kPadRows;
  if (p0 >= pad_off[E]) return;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  const int e = find_segment(pad_off, E, p0);
  const int64_t r0 = offsets[e] + (p0 - pad_off[e]);
  const int64_t r1 = min(r0 + kPadRows, (int64_t)offsets[e + 1]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    const float g = dl_row[r];
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + (int64_t)row_token[r] * d + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(g, __uint_as_float(w[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
  }
  f32x4* out = reinterpret_cast<f32x4*>(partial + q * d + c);
  out[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  out[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// dW_router[e][c] = sum of expert e's chunk partials (0 when empty) in a
// fixed order: lane l of a column's 8 lanes sums chunks l, l + 8, l + 16, ...
// in ascending order, then the 8 lane sums are added in lane order.  One
// workgroup covers 32 columns of one expert, so the long chunk lists of the
// busiest experts are read by 8 lanes at once.
__global__ void __launch_bounds__(256) router_reduce_kernel(const float* __restrict__ partial,
                                                            const int32_t* __restrict__ pad_off, int E, int d,
                                                            float* __restrict__ dw) {
  __shared__ float part[8][33];
  const int e = blockIdx.y;
  const int cl = threadIdx.x & 31, l = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + cl;
  const int q0 = pad_off[e] / kPadRows, q1 = pad_off[e + 1] / kPadRows;
  float acc = 0.0f;
  if (c < d)
    for (int q = q0 + l; q < q1; q += 8) acc += partial[(int64_t)q * d + c];
  part[l][cl] = acc;
  __syncthreads();
  if (l == 0 && c < d) {
    float s = part[0][cl];
#pragma unroll
    for (int m = 1; m < 8; ++m) s += part[m][cl];
    dw[(int64_t)e * d + c] = s;
  }
}

unsigned grid_for(int64_t work, int64_t cap) {
  int64_t g = (work + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

int64_t bwd_padded_rows(int64_t rows, int groups, int pad) {
  return (rows + pad - 1) / pad * pad + (int64_t)pad * groups;
}

hipError_t launch_pad_offsets(const int32_t* counts, int E, int64_t T, int pad, int32_t* pad_off, int32_t* single_off,
                              hipStream_t s) {
  if (pad % kPadRows) return hipErrorInvalidValue;
  pad_offsets_kernel<<<1, 1024, 0, s>>>(counts, E, T, pad, pad_off, single_off);
  return hipGetLastError();
}

hipError_t launch_transpose_quant(const bf16_t* src, int64_t ld_src, int cols, const int32_t* gather,
                                  const int32_t* seg_off, const int32_t* pad_off, int nseg, int64_t p_cap,
                                  uint8_t* dst, uint8_t* dst_scale, hipStream_t s) {
  if (p_cap == 0 || cols == 0) return hipSuccess;
  if (p_cap % 128 || ld_src % 8 || cols % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p_cap / 128), (unsigned)((cols + 64 * kTqChunks - 1) / (64 * kTqChunks)));
  transpose_quant_kernel<<<grid, 256, 0, s>>>(src, ld_src, cols, gather, seg_off, pad_off, nseg, dst, dst_scale);
  return hipGetLastError();
}

hipError_t launch_row_weight(const int32_t* token_row, const float* topk_w, int64_t R, float* w_row, hipStream_t s) {
  if (R == 0) return hipSuccess;
  row_weight_kernel<<<(unsigned)((R + 255) / 256), 256, 0, s>>>(token_row, topk_w, R, w_row);
  return hipGetLastError();
}

hipError_t launch_dg(const float* dg_part, int nparts, const int32_t* token_row, const float* topk_w, int64_t T, int k,
                     float* dtopk_w, float* dl, float* dl_row, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dg_kernel<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(dg_part, nparts, token_row, topk_w, T, k, dtopk_w, dl, dl_row);
  return hipGetLastError();
}

hipError_t launch_transpose_rows(const bf16_t* src, int64_t ld_src, int cols, const int32_t* gather,
                                 const int32_t* seg_off, const int32_t* pad_off, int nseg, int64_t p_cap, bf16_t* dst,
                                 hipStream_t s) {
  if (p_cap == 0 || cols == 0) return hipSuccess;
  if (p_cap % 64 || ld_src % 8 || cols % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p_cap / 64), (unsigned)((cols + 64 * kTrChunks - 1) / (64 * kTrChunks)));
  transpose_rows_kernel<<<grid, 256, 0, s>>>(src, ld_src, cols, gather, seg_off, pad_off, nseg, dst);
  return hipGetLastError();
}

hipError_t launch_transpose_batched(const bf16_t* src, int64_t batch, int64_t rows, int64_t cols, bf16_t* dst,
                                    hipStream_t s) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols + 63) / 64), (unsigned)batch);
  transpose_batched_kernel<<<grid, 256, 0, s>>>(src, rows, cols, dst);
  return hipGetLastError();
}

hipError_t launch_dx(const bf16_t* da_perm, const int32_t* token_row, const int32_t* topk_idx, const float* dl,
                     const bf16_t* w_router, const bf16_t* dx_shared, bf16_t* dx, int64_t T, int d, int k,
                     hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k < 1 || k > kMaxK || d % 8 || T > INT32_MAX) return hipErrorInvalidValue;
  launch_dx_k<1>(k, da_perm, token_row, topk_idx, dl, w_router, dx_shared, dx, T, d, s);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const bf16_t* x, const int32_t* row_token, const float* dl_row, const int32_t* offsets,
                               const int32_t* pad_off, int E, int d, int64_t p_cap, float* partial, float* dw,
                               hipStream_t s) {
  if (p_cap > 0) {
    const dim3 grid((unsigned)(p_cap / kPadRows), (unsigned)((d / 8 + 255) / 256));
    router_partial_kernel<<<grid, 256, 0, s>>>(x, row_token, dl_row, offsets, pad_off, E, d, partial);
  }
  router_reduce_kernel<<<dim3((unsigned)((d + 31) / 32), (unsigned)E), 256, 0, s>>>(partial, pad_off, E, d, dw);
  return hipGetLastError();
}

}  // namespace moe
