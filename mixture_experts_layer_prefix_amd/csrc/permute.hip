// Schedule and dispatch on one device, plus the MX (E4M3 + E8M0) quantizer.
//
// Mixture-of-Kittens blog post, "Choosing the right communication direction
// / Scheduling": count the routes of every expert, take an exclusive prefix
// sum of the counts as each expert's region offset, then walk the routes
// again and give each its row, so that an expert's tokens land in
// contiguous rows in token order.  With a single source rank the table
// entry of a row is the token index.  The pages run this fully on the
// device with no host round trip; so does this file.
//
// Three integer kernels, no floating point and no order-dependent atomics:
//  1. block histograms: block b counts the routes of its kTokBlock tokens
//     per expert (LDS integer atomics; counts do not depend on order);
//  2. one workgroup per expert scans that expert's column of block counts
//     (stored expert-major): before[e][b] = routes of e in blocks before b,
//     and counts[e] = its total;
//  3. block b takes offsets[e] = sum of earlier experts' counts (an LDS scan
//     of the E counts; block 0 also stores them), then re-walks its routes in
//     (token, slot) order, 256 at a time; a route's row is offsets[e] +
//     before[e][b] plus the number of earlier routes of e in the block (rank
//     among the 256 in flight plus a running LDS cursor).
// The result is the unique expert-major, token-ascending layout.
//
// The dispatch copy runs from token order: each token's row is read once and
// stored to its k routed rows with 16-byte accesses; the MXFP8 variant
// quantizes every 32-element block of the row once on the way (blog post,
// "MXFP8 support": activation quantization fused into the dispatch).
#include <mutex>

#include "common.h"

// Scratch of moe_permute_noalloc: the schedule's per-block expert histograms
// in a file-scope device array, for callers that cannot allocate.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: the host
// reaches the array only through the per-device address that
// hipGetSymbolAddress returns (moe::noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[16u << 20];

namespace moe {

namespace {

constexpr int kTokBlock = 32;  // tokens per schedule block: many blocks even for a few thousand tokens

__global__ void __launch_bounds__(256) hist_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k,
                                                   int32_t* __restrict__ block_counts) {
  __shared__ int32_t h[1024];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * kTokBlock * k;
  const int64_t r1 = min((int64_t)(blockIdx.x + 1) * kTokBlock, T) * k;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += 256) {
    const int e = topk_idx[r];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);  // ids outside [0, E) break the contract; skip them
  }
  __syncthreads();
  const int nb = gridDim.x;
  for (int e = threadIdx.x; e < E; e += 256) block_counts[(int64_t)e * nb + blockIdx.x] = h[e];  // expert-major
}

// Exclusive scan of one expert's column of block counts (workgroup e): each
// thread sums a contiguous run of blocks, a 256-wide LDS scan of the run
// sums gives each run its start, and the run is rewritten as prefixes.
// counts[e] = the column total.
__global__ void __launch_bounds__(256) scan_cols_kernel(int32_t* __restrict__ block_counts, int nb,
                                                        int32_t* __restrict__ counts) {
  __shared__ int32_t s[256];
  const int tid = threadIdx.x;
  int32_t* col = block_counts + (int64_t)blockIdx.x * nb;
  const int per = (nb + 255) / 256;
  const int b0 = min(tid * per, nb), b1 = min(b0 + per, nb);
  int32_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += col[b];
  s[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t v = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  int32_t run = s[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    const int32_t c = col[b];
    col[b] = run;
    run += c;
  }
  if (tid == 255) counts[blockIdx.x] = s[255];
}

// Zero counts and offsets of an empty batch.
__global__ void __launch_bounds__(256) zero_schedule_kernel(int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets, int E) {
  for (int e = threadIdx.x; e <= E; e += 256) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k,
                                                      const int32_t* __restrict__ block_base,
                                                      const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ row_token,
                                                      int32_t* __restrict__ token_row) {
  __shared__ int32_t cursor[1024];
  __shared__ int32_t s_e[256];
  // offsets[e] = sum of the counts of experts before e: 4 consecutive experts
  // per thread, a 256-wide LDS scan of their sums (s_e serves as its array)
  {
    const int tid = threadIdx.x, e0 = tid * 4;
    int32_t c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = e0 + q < E ? counts[e0 + q] : 0;
      sum += c[q];
    }
    s_e[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int32_t v = tid >= off ? s_e[tid - off] : 0;
      __syncthreads();
      s_e[tid] += v;
      __syncthreads();
    }
    int32_t run = s_e[tid] - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (e0 + q < E) {
        cursor[e0 + q] = run;
        if (blockIdx.x == 0) offsets[e0 + q] = run;
      }
      run += c[q];
    }
    if (blockIdx.x == 0 && tid == 255) offsets[E] = s_e[255];
    __syncthreads();
  }
  const int nb = gridDim.x;
  for (int e = threadIdx.x; e < E; e += 256) cursor[e] += block_base[(int64_t)e * nb + blockIdx.x];
  const int64_t r0 = (int64_t)blockIdx.x * kTokBlock * k;
  const int64_t r1 = min((int64_t)(blockIdx.x + 1) * kTokBlock, T) * k;
  for (int64_t c0 = r0; c0 < r1; c0 += 256) {
    const int64_t r = c0 + threadIdx.x;
    const int n = (int)min((int64_t)256, r1 - c0);
    int e = threadIdx.x < n ? topk_idx[r] : -1;
    if ((unsigned)e >= (unsigned)E) {
      if (threadIdx.x < n) token_row[r] = 0;  // invalid id: no row of its own (outside the contract)
      e = -1;
    }
    s_e[threadIdx.x] = e;
    __syncthreads();
    int rank = 0, later = 0;
    if (e >= 0) {
      for (int i = 0; i < n; ++i) {
        const int ei = s_e[i];
        rank += (ei == e) & (i < (int)threadIdx.x);
        later += (ei == e) & (i > (int)threadIdx.x);
      }
      const int32_t row = cursor[e] + rank;
      row_token[row] = (int32_t)(r / k);
      token_row[r] = row;
    }
    __syncthreads();
    if (e >= 0 && later == 0) cursor[e] += rank + 1;
    __syncthreads();
  }
}

// Dispatch as a push from token order: one workgroup per token reads the
// token's row of x once and stores it to each of its k routed rows
// (token_row).  The permutation is a bijection, so every routed row is
// written exactly once and x_perm[r] = x[row_token[r]].  The workgroup is
// sized so that each thread holds two 16-byte vectors of the row (all of
// it for rows up to 2048 vectors); the k destination rows are
// workgroup-uniform (scalar loads).
__global__ void __launch_bounds__(1024) dispatch_rows_kernel(const uint8_t* __restrict__ x,
                                                             const int32_t* __restrict__ token_row,
                                                             uint8_t* __restrict__ xp, int k, int vpr) {
  const int64_t t = blockIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(x) + t * vpr;
  for (int v0 = threadIdx.x; v0 < vpr; v0 += 2 * blockDim.x) {
    const int v1 = v0 + blockDim.x;
    const bool two = v1 < vpr;
    const u32x4 a = __builtin_nontemporal_load(src + v0);
    const u32x4 b = two ? __builtin_nontemporal_load(src + v1) : u32x4{0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      u32x4* dst = reinterpret_cast<u32x4*>(xp) + (int64_t)token_row[t * k + j] * vpr;
      dst[v0] = a;
      if (two) dst[v1] = b;
    }
  }
}

// The MXFP8 dispatch, pushed the same way: one workgroup per token, four
// lanes per 32-element block of its row (16 bytes each, contiguous across the
// wave); the block maximum is a two-step DPP maximum over the lane quad, each
// lane encodes its eight values once and stores them (8 bytes) to each of
// the token's k routed rows, the quad's first lane the E8M0 byte; scales
// row-major [R][d/32].  The workgroup size is a multiple of 64 and d / 8 a
// multiple of 4, so quads never straddle blocks.
__global__ void __launch_bounds__(1024) dispatch_quant_kernel(const bf16_t* __restrict__ x,
                                                              const int32_t* __restrict__ token_row,
                                                              uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                              int k, int d) {
  const int64_t t = blockIdx.x;
  const int cpr = d / 8, bpr = d / 32;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  for (int c = threadIdx.x; c < cpr; c += blockDim.x) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + t * d) + c);
    float v[8];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      m = max(m, (w[j] << 16) & 0x7FFFFFFFu);
      m = max(m, w[j] & 0x7FFF0000u);
    }
    m = max(m, dpp_u32<0xB1>(m));
    m = max(m, dpp_u32<0x4E>(m));
    const int e = mx_block_exp_bits(m);
    const float inv = mx_inv_scale(e);
    const u32x2 codes = u32x2{e4m3x4_rne_sat(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                              e4m3x4_rne_sat(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv)};
    for (int j = 0; j < k; ++j) {
      const int64_t row = token_row[t * k + j];
      *reinterpret_cast<u32x2*>(q + row * d + c * 8) = codes;
      if ((c & 3) == 0) scale[row * bpr + (c >> 2)] = (uint8_t)(e + 127);
    }
  }
}

// Threads of a per-token workgroup covering `items` items with `per` per
// thread: a whole number of waves, at most 1024.
unsigned token_block(int items, int per) {
  int th = (items + per - 1) / per;
  th = (th + 63) / 64 * 64;
  return (unsigned)(th < 64 ? 64 : (th > 1024 ? 1024 : th));
}

// Row blocks of 32 columns of a contiguous [R][d] array, four lanes per block
// (16 bytes each, so a wave reads 1 KiB of a row at once): the block maximum
// is a two-step DPP maximum over the lane quad (exact: the same scale as from
// the whole block in one thread), then each lane encodes its eight values.
// Scales row-major [R][d/32], or with slab_major slab-major [d/128][R][4] (the
// four blocks of a 128-column slab of one row form one dword; a slab's dwords
// are contiguous over the rows).
__global__ void __launch_bounds__(256) quant_rows_kernel(const bf16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ scale, int64_t R, int d,
                                                         bool slab_major) {
  const int cpr = d / 8;  // 16-byte chunks per row, a multiple of 4: quads never straddle rows
  const int64_t n = R * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;  // a multiple of 4: quads stay aligned
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / cpr;
    const int ck = (int)(i - r * cpr);
    const u32x4 w = *reinterpret_cast<const u32x4*>(x + i * 8);
    float v[8];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      m = max(m, (w[j] << 16) & 0x7FFFFFFFu);
      m = max(m, w[j] & 0x7FFF0000u);
    }
    m = max(m, dpp_u32<0xB1>(m));
    m = max(m, dpp_u32<0x4E>(m));
    const int e = mx_block_exp_bits(m);
    const float inv = mx_inv_scale(e);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(q + i * 8) = u32x2{e4m3x4_rne_sat(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                                                 e4m3x4_rne_sat(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv)};
    if ((ck & 3) == 0) {
      const int c = ck >> 2;
      scale[slab_major ? ((int64_t)(c >> 2) * R + r) * 4 + (c & 3) : r * (d / 32) + c] = (uint8_t)(e + 127);
    }
  }
}

// Slab-major scales of gathered rows: dst[s][r] = the dword of slab s (four
// 32-element block scales) of source row row_token[r], for row-major source
// scales [rows][K/32] (K % 128 == 0).  Thread per (r, s), rows fastest.
__global__ void __launch_bounds__(256) gather_scales_slab_kernel(const uint32_t* __restrict__ src,
                                                                 const int32_t* __restrict__ row_token, int64_t R,
                                                                 int slabs, uint32_t* __restrict__ dst) {
  const int64_t n = R * slabs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t sl = i / R, r = i - sl * R;
    dst[i] = src[(int64_t)row_token[r] * slabs + sl];
  }
}

// The same for K % 512 == 0: thread per (r, four consecutive slabs), one
// 16-byte load of the source row and four dword stores, rows fastest.
__global__ void __launch_bounds__(256) gather_scales_slab4_kernel(const u32x4* __restrict__ src,
                                                                  const int32_t* __restrict__ row_token, int64_t R,
                                                                  int groups, uint32_t* __restrict__ dst) {
  const int64_t n = R * groups;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t q = i / R, r = i - q * R;
    const u32x4 v = src[(int64_t)row_token[r] * groups + q];
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(4 * q + j) * R + r] = v[j];
  }
}

// Blocks of 32 consecutive rows of one column: thread per (row block, column).
__global__ void __launch_bounds__(256) quant_cols_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const int64_t nwork = rows / 32 * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwork; w += stride) {
    const int64_t rb = w / cols, c = w - rb * cols;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(src[(rb * 32 + i) * cols + c]);
    uint32_t packed[8];
    const uint32_t sc = mx_quant32(v, packed);
#pragma unroll
    for (int i = 0; i < 32; ++i) q[(rb * 32 + i) * cols + c] = (uint8_t)(packed[i >> 2] >> (8 * (i & 3)));
    scale[rb * cols + c] = (uint8_t)sc;
  }
}

unsigned stream_grid(int64_t work) {
  int64_t g = (work + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

}  // namespace

size_t noalloc_scratch_capacity() { return sizeof(scratch); }

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int permute_num_blocks(int64_t T) { return (int)((T + kTokBlock - 1) / kTokBlock); }

size_t permute_scratch_bytes(int64_t T, int E) { return (size_t)permute_num_blocks(T) * E * sizeof(int32_t); }

hipError_t launch_schedule(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, int32_t* token_row, void* scratch, hipStream_t s) {
  const int nb = permute_num_blocks(T);
  int32_t* bc = static_cast<int32_t*>(scratch);
  if (nb == 0) {
    zero_schedule_kernel<<<1, 256, 0, s>>>(counts, offsets, E);
    return hipGetLastError();
  }
  hist_kernel<<<nb, 256, 0, s>>>(topk_idx, T, E, k, bc);
  scan_cols_kernel<<<E, 256, 0, s>>>(bc, nb, counts);
  scatter_kernel<<<nb, 256, 0, s>>>(topk_idx, T, E, k, bc, counts, offsets, row_token, token_row);
  return hipGetLastError();
}

hipError_t launch_dispatch_rows(const void* x, const int32_t* token_row, void* x_perm, int64_t T, int k, int d,
                                int elem_bytes, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (((int64_t)d * elem_bytes) % 16 || T > INT32_MAX) return hipErrorInvalidValue;
  const int vpr = (int)((int64_t)d * elem_bytes / 16);
  dispatch_rows_kernel<<<(unsigned)T, token_block(vpr, 2), 0, s>>>(static_cast<const uint8_t*>(x), token_row,
                                                                   static_cast<uint8_t*>(x_perm), k, vpr);
  return hipGetLastError();
}

hipError_t launch_dispatch_quant_mx(const bf16_t* x, const int32_t* token_row, uint8_t* q, uint8_t* scale, int64_t T,
                                    int k, int d, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (d % 32 || T > INT32_MAX) return hipErrorInvalidValue;
  dispatch_quant_kernel<<<(unsigned)T, token_block(d / 8, 1), 0, s>>>(x, token_row, q, scale, k, d);
  return hipGetLastError();
}

hipError_t launch_gather_scales_slab(const uint8_t* scale_rows, const int32_t* row_token, int64_t R, int K,
                                     uint8_t* dst, hipStream_t s) {
  if (R == 0) return hipSuccess;
  if (K % 128) return hipErrorInvalidValue;
  if (K % 512 == 0 && (reinterpret_cast<uintptr_t>(scale_rows) & 15) == 0)
    gather_scales_slab4_kernel<<<stream_grid(R * (K / 512)), 256, 0, s>>>(
        reinterpret_cast<const u32x4*>(scale_rows), row_token, R, K / 512, reinterpret_cast<uint32_t*>(dst));
  else
    gather_scales_slab_kernel<<<stream_grid(R * (K / 128)), 256, 0, s>>>(
        reinterpret_cast<const uint32_t*>(scale_rows), row_token, R, K / 128, reinterpret_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const bf16_t* src, int64_t rows, int64_t cols, int axis, uint8_t* dst, uint8_t* scale,
                              hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (axis == 0 || axis == 2)
    quant_rows_kernel<<<stream_grid(rows * (cols / 8)), 256, 0, s>>>(src, dst, scale, rows, (int)cols, axis == 2);
  else
    quant_cols_kernel<<<stream_grid(rows / 32 * cols), 256, 0, s>>>(src, rows, cols, dst, scale);
  return hipGetLastError();
}

}  // namespace moe
