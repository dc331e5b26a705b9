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
//  2. one workgroup scans them expert-major: offsets[e] = sum of earlier
//     experts' totals and before[b][e] = routes of e in blocks before b;
//  3. block b re-walks its routes in (token, slot) order, 256 at a time; a
//     route's row is offsets[e] + before[b][e] plus the number of earlier
//     routes of e in the block (rank among the 256 in flight plus a running
//     LDS cursor).
// The result is the unique expert-major, token-ascending layout.
//
// The gather copies rows with 16-byte loads and stores; the MXFP8 variant
// quantizes every 32-element block of a row on the way (blog post, "MXFP8
// support": activation quantization fused into the dispatch).
#include <mutex>

#include "common.h"

// Scratch of moe_permute_noalloc: the schedule's per-block expert histograms
// in a file-scope device array, for callers that cannot allocate.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: the host
// reaches the array only through the per-device address that
// hipGetSymbolAddress returns (moe::noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[4u << 20];

namespace moe {

namespace {

constexpr int kTokBlock = 128;

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
  for (int e = threadIdx.x; e < E; e += 256) block_counts[(int64_t)blockIdx.x * E + e] = h[e];
}

// block_counts[b][e] becomes the number of expert-e routes in the blocks
// before b (loads batched so that many are in flight); counts and offsets
// (exclusive scan over the experts) are written once.  The scatter adds
// offsets[e] to the block's running count.
__global__ void __launch_bounds__(1024) scan_kernel(int32_t* __restrict__ block_counts, int nb, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  constexpr int kBatch = 16;
  __shared__ int32_t s[1024];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nb; b0 += kBatch) {
      int32_t c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) c[i] = b0 + i < nb ? block_counts[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < nb) block_counts[(int64_t)(b0 + i) * E + e] = total;
        total += c[i];
      }
    }
  }
  s[e] = total;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t v = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) {
    counts[e] = total;
    offsets[e] = s[e] - total;
    if (e == E - 1) offsets[E] = s[e];
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ topk_idx, int64_t T, int E, int k,
                                                      const int32_t* __restrict__ block_base,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ row_token,
                                                      int32_t* __restrict__ token_row) {
  __shared__ int32_t cursor[1024];
  __shared__ int32_t s_e[256];
  for (int e = threadIdx.x; e < E; e += 256) cursor[e] = block_base[(int64_t)blockIdx.x * E + e] + offsets[e];
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

template <int EB>
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ x, const int32_t* __restrict__ row_token,
                                                     uint8_t* __restrict__ xp, int64_t R, int64_t vpr) {
  // vpr: 16-byte vectors per row
  const int64_t nvec = R * vpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t r = v / vpr, c = v - r * vpr;
    const int64_t src = row_token[r];
    const u32x4 val = *reinterpret_cast<const u32x4*>(x + (src * vpr + c) * 16);
    *reinterpret_cast<u32x4*>(xp + (r * vpr + c) * 16) = val;
  }
}

// Row blocks of 32 columns, rows optionally gathered.  Scales row-major
// [R][d/32], or with slab_major slab-major [d/128][R][4] (the four blocks of
// a 128-column slab of one row form one dword; a slab's dwords are
// contiguous over the rows).
__global__ void __launch_bounds__(256) gather_quant_kernel(const bf16_t* __restrict__ x,
                                                           const int32_t* __restrict__ row_token,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                           int64_t R, int d, bool slab_major) {
  const int bpr = d / 32;
  const int64_t nblk = R * bpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    const int64_t r = b / bpr, c = b - r * bpr;
    const int64_t src = row_token ? (int64_t)row_token[r] : r;
    const u32x4* in = reinterpret_cast<const u32x4*>(x + src * d + c * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w = in[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
    uint32_t packed[8];
    const uint32_t sc = mx_quant32(v, packed);
    u32x4* out = reinterpret_cast<u32x4*>(q + r * d + c * 32);
    out[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
    out[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
    scale[slab_major ? ((c >> 2) * R + r) * 4 + (c & 3) : r * bpr + c] = (uint8_t)sc;
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
  if (nb > 0) hist_kernel<<<nb, 256, 0, s>>>(topk_idx, T, E, k, bc);
  scan_kernel<<<1, 1024, 0, s>>>(bc, nb, E, counts, offsets);
  if (nb > 0) scatter_kernel<<<nb, 256, 0, s>>>(topk_idx, T, E, k, bc, offsets, row_token, token_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, void* x_perm, int64_t R, int d, int elem_bytes,
                              hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int64_t vpr = (int64_t)d * elem_bytes / 16;
  gather_kernel<16><<<stream_grid(R * vpr), 256, 0, s>>>(static_cast<const uint8_t*>(x), row_token,
                                                          static_cast<uint8_t*>(x_perm), R, vpr);
  return hipGetLastError();
}

hipError_t launch_gather_quant_mx(const bf16_t* x, const int32_t* row_token, uint8_t* q, uint8_t* scale, int64_t R,
                                  int d, hipStream_t s) {
  if (R == 0) return hipSuccess;
  gather_quant_kernel<<<stream_grid(R * (d / 32)), 256, 0, s>>>(x, row_token, q, scale, R, d, false);
  return hipGetLastError();
}

hipError_t launch_gather_scales_slab(const uint8_t* scale_rows, const int32_t* row_token, int64_t R, int K,
                                     uint8_t* dst, hipStream_t s) {
  if (R == 0) return hipSuccess;
  if (K % 128) return hipErrorInvalidValue;
  gather_scales_slab_kernel<<<stream_grid(R * (K / 128)), 256, 0, s>>>(
      reinterpret_cast<const uint32_t*>(scale_rows), row_token, R, K / 128, reinterpret_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const bf16_t* src, int64_t rows, int64_t cols, int axis, uint8_t* dst, uint8_t* scale,
                              hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (axis == 0 || axis == 2)
    gather_quant_kernel<<<stream_grid(rows * (cols / 32)), 256, 0, s>>>(src, nullptr, dst, scale, rows, (int)cols,
                                                                        axis == 2);
  else
    quant_cols_kernel<<<stream_grid(rows / 32 * cols), 256, 0, s>>>(src, rows, cols, dst, scale);
  return hipGetLastError();
}

}  // namespace moe
