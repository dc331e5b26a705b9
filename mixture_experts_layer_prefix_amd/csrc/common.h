// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // storage type of bf16 values (bit pattern)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// A 64-bit value that is the same in every lane, held in scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 1 / (1 + e^-z) with the hardware reciprocal (about 1 ulp; outputs are
// rounded to bf16 or E4M3 afterwards).
__device__ __forceinline__ float sigmoid_f32(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ float silu_f32(float z) { return z * sigmoid_f32(z); }

// Direct global -> LDS load of BYTES per lane (buffer_load ... lds): the wave
// writes 64 * BYTES contiguous bytes starting at lds_dst.  Only whole-dword
// transfers are allowed: a 1- or 2-byte transfer still writes a full dword
// per lane, which overruns the destination (it once corrupted the group
// tables behind a slab ring).  The destination must be BYTES-aligned.
typedef __attribute__((address_space(3))) void lds_void_t;
template <int BYTES>
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t rsrc, void* lds_dst, uint32_t voffset,
                                        uint32_t soffset) {
  static_assert(BYTES == 4 || BYTES == 16, "LDS-DMA transfers whole dwords: 4 or 16 bytes per lane");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_dst, 16, voffset, soffset, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_dst, 4, voffset, soffset, 0, 0);
}

// Reductions over the 32 lanes of each wave half (lanes 0-31 and 32-63) with
// the result in every lane of the half, without LDS round trips: four DPP
// steps inside each 16-lane row (partner lane l^1, l^2, then the mirrored
// 8-lane and 16-lane halves), then v_permlane16_swap, which hands every lane
// both rows' values of its half.  Every lane combines the same operands in
// the same order, so all 32 lanes hold bit-identical results.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Unsigned maximum (of magnitudes as bit patterns: no float canonicalization).
__device__ __forceinline__ uint32_t half_max32_u(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}
__device__ __forceinline__ float half_sum32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// MX (OCP MX v1.0 format) E4M3 elements with one E8M0 scale per 32 values:
// the block exponent is the smallest e with max|v| / 2^e <= 448 (the finest
// power-of-two scale at which the block maximum is an E4M3 value without
// clipping), clamped to [-127, 127] (-127 for an all-zero block); elements
// are v / 2^e rounded to nearest-even E4M3, sign kept.
// ---------------------------------------------------------------------------
// E4M3 code of s, round to nearest even, saturating at +-448: the clamp to
// +-448 followed by gfx950's OCP E4M3 conversion, which rounds to nearest
// even (bit-identical to that definition for every fp32 input of magnitude
// below 512, checked exhaustively on the hardware).  With the block scale
// above every scaled element is at most 448, so the clamp never acts.
__device__ __forceinline__ float e4m3_clamp(float s) { return __builtin_amdgcn_fmed3f(s, -448.0f, 448.0f); }
__device__ __forceinline__ uint32_t e4m3_rne_sat(float s) {
  const float c = e4m3_clamp(s);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}
// Four codes packed into one word, a in the lowest byte.
__device__ __forceinline__ uint32_t e4m3x4_rne_sat(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}

// Block exponent (unbiased) from the fp32 bit pattern of the block's largest
// magnitude (sign bit clear).  floor(log2 amax) - 8 places amax / 2^e in
// [256, 512); a mantissa above 1.75 (field above 0x600000) would land past
// 448, so the exponent is one larger there.  Zero and fp32 subnormals clamp
// to -127; finite fp32 values never reach the upper clamp.
__device__ __forceinline__ int mx_block_exp_bits(uint32_t abits) {
  const int e = (int)(abits >> 23) - 135 + ((abits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(e, -127);
}

// Block exponent of a 32-value block from its max magnitude.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  return mx_block_exp_bits(__float_as_uint(amax));
}

// 2^-e as an fp32 (exact for e in [-127, 126]).
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Quantize 32 values in registers: returns the E8M0 byte, fills 8 packed words.
__device__ __forceinline__ uint32_t mx_quant32(const float (&v)[32], uint32_t (&packed)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_block_exp(amax);
  const float inv = mx_inv_scale(e);
#pragma unroll
  for (int w = 0; w < 8; ++w)
    packed[w] = e4m3x4_rne_sat(v[4 * w] * inv, v[4 * w + 1] * inv, v[4 * w + 2] * inv, v[4 * w + 3] * inv);
  return (uint32_t)(e + 127);
}

// Weight-gradient tile order.  Each group's mtl x ntl grid of output tiles is
// cut into 8 rectangles, one per XCD: a parts along M times 8/a along N, with
// a chosen so that a rectangle spans the fewest A plus B tile strips.  XCD x
// works through rectangle x of group 0, then of group 1, and so on, so the
// workgroups of one XCD stream the same token-axis slabs of A and B through
// that XCD's L2 instead of every XCD reading all of them.
struct WgradRect {
  int mt0, nt0, bm, bn;
};

// Weight-gradient groups in descending K length (ties: lower id) into
// order[0..G), from the K offset table koff[0..G] (both in LDS; every thread
// of the block takes part).  Tiles are then handed out longest first, each
// XCD's workgroups taking positions in snake order (see wgrad_pos), so the
// few long tiles of the busiest experts spread over the workgroups before
// the many short ones fill in (longest-processing-time list scheduling).
__device__ __forceinline__ void wgrad_order(const int32_t* koff, int G, int32_t* order) {
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int kg = koff[g + 1] - koff[g];
    int r = 0;
    for (int h = 0; h < G; ++h) {
      const int kh = koff[h + 1] - koff[h];
      r += (kh > kg) || (kh == kg && h < g);
    }
    order[r] = g;
  }
}

// Position of round r of workgroup `slot` among the `per_xcd` workgroups of
// its XCD: slot s takes r * per_xcd + s on even rounds and
// r * per_xcd + per_xcd - 1 - s on odd ones.
__device__ __forceinline__ int wgrad_pos(int r, int slot, int per_xcd) {
  return r * per_xcd + ((r & 1) ? per_xcd - 1 - slot : slot);
}
__device__ __forceinline__ WgradRect wgrad_rect(int mtl, int ntl, int xcd) {
  int a = 1, best = 1 << 30;
  for (int c = 1; c <= 8; c *= 2) {
    const int cost = (mtl + c - 1) / c + (ntl + 8 / c - 1) / (8 / c);
    if (cost < best) best = cost, a = c;
  }
  const int b = 8 / a, bi = xcd / b, bj = xcd - bi * b;
  WgradRect r;
  r.mt0 = bi * mtl / a;
  r.bm = (bi + 1) * mtl / a - r.mt0;
  r.nt0 = bj * ntl / b;
  r.bn = (bj + 1) * ntl / b - r.nt0;
  return r;
}

// ---------------------------------------------------------------------------
// Kernel launchers (each returns hipGetLastError() of its launches)
// ---------------------------------------------------------------------------

// Router: logits (fp32) from x and W_r; top-k + weights (with fp64 refinement
// of near-tie tokens).  act_f32: x and W_r are fp32 instead of bf16.
// The logits kernel sums each logit as an fp64 sum of fp32 partial sums over
// kLogitChunkBf16 (bf16 path) or kLogitChunkF32 (fp32 path) consecutive
// products, rounded once to fp32 before the bias is added; it also leaves,
// in topk_w[t * k] (zeroed first), the bits of max_e sum_i |x_ti| |W_r[e][i]|
// (fp32), which bounds the partial sums' error for every logit of token t.
// The top-k kernel reads it before writing topk_w.
constexpr int kLogitChunkBf16 = 64;  // the bf16 GEMM's K slab
constexpr int kLogitChunkF32 = 16;   // the fp32 GEMM's K step
hipError_t launch_router_logits(bool act_f32, const void* x, const void* w_router, const float* bias,
                                float* logits, float* topk_w, int64_t T, int d, int E, int k, hipStream_t s);
hipError_t launch_topk(bool act_f32, const float* logits, const void* x, const void* w_router,
                       const float* bias, int32_t* topk_idx, float* topk_w, int64_t T, int d, int E,
                       int k, hipStream_t s);

// Schedule: per-block histograms -> scan -> stable scatter.
int permute_num_blocks(int64_t T);
size_t permute_scratch_bytes(int64_t T, int E);
// The static scratch of moe_permute_noalloc: its size, and its device address
// on the current device (looked up once per device, then cached).
size_t noalloc_scratch_capacity();
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_schedule(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts,
                           int32_t* offsets, int32_t* row_token, int32_t* token_row, void* scratch,
                           hipStream_t s);
// x_perm[r] = x[row_token[r]], pushed from token order through token_row
// (T tokens, k routes each); elem_bytes 2 or 4 (d elements per row).
hipError_t launch_dispatch_rows(const void* x, const int32_t* token_row, void* x_perm, int64_t T, int k, int d,
                                int elem_bytes, hipStream_t s);
// The same with MX quantization along d (codes [R][d], scales [R][d/32]).
hipError_t launch_dispatch_quant_mx(const bf16_t* x, const int32_t* token_row, uint8_t* q, uint8_t* scale, int64_t T,
                                    int k, int d, hipStream_t s);
// Slab-major [K/128][R][4] scales of the rows row_token[0..R) of a
// row-major [rows][K/32] scale array (the grouped GEMMs' A-scale layout for
// gathered token rows).
hipError_t launch_gather_scales_slab(const uint8_t* scale_rows, const int32_t* row_token, int64_t R, int K,
                                     uint8_t* dst, hipStream_t s);
hipError_t launch_quantize_mx(const bf16_t* src, int64_t rows, int64_t cols, int axis, uint8_t* dst,
                              uint8_t* scale, hipStream_t s);

// Zero-fill with a kernel (bytes % 16 == 0, 16-byte aligned); no memset
// nodes, so the sequence stays safe to capture in a graph.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// Combine (weighted sum).  act_f32: fp32 tensors, else bf16.
hipError_t launch_combine(bool act_f32, const void* o_perm, const int32_t* token_row, const float* topk_w,
                          const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s);

// Backward helpers.  Padded row capacity of a K-grouped operand: every
// group's rows rounded up to `pad` (a multiple of 64).
int64_t bwd_padded_rows(int64_t rows, int groups, int pad);
// pad_off[E+1]: padded prefix of counts; single[4] = {0, round_up(T, pad), 0, T}.
hipError_t launch_pad_offsets(const int32_t* counts, int E, int64_t T, int pad, int32_t* pad_off, int32_t* single,
                              hipStream_t s);
// Expert-blocked output: segment e is a [cols][Kp_e] block at pad_off[e] * cols,
// its scales a slab-major [Kp_e/128][cols][4] block at pad_off[e] * cols / 32
// (segments whole multiples of 128 positions; p_cap, cols multiples of 128, 8).
hipError_t launch_transpose_quant(const bf16_t* src, int64_t ld_src, int cols, const int32_t* gather,
                                  const int32_t* seg_off, const int32_t* pad_off, int nseg, int64_t p_cap,
                                  uint8_t* dst, uint8_t* dst_scale, hipStream_t s);
hipError_t launch_row_weight(const int32_t* token_row, const float* topk_w, int64_t R, float* w_row, hipStream_t s);
hipError_t launch_dg(const float* dg_part, int nparts, const int32_t* token_row, const float* topk_w, int64_t T, int k,
                     float* dtopk_w, float* dl, float* dl_row, hipStream_t s);
// [rows][cols] -> expert-blocked transposed operand (segment e: a [cols][Kp_e]
// block at element pad_off[e] * cols), rows optionally gathered.
hipError_t launch_transpose_rows(const bf16_t* src, int64_t ld_src, int cols, const int32_t* gather,
                                 const int32_t* seg_off, const int32_t* pad_off, int nseg, int64_t p_cap, bf16_t* dst,
                                 hipStream_t s);
hipError_t launch_transpose_batched(const bf16_t* src, int64_t batch, int64_t rows, int64_t cols, bf16_t* dst,
                                    hipStream_t s);
hipError_t launch_dx(const bf16_t* da_perm, const int32_t* token_row, const int32_t* topk_idx, const float* dl,
                     const bf16_t* w_router, const bf16_t* dx_shared, bf16_t* dx, int64_t T, int d, int k,
                     hipStream_t s);
hipError_t launch_router_wgrad(const bf16_t* x, const int32_t* row_token, const float* dl_row, const int32_t* offsets,
                               const int32_t* pad_off, int E, int d, int64_t p_cap, float* partial, float* dw,
                               hipStream_t s);

// ---------------------------------------------------------------------------
// Grouped GEMMs.  A group g owns rows [row_off[g], row_off[g+1]) of the
// routed rows; with row_off == nullptr there is one group of M rows.
// ---------------------------------------------------------------------------
enum GemmMode {
  GEMM_GATEUP = 0,       // h = SiLU(A Wg^T) * (A Wu^T)
  GEMM_DOWN = 1,         // C = A B^T (bf16 out)
  GEMM_PLAIN_F32OUT = 2, // C = A B^T + bias (fp32 out, single group)
  GEMM_GU = 3,           // [G | U] = [A Wg^T | A Wu^T] (bf16, ldc = 2N)
  GEMM_SWIGLU_BWD = 4,   // dH' = A B^T, then SwiGLU backward and router-weight partials
  GEMM_DUALK = 5,        // C = A [B0 | B1]^T with K split in halves over two matrices
  GEMM_WGRAD = 6         // per group g: C_g = A[:, K_g] B[:, K_g]^T over the group's K range
};

struct GemmProblem {
  int mode;
  const void* A;            // [rows][K] (bf16 / fp32 / e4m3)
  const uint8_t* A_scale;   // MX: [rows][K/32]
  const int32_t* a_rows;    // optional row gather: row r reads A row a_rows[r]
  const uint8_t* A_scale_slab;  // MX, optional: the A scales of the (gathered) rows in row order,
                                // slab-major [K/128][M][4]; A_scale is then unused
  int64_t a_bytes;          // size of A in bytes when a_rows is set
  int64_t lda;
  const int32_t* row_off;   // [G+1] or nullptr
  int64_t M;                // rows when row_off == nullptr
  int G;
  const void* B0;           // [G][N0][K]: W_gate / W_down / W_router
  const void* B1;           // [G][N0][K]: W_up (gate/up mode)
  const uint8_t* B0_scale;  // MX scales [G][N0][K/32]
  const uint8_t* B1_scale;
  int64_t b_group_stride;   // elements between groups in B0/B1
  int N;                    // output columns (h columns in gate/up mode)
  int K;
  void* C;                  // [rows][N]
  uint8_t* C_scale;         // MX output scales [rows][N/32] (MXFP8 gate/up)
  int64_t ldc;
  const float* bias;        // [N] (plain mode)
  float* rowabs;            // router GEMM, optional: max over the columns of sum_k |A[r][k]| |B[c][k]|,
  int rowabs_stride;        // at rowabs[r * rowabs_stride] (atomic max of fp32 bits; caller zeroes it);
                            // with it, C is an fp64 sum of fp32 partial sums per K chunk (router logits)
  int32_t* tile_prefix;     // scratch [2(G+1)] (device), M-tile prefixes per group
  int64_t ldb;              // B row stride in elements (0: K; DUALK: K/2 each)
  // SwiGLU backward epilogue
  const void* gu;           // [rows][2N] saved/recomputed G | U
  const float* w_row;       // [rows] router weight per routed row (nullptr: 1)
  void* dgu;                // [rows][2N] out: dG | dU
  void* h_out;              // [rows][N] out: w_row * h (nullptr: skip)
  float* dg_part;           // [rows][N/32] out: partial <dH', h> per 32 columns (nullptr: skip)
  void* gu_out;              // gate/up: optional [rows][2N] bf16 G | U (kept for the backward)
  uint8_t* dgu_q;           // MX: [rows][2N] dG | dU quantized along the columns
  uint8_t* dgu_scale;       // MX: [rows][2N/32]
  uint8_t* dgu_t;           // MX: [dG^T; dU^T] quantized along the routed rows, expert-blocked as the
                            // weight-gradient operand of M = 2N rows ([2N][Kp_g] at pad_off[g] * 2N,
                            // dG^T in rows [0, N), dU^T in rows [N, 2N))
  uint8_t* dgu_t_scale;     // MX: their scales, slab-major ([Kp_g/128][2N][4] at pad_off[g] * 2N / 32)
  uint8_t* gh_t;            // MX: (w h)^T in the same layout ([N][Kp_g] at pad_off[g] * N)
  uint8_t* gh_t_scale;      // MX: its scales, slab-major
  const int32_t* pad_off;   // MX: [G+1] padded group row offsets (multiples of 128)
  int64_t t_ld;             // MX: total padded rows
  // K-grouped (weight gradient) mode
  const int32_t* k_off;     // [G+1] K ranges (multiples of 64) of the groups; the operands are
                            // expert-blocked ([M][Kp_g] block at k_off[g] * M, B alike); MX scales
                            // slab-major ([Kp_g/128][M][4] at k_off[g] * M / 32)
  int64_t c_group_stride;   // elements between group outputs
  void* C1;                 // K-grouped mode, optional: rows [m_split, M) of every group's output go to
  int64_t m_split;          // C1 (at row - m_split, same strides), rows [0, m_split) to C: two gradient
                            // tensors from one launch (dW_gate and dW_up over [dG^T; dU^T])
};

// Workgroups of the persistent GEMM grids: all compute units, or at most
// the cap set with moe_set_max_workgroups (rounded down to a multiple of 8,
// at least 8).  Results do not depend on it.
int gemm_grid(int num_cus);
hipError_t launch_gemm_bf16(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_f32(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_mxfp8(const GemmProblem& p, hipStream_t s);
// One bf16 MFMA per tile (moe_bf16_mma_tiles).
hipError_t launch_bf16_mma_tiles(const bf16_t* a, const bf16_t* b, const float* c, float* d, int64_t n,
                                 hipStream_t s);
// One scaled MFMA per tile (moe_mx_mma_tiles).
hipError_t launch_mx_mma_tiles(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, const uint8_t* b_scale,
                               const float* c, float* d, int64_t n, hipStream_t s);

}  // namespace moe
