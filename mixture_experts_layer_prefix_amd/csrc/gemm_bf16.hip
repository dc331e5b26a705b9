// Expert-grouped bf16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// C[rows of group g][N] = A[rows of g][K] . B[g][N][K]^T, fp32 accumulation.
// Both operands are K-contiguous ("NT"), which is the layout of the token
// rows and of nn.Linear-style [out][in] weights.  The grouping follows the
// expert-contiguous rows of the schedule (Mixture-of-Kittens blog post,
// "Scheduling": tokens of an expert land in contiguous rows so the
// expert-grouped GEMMs start without reordering).
//
// Tiles.  One persistent grid of one 512-thread workgroup per compute unit
// (8 waves as 2 x 4, two per SIMD) loops over output tiles of two kinds:
//  * big tiles, 256 x 256: each wave owns 128 x 64 as 4 x 2 MFMA blocks of
//    32 x 32 (v_mfma_f32_32x32x16_bf16, fp32 accumulators);
//  * small tiles, 64 x 256, for the last rows of an expert (a group of n
//    rows gets floor(n / 256) big tiles, one more if the remainder exceeds
//    128, and 64-row tiles for a smaller remainder).  Under skewed routing
//    most experts hold a few rows: their cost is streaming the expert's
//    weights, and a 64-row tile does that without 4x the wasted MFMA work.
//    Small tiles keep three slabs in LDS (two in flight) since they are
//    bound by memory latency.  In the down projection they are spread
//    evenly through the tile order so they stream weights while other CUs
//    run big tiles.
// K advances 64 at a time through a ring of LDS slabs filled straight from
// global memory by buffer_load ... lds (16 bytes per lane, no register
// staging; 32-bit per-lane offsets with the K position in the scalar offset
// and buffer descriptors bounding every access), one barrier per slab.  Each
// 128-byte LDS row holds its eight 16-byte chunks XOR-swizzled by the row
// index (swz), so the 16-byte fragment reads of 32 consecutive rows are free
// of bank conflicts; the fragment reads of the next K step are interleaved
// with the MFMAs of the current one.
//
// Order.  M-tile prefixes per group are built on the device (empty experts
// cost nothing, the host never learns the counts).  Logical tiles are dealt
// so each XCD (workgroup id mod 8) owns a contiguous run; within a run the
// N-tiles of one M-tile come before the next M-tile, so the workgroups of an
// XCD share A and B slabs in that XCD's L2.
//
// Gate/up mode: the B tile interleaves 32-row blocks of W_gate and W_up for
// the same output columns, so each wave holds G and U of the same elements
// and applies SwiGLU, h = SiLU(G) * U, in registers before the store (blog
// post, "Scheduling the overlaps": SwiGLU runs with the grouped GEMMs).
#include "common.h"

namespace moe {

namespace {

constexpr int kPad = 8;     // bf16 elements of padding per LDS row (16 bytes)
constexpr int kBK = 64;     // K slab
constexpr int kLdsK = kBK + kPad;
constexpr int kBigM = 256, kSmallM = 64, kBN = 256;
#ifndef MOE_GEMM_WAVES_N
#define MOE_GEMM_WAVES_N 4
#endif
constexpr int kWavesM = 2, kWavesN = MOE_GEMM_WAVES_N;  // 2 x 4: 8 waves, 2 per SIMD
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr size_t kSmemBytes = 2ull * (kBigM + kBN) * kBK * sizeof(bf16_t);  // 131,072 B
// Group tables (tile prefixes and row offsets, or K offsets) are copied into
// LDS after the slab ring, so each tile's group lookup is a short LDS binary
// search instead of a chain of dependent global loads.
constexpr int kMaxGroups = 1024;
constexpr size_t kTabBytes = 3ull * (kMaxGroups + 1) * sizeof(int32_t);

// Tile counts of a group of `rows` rows.
__host__ __device__ __forceinline__ void tiles_of(int64_t rows, int& nb, int& ns) {
  int64_t b = rows / kBigM, r = rows - b * kBigM;
  if (r > kBigM / 2) {
    ++b;
    r = 0;
  }
  nb = (int)b;
  ns = (int)((r + kSmallM - 1) / kSmallM);
}

// Exclusive prefixes of the big and small M-tile counts over the groups.
__global__ void __launch_bounds__(1024) tile_prefix_kernel(const int32_t* __restrict__ row_off, int G,
                                                            int32_t* __restrict__ big, int32_t* __restrict__ small) {
  __shared__ int32_t sb[1024], ss[1024];
  __shared__ int32_t cb, cs;
  if (threadIdx.x == 0) {
    cb = cs = 0;
    big[0] = small[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < G; base += 1024) {
    const int g = base + threadIdx.x;
    int nb = 0, ns = 0;
    if (g < G) tiles_of((int64_t)(row_off[g + 1] - row_off[g]), nb, ns);
    sb[threadIdx.x] = nb;
    ss[threadIdx.x] = ns;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int vb = threadIdx.x >= off ? sb[threadIdx.x - off] : 0;
      const int vs = threadIdx.x >= off ? ss[threadIdx.x - off] : 0;
      __syncthreads();
      sb[threadIdx.x] += vb;
      ss[threadIdx.x] += vs;
      __syncthreads();
    }
    if (g < G) {
      big[g + 1] = cb + sb[threadIdx.x];
      small[g + 1] = cs + ss[threadIdx.x];
    }
    __syncthreads();
    if (threadIdx.x == 1023) {
      cb += sb[1023];
      cs += ss[1023];
    }
    __syncthreads();
  }
}

struct KArgs {
  const bf16_t* A;
  const int32_t* a_rows;
  int64_t lda;
  const int32_t* row_off;  // [G+1] or nullptr (one group of M rows)
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
  uint32_t a_bytes;      // bytes of A when rows are gathered through a_rows
  const int32_t* big;    // big M-tile prefix [G+1] (nullptr: single group)
  const int32_t* small;  // small M-tile prefix [G+1]
  int single_big, single_small;
  int spread_small;      // interleave small tiles among big ones (else big first)
  int64_t ldb;           // B row stride (elements)
  int k_half;            // DUALK: K of the first matrix
  const bf16_t* gu;
  const float* w_row;
  bf16_t* dgu;
  bf16_t* h_out;
  float* dg_part;
  const int32_t* k_off;
  int64_t c_group_stride;
  bf16_t* C1;               // optional second output: rows [m_split, M) of every group
  int64_t m_split;
  bf16_t* gu_out;        // gate/up: optional [rows][2N] G | U output
  float* rowabs;         // router GEMM, optional: rowabs[row * rowabs_stride] = max over the columns of
  int rowabs_stride;     // sum_k |A[row][k]| |B[col][k]| (as fp32 bits, by atomic max; zeroed by the caller)
};

// LDS swizzle of a 128-byte row: chunk position = logical chunk ^ swz(row).
// 16 consecutive rows then spread a 16-byte column read over 16 distinct
// 16-byte bank groups of a 256-byte bank window (even and odd rows sit in
// opposite halves), and any 8 consecutive rows over 8 distinct groups of a
// 128-byte window.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// A pointer the whole wave agrees on, kept in scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Largest g with prefix[g] <= mt (prefix non-decreasing, prefix[0] = 0).
__device__ __forceinline__ int find_group(const int32_t* prefix, int G, int mt) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// One BM x kBN output tile of group g: rows [m0, m0 + BM) of the group.
//
// Slabs of 64 K-elements go global -> LDS directly (buffer_load ... lds, no
// register staging): one instruction moves 8 rows x 128 bytes for a wave.
// Per-lane byte offsets are fixed for the whole tile, the K position rides
// in the scalar offset, and the buffer descriptors bound every access to its
// tensor.  LDS rows are dense 128-byte lines with the 16-byte chunks
// XOR-swizzled per row (swz), realised by letting each lane fetch the chunk
// that belongs at its LDS slot; the MFMA fragment reads of 8 consecutive rows
// then hit 8 distinct bank groups.
//
// Per slab the four 16-deep K steps are software-pipelined: fragments of
// step s+1 are read from LDS while the MFMAs of step s run (two register
// sets).  The barrier sits before the last step's MFMAs, so the load of the
// slab after next and the first fragments of the next slab overlap them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int MODE, int NS>
__device__ __forceinline__ void gemm_tile(const KArgs& p, bf16_t* smem, int g, int64_t row_begin, int64_t n_g,
                                          int64_t m0, int ntile, int k_begin, int KT) {
  constexpr int BN = kBN;
  constexpr int WM = BM / kWavesM, WN = BN / kWavesN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int RPR = kThreads / 8;          // rows per load round (8 rows per wave)
  constexpr int AR = BM / RPR, BR = BN / RPR;
  constexpr bool PAIRED = MODE == GEMM_GATEUP || MODE == GEMM_GU;  // B rows interleave two matrices
  static_assert(AR * RPR == BM && BR * RPR == BN, "tile/thread mismatch");
  static_assert(!PAIRED || FN % 2 == 0, "gate/up needs G,U block pairs per wave");
  bf16_t* As = smem;                    // [NS][BM][64]
  bf16_t* Bs = smem + NS * BM * kBK;    // [NS][BN][64]
  constexpr int LPS = AR + BR;          // loads per slab per thread

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int lrow = wave * 8 + (lane >> 3);       // row inside a load round
  // global 16-byte chunk for this lane's LDS slot: slot (lane & 7) of row r
  // holds chunk slot ^ swz(r), r & 7 = lane >> 3 and (r >> 3) & 1 = wave & 1
  const int chunk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  // Weight-gradient operands are expert-blocked: group g's A is a dense
  // [M][Kp] block at element k_off[g] * M (B alike with N rows), Kp its
  // padded row count, so a tile's K slabs are contiguous.
  constexpr bool KGROUPED = MODE == GEMM_WGRAD;
  int64_t lda = KGROUPED ? (int64_t)KT * kBK : p.lda;
  int64_t ldb = KGROUPED ? (int64_t)KT * kBK : p.ldb;
  asm volatile("" : "+s"(lda), "+s"(ldb));  // keep per-tile address arithmetic inside the tile
  const bf16_t* Ag = KGROUPED ? p.A + (int64_t)k_begin * p.M : p.A;
  const bf16_t* Bg0 = KGROUPED ? p.B0 + (int64_t)k_begin * p.N : p.B0;
  if (KGROUPED) k_begin = 0;

  // A: this tile's rows of the group (or gathered token rows); descriptor over
  // the tile's rows, or over the whole gather source.
  const bool gath = p.a_rows != nullptr;
  const int64_t tile_rows = min<int64_t>(BM, n_g - m0);
  const bf16_t* abase = uniform_ptr(gath ? p.A : Ag + (row_begin + m0) * lda);
  const uint32_t abytes = __builtin_amdgcn_readfirstlane(gath ? p.a_bytes : (uint32_t)(tile_rows * lda * 2));
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, (int)abytes, 0x00020000);
  uint32_t aoff[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int64_t lr0 = i * RPR + lrow;           // row within the tile
    const int64_t lr = lr0 < tile_rows ? lr0 : 0;
    const int64_t src = gath ? (int64_t)p.a_rows[row_begin + m0 + lr] : lr;
    aoff[i] = (uint32_t)(src * lda * 2) + chunk * 16;
  }
  // B: the group's [N][ldb] matrix, rebased at the first row this N-tile
  // reads.  Paired modes interleave 32-row blocks of two matrices (W_gate,
  // W_up) for the same output columns; the rows a wave loads in one round lie
  // in one block, so the matrix choice is wave-uniform.  DUALK switches
  // matrix halfway along K (uniform per slab).
  const int span = PAIRED ? BN / 2 : BN;          // B rows one N-tile covers per matrix
  const int first_row = ntile * span;
  const uint32_t bbytes =
      __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)min(span, p.N - first_row) * ldb * 2));
  const bf16_t* b0 = Bg0 + (int64_t)g * p.b_group_stride + (int64_t)first_row * ldb;
  const bf16_t* b1 = (PAIRED || MODE == GEMM_DUALK) ? p.B1 + (int64_t)g * p.b_group_stride + (int64_t)first_row * ldb
                                                    : b0;
  const __amdgpu_buffer_rsrc_t br0 =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(b0), (short)0, (int)bbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t br1 = (PAIRED || MODE == GEMM_DUALK)
      ? __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(b1), (short)0, (int)bbytes, 0x00020000)
      : br0;
  const uint32_t boff = (uint32_t)((lane >> 3) * ldb * 2) + chunk * 16;

  auto issue = [&](int buf, int k0) {
    const int ka = k_begin + k0;
#pragma unroll
    for (int i = 0; i < AR; ++i)
      lds_dma<16>(ar, As + (buf * BM + i * RPR + wave * 8) * kBK, aoff[i], ka * 2);
    const bool second = MODE == GEMM_DUALK && k0 >= p.k_half;
    const int kb = MODE == GEMM_DUALK ? (second ? k0 - p.k_half : k0) : ka;
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      // LDS rows lr.. lr+7 of this wave in round i; paired modes fill 32-row
      // LDS blocks alternately from the two matrices (block b: matrix b & 1,
      // matrix rows (b >> 1) * 32 ..), so the matrix choice is wave-uniform.
      const int lr = i * RPR + wave * 8;
      const int blk = lr >> 5;
      int r0 = PAIRED ? (blk >> 1) * 32 + (lr & 31) : lr;
      r0 = min(r0, p.N - first_row - 8);  // rows past N load valid rows; their outputs are not stored
      const bool use1 = PAIRED ? (blk & 1) != 0 : second;
      lds_dma<16>(use1 ? br1 : br0, Bs + (buf * BN + lr) * kBK, boff, (uint32_t)((r0 * ldb + kb) * 2));
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](int set, int buf, int kk) {
    const bf16_t* Ab = As + buf * BM * kBK;
    const bf16_t* Bb = Bs + buf * BN * kBK;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + i * 32 + (lane & 31);
      fa[set][i] = *reinterpret_cast<const bf16x8*>(Ab + r * kBK + ((c ^ swz(r)) << 3));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WN + j * 32 + (lane & 31);
      fb[set][j] = *reinterpret_cast<const bf16x8*>(Bb + r * kBK + ((c ^ swz(r)) << 3));
    }
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
  };

  // Ask the scheduler to interleave the fragment reads of the next step with
  // the MFMAs of the current one (one LDS read per MFMA_PER_READ MFMAs).
  constexpr int NREAD = FM + FN, NMMA = FM * FN;
  constexpr int MFMA_PER_READ = NMMA / NREAD > 0 ? NMMA / NREAD : 1;
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < NREAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, MFMA_PER_READ, 0);  // MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NREAD * MFMA_PER_READ > 0 ? NMMA - NREAD * MFMA_PER_READ : 0,
                                         0);
  };

  // NS-slab ring in LDS: slabs 0..NS-1 go out first; after the barrier of
  // iteration kt slab kt's buffer is free and takes slab kt+NS.  Before the
  // barrier only slab kt+1 must have landed, so vmcnt may leave the younger
  // slabs (LPS loads each) in flight.
  // Stores of the previous tile may still be in flight: they are older than
  // this tile's loads, and loads return in order, so a wait for "at most n
  // outstanding" still guarantees that every load but the youngest n landed.
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0)
    if (s0 < KT) issue(s0, s0 * kBK);
  if (KT >= NS) wait_vmcnt<(NS - 1) * LPS>(); else wait_vmcnt<0>();
  __syncthreads();
  read_frags(0, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt % NS;
    read_frags(1, buf, 1);
    mma(0);
    interleave();
    read_frags(0, buf, 2);
    mma(1);
    interleave();
    read_frags(1, buf, 3);
    mma(0);
    interleave();
    if (kt + NS - 1 < KT) wait_vmcnt<(NS - 2) * LPS>(); else wait_vmcnt<0>();
    __syncthreads();
    if (kt + NS < KT) issue(buf, (kt + NS) * kBK);
    if (kt + 1 < KT) read_frags(0, (kt + 1) % NS, 0);
    mma(1);
    interleave();
  }

  // Epilogue.  32x32 block layout: lane holds column (lane & 31) and rows
  // 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
  int64_t ldc = p.ldc;
  asm volatile("" : "+s"(ldc));
  int64_t row0 = row_begin + m0;
  // Split K-grouped output: a tile wholly past m_split writes C1; a tile
  // straddling m_split picks the tensor per row (bounds-checked path).
  bf16_t* Cg = static_cast<bf16_t*>(p.C);
  bool straddle = false;
  if (MODE == GEMM_WGRAD && p.C1) {
    if (row0 >= p.m_split) {
      Cg = p.C1;
      row0 -= p.m_split;
    } else {
      straddle = row0 + BM > p.m_split;
    }
  }
  bf16_t* C = Cg + (MODE == GEMM_WGRAD ? (int64_t)g * p.c_group_stride : 0) + row0 * ldc;
  const int rows_left = (int)tile_rows;
  if constexpr (MODE == GEMM_SWIGLU_BWD) {
    // dH' (unscaled by the router weight w) -> dG, dU, w h (the down
    // projection's weight-gradient operand) and the partial router-weight
    // gradient <dH', h> over these 32 columns (all lanes take part in the
    // reduction).  The G, U and router-weight loads of a batch of VB rows are
    // all issued before the first use: one memory round trip per batch
    // instead of one per row.
    constexpr int VB = 8;
    const int N = p.N;
#pragma clang loop unroll(full)
    for (int i = 0; i < FM; ++i) {
#pragma clang loop unroll(full)
      for (int vb = 0; vb < 16; vb += VB) {
        float wrb[VB];
        bf16_t gb[VB][FN], ub[VB][FN];
#pragma clang loop unroll(full)
        for (int u = 0; u < VB; ++u) {
          const int rl = wm * WM + i * 32 + 8 * ((vb + u) >> 2) + 4 * (lane >> 5) + ((vb + u) & 3);
          const int64_t grow = row0 + min(rl, rows_left - 1);
          wrb[u] = p.w_row ? p.w_row[grow] : 1.0f;
          const bf16_t* gurow = p.gu + grow * 2 * N;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = min(ntile * BN + wn * WN + j * 32 + (lane & 31), N - 1);
            gb[u][j] = gurow[col];
            ub[u][j] = gurow[N + col];
          }
        }
#pragma clang loop unroll(full)
        for (int u = 0; u < VB; ++u) {
          const int v = vb + u;
          const int rl = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int64_t grow = row0 + min(rl, rows_left - 1);
          const float wr = wrb[u];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col0 = ntile * BN + wn * WN + j * 32 + (lane & 31);
            const int col = min(col0, N - 1);
            const float gv = bf16_to_f32(gb[u][j]);
            const float uv = bf16_to_f32(ub[u][j]);
            const float sg = sigmoid_f32(gv);
            const float sl = gv * sg;
            const float h = sl * uv;
            const float dhp = acc[i][j][v];
            const float dh = wr * dhp;
            const float part = half_sum32(dhp * h);
            if (rl < rows_left && col0 < N) {
              bf16_t* drow = p.dgu + grow * 2 * N;
              drow[col] = f32_to_bf16(dh * uv * sg * (1.0f + gv * (1.0f - sg)));
              drow[N + col] = f32_to_bf16(dh * sl);
              if (p.h_out) p.h_out[grow * N + col] = f32_to_bf16(wr * h);
              if (p.dg_part && (lane & 31) == 0) p.dg_part[grow * (N / 32) + col / 32] = part;
            }
          }
        }
      }
    }
    return;
  }
  // One per-lane base pointer; rows step by compile-time multiples of ldc and
  // column blocks by immediate offsets.  Interior tiles skip the bounds checks.
  const int rl0 = wm * WM + 4 * (lane >> 5);  // tile row of (i = 0, v = 0)
  const bool full_rows = rows_left == BM;
  const int N = p.N;
  if constexpr (PAIRED) {
    const int colb = ntile * (BN / 2) + wn * (FN / 2) * 32 + (lane & 31);
    const bool full_cols = ntile * (BN / 2) + BN / 2 <= N;
    bf16_t* Cb = C + (int64_t)rl0 * ldc + colb;
    bf16_t* Sb = p.gu_out ? p.gu_out + (row0 + rl0) * 2 * N + colb : nullptr;
#pragma clang loop unroll(full)
    for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
      for (int v = 0; v < 16; ++v) {
        const int r = i * 32 + 8 * (v >> 2) + (v & 3);
        if (!full_rows && rl0 + r >= rows_left) continue;
        bf16_t* Cr = Cb + (int64_t)r * ldc;
#pragma unroll
        for (int q = 0; q < FN / 2; ++q) {
          if (!full_cols && colb + q * 32 >= N) continue;
          const float gv = acc[i][2 * q][v], uv = acc[i][2 * q + 1][v];
          if (MODE == GEMM_GATEUP) {
            Cr[q * 32] = f32_to_bf16(silu_f32(gv) * uv);
            if (Sb) {  // G | U kept for the backward
              bf16_t* Sr = Sb + (int64_t)r * 2 * N;
              Sr[q * 32] = f32_to_bf16(gv);
              Sr[N + q * 32] = f32_to_bf16(uv);
            }
          } else {
            Cr[q * 32] = f32_to_bf16(gv);
            Cr[N + q * 32] = f32_to_bf16(uv);
          }
        }
      }
  } else {
    const int colb = ntile * BN + wn * WN + (lane & 31);
    const bool full_cols = ntile * BN + BN <= N;
    bf16_t* Cb = C + (int64_t)rl0 * ldc + colb;
#pragma clang loop unroll(full)
    for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
      for (int v = 0; v < 16; ++v) {
        const int r = i * 32 + 8 * (v >> 2) + (v & 3);
        if (!full_rows && rl0 + r >= rows_left) continue;
        bf16_t* Cr = Cb + (int64_t)r * ldc;
        if (MODE == GEMM_WGRAD && straddle && row0 + rl0 + r >= p.m_split)  // this row belongs to C1
          Cr = p.C1 + (int64_t)g * p.c_group_stride + (row0 + rl0 + r - p.m_split) * ldc + colb;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (full_cols || colb + j * 32 < N) Cr[j * 32] = f32_to_bf16(acc[i][j][v]);
      }
  }
}

// Zero rows [m0, m0 + 256) x columns [n0, n0 + 256) of one group's output
// (a weight gradient of an expert without rows) with 16-byte stores.
__device__ __forceinline__ void zero_tile(const KArgs& p, int g, int64_t m0, int n0) {
  const int rows = (int)min<int64_t>(kBigM, p.M - m0);
  const int cols = min(kBN, p.N - n0);
  const int cpr = cols / 8;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < rows * cpr; c += kThreads) {
    const int r = c / cpr, q = c - r * cpr;
    int64_t row = m0 + r;
    bf16_t* C = static_cast<bf16_t*>(p.C);
    if (p.C1 && row >= p.m_split) {  // split output: rows past m_split live in C1
      C = p.C1;
      row -= p.m_split;
    }
    *reinterpret_cast<u32x4*>(C + (int64_t)g * p.c_group_stride + row * p.ldc + n0 + q * 8) = u32x4{0, 0, 0, 0};
  }
}

template <int MODE>
__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_kernel(KArgs p) {
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  int32_t* tab = reinterpret_cast<int32_t*>(smem + kSmemBytes / sizeof(bf16_t));
  const bool single = p.big == nullptr;
  const int32_t* t_big = tab;
  const int32_t* t_small = tab + (p.G + 1);
  const int32_t* t_row = tab + 2 * (p.G + 1);
  if (MODE == GEMM_WGRAD) {
    for (int i = threadIdx.x; i <= p.G; i += kThreads) tab[i] = p.k_off[i];
    __syncthreads();
  } else if (!single) {
    for (int i = threadIdx.x; i <= p.G; i += kThreads) {
      tab[i] = p.big[i];
      tab[p.G + 1 + i] = p.small[i];
      tab[2 * (p.G + 1) + i] = p.row_off[i];
    }
    __syncthreads();
  }
  const int nbig = single ? p.single_big : t_big[p.G];
  const int nsmall = single ? p.single_small : t_small[p.G];
  const int tb = nbig * p.ntiles;
  const int total = tb + nsmall * p.ntiles;
  const int nwg = gridDim.x;
  const int per_xcd = nwg >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // N-tiles of one M-tile visited before the next M-tile: 8 for the modes
  // whose B is a down projection, both dgrad weights or the SwiGLU backward's
  // 8 N-tiles (each A strip is read fewer times; measured 1-2% faster), 4 for
  // the paired gate/up (more B reuse).
  constexpr int GN = (MODE == GEMM_DOWN || MODE == GEMM_DUALK || MODE == GEMM_SWIGLU_BWD) ? 8 : 4;

  if (MODE == GEMM_WGRAD) {
    // One output per group, all of it in big tiles; K range from k_off.
    const WgradRect rc = wgrad_rect((int)((p.M + kBigM - 1) / kBigM), p.ntiles, xcd);
    const int per_g = rc.bm * rc.bn;
    const int tot = p.G * per_g;
    int32_t* order = tab + (p.G + 1);
    wgrad_order(tab, p.G, order);
    __syncthreads();
    for (int rd = 0;; ++rd) {
      const int P = wgrad_pos(rd, slot, per_xcd);
      if (P >= tot) break;
      const int gi = P / per_g;
      const int g = __builtin_amdgcn_readfirstlane(order[gi]);
      const int r = P - gi * per_g;
      const int mt = rc.mt0 + r / rc.bn, nt = rc.nt0 + r % rc.bn;
      const int kb = __builtin_amdgcn_readfirstlane(tab[g]);
      const int kt = __builtin_amdgcn_readfirstlane((tab[g + 1] - kb) / kBK);
      if (kt == 0) {
        zero_tile(p, g, (int64_t)mt * kBigM, nt * kBN);
        continue;
      }
      gemm_tile<kBigM, MODE, 2>(p, smem, g, 0, p.M, uniform_i64((int64_t)mt * kBigM),
                                __builtin_amdgcn_readfirstlane(nt), kb, kt);
      __syncthreads();
    }
    return;
  }
  const int ts = total - tb;
  const int KT = p.K / kBK;
  for (int it = 0;; ++it) {
    const int P = it * nwg + xcd * per_xcd + slot;
    if (P >= total) break;
    // Small tiles (weight streaming, HBM-bound) are spread evenly among the
    // big ones (MFMA-bound), so both kinds run side by side on different CUs:
    // position P is small when the running share of small tiles steps up.
    bool is_big;
    int L;
    if (p.spread_small) {
      const int s_before = (int)((int64_t)P * ts / total);
      is_big = (int)((int64_t)(P + 1) * ts / total) == s_before;
      L = is_big ? P - s_before : s_before;
    } else {
      is_big = P < tb;
      L = is_big ? P : P - tb;
    }
    const int nm = is_big ? nbig : nsmall;
    const int ng = L / (nm * GN);
    const int r0 = L - ng * nm * GN;
    const int gn = min(GN, p.ntiles - ng * GN);
    const int mt = r0 / gn;
    const int ntile = ng * GN + (r0 - mt * gn);
    int g = 0;
    int64_t row_begin = 0, n_g = p.M, m0;
    if (single) {
      m0 = is_big ? (int64_t)mt * kBigM : (int64_t)p.single_big * kBigM + (int64_t)mt * kSmallM;
    } else {
      const int32_t* pre = is_big ? t_big : t_small;
      g = find_group(pre, p.G, mt);
      row_begin = t_row[g];
      n_g = t_row[g + 1] - t_row[g];
      const int nb_g = t_big[g + 1] - t_big[g];
      m0 = is_big ? (int64_t)(mt - pre[g]) * kBigM : (int64_t)nb_g * kBigM + (int64_t)(mt - pre[g]) * kSmallM;
    }
    g = __builtin_amdgcn_readfirstlane(g);
    row_begin = uniform_i64(row_begin);
    n_g = uniform_i64(n_g);
    m0 = uniform_i64(m0);
    if (is_big) gemm_tile<kBigM, MODE, 2>(p, smem, g, row_begin, n_g, m0, __builtin_amdgcn_readfirstlane(ntile), 0, KT);
    else gemm_tile<kSmallM, MODE, 3>(p, smem, g, row_begin, n_g, m0, __builtin_amdgcn_readfirstlane(ntile), 0, KT);
    __syncthreads();
  }
}

// Router-sized GEMM with fp32 output and bias: 64 x 64 tiles (the output has
// only E columns, so big tiles would leave most CUs idle).
__global__ void __launch_bounds__(256) gemm_bf16_small_n_kernel(KArgs p) {
  constexpr int BM = 64, BN = 64, WM = 32, WN = 32;
  constexpr int KV = kBK / 8;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM][kLdsK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN][kLdsK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int ntile = blockIdx.y;
  const bf16_t* pa[2];
  const bf16_t* pb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + i * 256, row = v / KV, kc = (v % KV) * 8;
    const int64_t r = min(m0 + row, p.M - 1);
    pa[i] = p.A + r * p.lda + kc;
    pb[i] = p.B0 + (int64_t)min(ntile * BN + row, p.N - 1) * p.K + kc;
  }
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  // Slabs move global -> registers -> LDS; kPD slabs are in flight in
  // registers (one K loop of a 64 x 64 tile is otherwise a chain of
  // load-latency waits).
  constexpr int kPD = 4;
  u32x4 ra[kPD][2], rb[kPD][2];
  const int KT = p.K / kBK;
  auto ld = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[slot][i] = *reinterpret_cast<const u32x4*>(pa[i] + k0);
      rb[slot][i] = *reinterpret_cast<const u32x4*>(pb[i] + k0);
    }
  };
  auto st = [&](int slot, int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + i * 256;
      *reinterpret_cast<u32x4*>(&As[b][v / KV][(v % KV) * 8]) = ra[slot][i];
      *reinterpret_cast<u32x4*>(&Bs[b][v / KV][(v % KV) * 8]) = rb[slot][i];
    }
  };
#pragma unroll
  for (int j = 0; j < kPD; ++j)
    if (j < KT) ld(j, j * kBK);
  st(0, 0);
  __syncthreads();
  for (int kt0 = 0; kt0 < KT; kt0 += kPD) {
#pragma unroll
    for (int u = 0; u < kPD; ++u) {
      const int kt = kt0 + u;  // slab kt sits in LDS buffer u & 1 (kPD is even)
      if (kt < KT) {
        if (kt + kPD < KT) ld(u, (kt + kPD) * kBK);  // register slot u was stored at step kt - 1
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
          const int kof = kk * 16 + (lane >> 5) * 8;
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[u & 1][wm * WM + (lane & 31)][kof]);
          const bf16x8 bf = *reinterpret_cast<const bf16x8*>(&Bs[u & 1][wn * WN + (lane & 31)][kof]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
        }
        if (kt + 1 < KT) st((u + 1) % kPD, (u + 1) & 1);
        __syncthreads();
      }
    }
  }
  float* C = static_cast<float*>(p.C);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = m0 + wm * WM + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const int col = ntile * BN + wn * WN + (lane & 31);
    if (row < p.M && col < p.N) C[row * p.ldc + col] = acc[v] + (p.bias ? p.bias[col] : 0.0f);
  }
}

// Router logits (rowabs set): 64 x 64 tiles of C = A . B^T + bias, where each
// logit is an fp64 sum, in K order, of fp32 partial sums of one 64-element
// K slab (the matrix cores sum a slab into a fresh accumulator), rounded once
// to fp32 before the bias; and rowabs[row * rowabs_stride] = the maximum over
// the tile's columns of sum_k |A[row][k]| |B[col][k]| (fp32 bits, by atomic
// maximum: order-independent).  Operands go global -> LDS by LDS DMA into a
// two-slab ring of swizzled 128-byte rows (as the grouped GEMMs), so no
// register staging competes with the fp64 sums: about 110 registers, four
// waves per SIMD, and the workgroups of a 16,384-token launch all resident.
__global__ void __launch_bounds__(256) gemm_bf16_logits_kernel(KArgs p) {
  constexpr int BM = 64, BN = 64, WM = 32, WN = 32;
  static_assert(kBK == kLogitChunkBf16, "logit chunk = K slab");
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * kBK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int rows_a = (int)min<int64_t>(BM, p.M - m0), rows_b = min(BN, p.N - n0);
  // Descriptors over the tile's rows; rows past the end load the last row
  // (their outputs are not stored).  Wave w fills LDS rows 16 w .. 16 w + 15
  // of A and of B, 8 rows per load; slot (lane & 7) of row r holds the
  // 16-byte chunk slot ^ swz(r), r & 7 = lane >> 3, (r >> 3) & 1 = j.
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.A + m0 * p.lda), (short)0, (int)(rows_a * p.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(p.B0 + (int64_t)n0 * p.K), (short)0, (int)(rows_b * p.K * 2), 0x00020000);
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wave * 16 + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ (lane >> 3) ^ j;
    aoff[j] = (uint32_t)(min(r, rows_a - 1) * p.lda * 2) + chunk * 16;
    boff[j] = (uint32_t)(min(r, rows_b - 1) * p.K * 2) + chunk * 16;
  }
  auto issue = [&](int buf, int k0) {  // 4 loads per wave
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lds_dma<16>(ar, &As[buf][(wave * 16 + 8 * j) * kBK], aoff[j], (uint32_t)k0 * 2);
      lds_dma<16>(br, &Bs[buf][(wave * 16 + 8 * j) * kBK], boff[j], (uint32_t)k0 * 2);
    }
  };
  auto abs8 = [](bf16x8 v) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] &= 0x7FFF7FFFu;
    return __builtin_bit_cast(bf16x8, u);
  };
  f32x16 part, aab;
  double acc64[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    part[v] = aab[v] = 0.0f;
    acc64[v] = 0.0;
  }
  const int KT = p.K / kBK;
  const int ra = wm * WM + (lane & 31), rb = wn * WN + (lane & 31);
  issue(0, 0);
  if (KT > 1) issue(1, kBK);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) wait_vmcnt<4>(); else wait_vmcnt<0>();  // this slab's loads (the next slab's may fly)
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[buf][ra * kBK + ((c ^ swz(ra)) << 3)]);
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(&Bs[buf][rb * kBK + ((c ^ swz(rb)) << 3)]);
      part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, kk == 0 ? f32x16{} : part, 0, 0, 0);
      aab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abs8(af), abs8(bf), aab, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) acc64[v] += (double)part[v];
    __syncthreads();  // every wave is done with this buffer: slab kt + 2 goes there
    if (kt + 2 < KT) issue(buf, (kt + 2) * kBK);
  }
  float* C = static_cast<float*>(p.C);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = m0 + wm * WM + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const int col = n0 + wn * WN + (lane & 31);
    if (row < p.M && col < p.N) C[row * p.ldc + col] = (float)acc64[v] + (p.bias ? p.bias[col] : 0.0f);
  }
  // Largest sum of |a_k| |b_k| of each row over this tile's 64 columns: the
  // 32 columns of a wave half in DPP steps, then an atomic maximum of the
  // (non-negative) fp32 bits; order-independent, so deterministic.  Columns
  // past N repeat expert N-1 (clamped loads): a real expert's sum.
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t row = m0 + wm * WM + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const uint32_t m = half_max32_u(__float_as_uint(aab[v]) & 0x7FFFFFFFu);
    if ((lane & 31) == 0 && row < p.M) atomicMax(reinterpret_cast<unsigned int*>(p.rowabs + row * p.rowabs_stride), m);
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

template <int MODE>
hipError_t run_grouped(const GemmProblem& q, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_kernel<MODE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(kSmemBytes + kTabBytes));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  KArgs a = {};
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
  constexpr bool paired = MODE == GEMM_GATEUP || MODE == GEMM_GU;
  a.ntiles = paired ? (q.N + kBN / 2 - 1) / (kBN / 2) : (q.N + kBN - 1) / kBN;
  a.ldb = q.ldb ? q.ldb : (MODE == GEMM_DUALK ? q.K / 2 : q.K);
  a.k_half = q.K / 2;
  a.gu = static_cast<const bf16_t*>(q.gu);
  a.w_row = q.w_row;
  a.dgu = static_cast<bf16_t*>(q.dgu);
  a.h_out = static_cast<bf16_t*>(q.h_out);
  a.dg_part = q.dg_part;
  a.k_off = q.k_off;
  a.c_group_stride = q.c_group_stride;
  a.C1 = static_cast<bf16_t*>(q.C1);
  a.m_split = q.m_split;
  a.gu_out = static_cast<bf16_t*>(q.gu_out);
  a.C = q.C;
  a.ldc = q.ldc;
  a.bias = q.bias;
  a.a_bytes = (uint32_t)q.a_bytes;
  // Interleaving helps the short-K down projection (small tiles overlap the
  // big ones); for the long-K gate/up GEMM the big tiles are latency-bound
  // and lose more from the shared memory traffic than the overlap gains.
  a.spread_small = MODE == GEMM_DOWN ? 1 : 0;
  if (MODE == GEMM_WGRAD) {
    a.big = a.small = nullptr;
  } else if (q.row_off) {
    a.big = q.tile_prefix;
    a.small = q.tile_prefix + (q.G + 1);
    tile_prefix_kernel<<<1, 1024, 0, s>>>(q.row_off, q.G, q.tile_prefix, q.tile_prefix + (q.G + 1));
  } else {
    a.big = a.small = nullptr;
    a.G = 1;
    tiles_of(q.M, a.single_big, a.single_small);
  }
  const int wg = gemm_grid(num_cus());
  gemm_bf16_kernel<MODE><<<(unsigned)wg, kThreads, kSmemBytes + kTabBytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmProblem& q, hipStream_t s) {
  if (q.K % kBK != 0 || q.G > kMaxGroups) return hipErrorInvalidValue;
  switch (q.mode) {
    case GEMM_GATEUP:
      if (q.N % 8 != 0) return hipErrorInvalidValue;
      return run_grouped<GEMM_GATEUP>(q, s);
    case GEMM_DOWN:
      if (q.N % 8 != 0) return hipErrorInvalidValue;
      return run_grouped<GEMM_DOWN>(q, s);
    case GEMM_GU:
      if (q.N % 32 != 0) return hipErrorInvalidValue;
      return run_grouped<GEMM_GU>(q, s);
    case GEMM_SWIGLU_BWD:
      if (q.N % 32 != 0 || !q.gu || !q.dgu) return hipErrorInvalidValue;
      return run_grouped<GEMM_SWIGLU_BWD>(q, s);
    case GEMM_DUALK:
      if (q.N % 8 != 0 || (q.K / 2) % kBK != 0) return hipErrorInvalidValue;
      return run_grouped<GEMM_DUALK>(q, s);
    case GEMM_WGRAD:
      if (q.N % 8 != 0 || !q.k_off || q.G < 1) return hipErrorInvalidValue;
      // with a second output: two halves of M/2 rows each, the group stride of both
      if (q.C1 && (q.M != 2 * q.m_split || q.c_group_stride != q.m_split * (int64_t)q.N)) return hipErrorInvalidValue;
      return run_grouped<GEMM_WGRAD>(q, s);
    default: {
      if (q.row_off) return hipErrorInvalidValue;
      KArgs a = {};
      a.A = static_cast<const bf16_t*>(q.A);
      a.lda = q.lda;
      a.M = q.M;
      a.B0 = static_cast<const bf16_t*>(q.B0);
      a.N = q.N;
      a.K = q.K;
      a.C = q.C;
      a.ldc = q.ldc;
      a.bias = q.bias;
      a.rowabs = q.rowabs;
      a.rowabs_stride = q.rowabs_stride;
      const dim3 grid((unsigned)((q.M + 63) / 64), (unsigned)((q.N + 63) / 64));
      if (a.rowabs) gemm_bf16_logits_kernel<<<grid, 256, 0, s>>>(a);
      else gemm_bf16_small_n_kernel<<<grid, 256, 0, s>>>(a);
      return hipGetLastError();
    }
  }
}

}  // namespace moe
