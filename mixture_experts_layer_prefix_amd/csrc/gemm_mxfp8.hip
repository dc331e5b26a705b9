// Expert-grouped MXFP8 GEMMs on gfx950 scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, E8M0 block scales).
//
// Mixture-of-Kittens blog post, "Other features / MXFP8 support": routed
// experts run in MXFP8 (the shared expert stays BF16), weights are
// pre-quantized, and activation quantization is fused into the dispatch, the
// grouped GEMMs and the SwiGLU.  Block format: OCP MX v1.0 (the MX paper
// cited by the pages): 32 E4M3 values along K share one E8M0 scale.
//
// C[rows of g] = A[rows of g] . B[g]^T with both operands stored K-major as
// bytes plus a [rows][K/32] scale array.  The structure follows the bf16
// kernel (csrc/gemm_bf16.hip): a persistent grid with device-built lists of
// 256 x 256 and 64 x 256 tiles, 8 waves of 128 x 64 (4 x 2 MFMA blocks),
// direct buffer -> LDS slabs with the same conflict-free swizzle.  A slab is
// 128 K-elements = 128 bytes per row, so one 32x32x64 MFMA consumes half a
// slab row: each lane holds 32 bytes of one row (two 16-byte LDS reads, see
// read_frags for the operand layout) and the E8M0 scale of its lane group's
// 32-element block.  Scales travel through LDS with the data (one dword,
// four blocks, per row and slab).
//
// Gate/up mode writes h = SiLU(G) * U quantized along I (the down GEMM's K):
// the 32 values of one 32-column block of a row sit in 32 lanes of a wave;
// each lane quad transposes a 4 x 4 block so that a lane holds four adjacent
// columns of one row, the block maximum is a local maximum of four values
// plus three cross-lane steps, and each lane encodes and stores its four
// codes as one dword (blog post, "MXFP8 support": quantization fused into the
// SwiGLU).
#include "common.h"

namespace moe {

namespace {

constexpr int kBKB = 128;  // K elements (bytes) per slab
constexpr int kBigM = 256, kSmallM = 64, kBN = 256;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr int stage_bytes(int bm) { return bm * kBKB + kBN * kBKB + bm * 4 + kBN * 4; }
// Every LDS-DMA destination (16-byte data rows, 4-byte scale dwords) stays
// aligned to its transfer size when the stages are laid out back to back.
static_assert(stage_bytes(256) % 16 == 0 && stage_bytes(64) % 16 == 0 && kBKB % 16 == 0, "LDS-DMA alignment");
constexpr size_t kSmemBytes = 2 * stage_bytes(kBigM) > 3 * stage_bytes(kSmallM) ? 2 * stage_bytes(kBigM)
                                                                                 : 3 * stage_bytes(kSmallM);
// Group tables in LDS after the slab ring (see the bf16 kernel).
constexpr int kMaxGroups = 1024;
constexpr size_t kTabBytes = 3ull * (kMaxGroups + 1) * sizeof(int32_t);

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void tiles_of(int64_t rows, int& nb, int& ns) {
  int64_t b = rows / kBigM, r = rows - b * kBigM;
  if (r > kBigM / 2) {
    ++b;
    r = 0;
  }
  nb = (int)b;
  ns = (int)((r + kSmallM - 1) / kSmallM);
}

__global__ void __launch_bounds__(1024) mx_tile_prefix_kernel(const int32_t* __restrict__ row_off, int G,
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

struct MxArgs {
  const uint8_t* A;
  const uint8_t* As;        // A scales [rows][lda/32]
  const int32_t* a_rows;
  const uint8_t* As_slab;   // optional slab-major A scales in row order (gathered rows)    // optional gather of A rows (and their scales)
  uint32_t a_bytes, as_bytes;  // sizes of A and its scales when gathered
  int64_t lda;              // bytes per A row
  const int32_t* row_off;
  int64_t M;
  int G;
  const uint8_t* B0;
  const uint8_t* B1;
  const uint8_t* B0s;
  const uint8_t* B1s;
  int64_t b_stride;         // bytes between experts in B
  int64_t ldb;              // bytes per B row
  int N, K, ntiles;
  int k_half;               // DUALK: K of the first matrix
  void* C;                  // gate/up: E4M3 h [rows][N]; others: bf16 [rows][N] (G|U: [rows][2N])
  uint8_t* Cs;              // gate/up: h scales [rows][N/32]
  int64_t ldc;
  const int32_t* big;
  const int32_t* small;
  int spread_small;
  // SwiGLU backward epilogue
  const bf16_t* gu;         // [rows][2N] G | U
  const float* w_row;       // [rows] router weight (nullptr: 1)
  bf16_t* dgu;              // [rows][2N] dG | dU (bf16)
  uint8_t* dguq;            // [rows][2N] dG | dU quantized along the columns
  uint8_t* dgus;            // [rows][2N/32] their scales
  uint8_t* dgu_t;           // [dG^T; dU^T], E4M3 along the routed rows, expert-blocked (see the epilogue)
  uint8_t* dgu_ts;          // their scales
  uint8_t* gh_t;            // (w h)^T, the same layout (N rows)
  uint8_t* gh_ts;
  const int32_t* pad_off;   // [G+1] padded row offsets of the groups (multiples of 128)
  int64_t t_ld;             // padded rows of all groups
  float* dg_part;           // [rows][N/32]
  // K-grouped weight-gradient mode
  const int32_t* k_off;
  int64_t c_group_stride;
  bf16_t* C1;               // optional second output: rows [m_split, M) of every group
  int64_t m_split;
  bf16_t* gu_out;           // gate/up: optional [rows][2N] G | U output
};

__device__ __forceinline__ int find_group(const int32_t* prefix, int G, int mt) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// 4 x 4 transpose inside each lane quad: lane j of the quad enters with
// v[k] = element (k, j) and leaves with v[k] = element (j, k).  Two exchange
// steps (partner lane j ^ 1, then j ^ 2), each swapping the two elements whose
// index bit differs from the lane's.
__device__ __forceinline__ void quad_transpose4(float (&v)[4], int j) {
  const bool odd = j & 1;
  const float ra = dpp_f32<0xB1>(odd ? v[0] : v[1]);  // quad_perm [1, 0, 3, 2]
  const float rb = dpp_f32<0xB1>(odd ? v[2] : v[3]);
  if (odd) {
    v[0] = ra;
    v[2] = rb;
  } else {
    v[1] = ra;
    v[3] = rb;
  }
  const bool hi = j & 2;
  const float rc = dpp_f32<0x4E>(hi ? v[0] : v[2]);  // quad_perm [2, 3, 0, 1]
  const float rd = dpp_f32<0x4E>(hi ? v[1] : v[3]);
  if (hi) {
    v[0] = rc;
    v[1] = rd;
  } else {
    v[2] = rc;
    v[3] = rd;
  }
}

// Load state of one output tile: buffer descriptors over its operands and
// the per-lane byte offsets (the K position rides in the scalar offset).
// Built once per tile, so the next tile's first slabs can be issued while the
// current tile finishes.
template <int BM>
struct MxLoad {
  __amdgpu_buffer_rsrc_t ar, asr, br0, br1, bsr0, bsr1;
  uint32_t aoff[BM / (kThreads / 8)];
  uint32_t scoff, boff;
  uint32_t sa_slab, sb_slab;  // bytes between the scale dwords of consecutive slabs (0: row-major A scales)
  int k_begin, brows, ldb;
};

template <int BM, int MODE>
__device__ __forceinline__ void mx_setup(const MxArgs& p, MxLoad<BM>& L, int g, int64_t row_begin, int64_t n_g,
                                         int64_t m0, int ntile, int k_begin, int kp = 0) {
  constexpr int BN = kBN;
  constexpr int RPR = kThreads / 8;
  constexpr int AR = BM / RPR;
  constexpr bool PAIRED = MODE == GEMM_GATEUP || MODE == GEMM_GU;
  constexpr bool DUAL = MODE == GEMM_DUALK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = wave * 8 + (lane >> 3);
  const int chunk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  // Weight-gradient operands are stored expert-blocked: group g's A rows are
  // a contiguous [M][Kp] block at byte koff[g] * M (B alike with N rows), Kp
  // its padded row count, so a tile's K slabs are dense (few pages per slab).
  constexpr bool KGROUPED = MODE == GEMM_WGRAD;
  int64_t lda = KGROUPED ? (int64_t)kp : p.lda;
  int64_t ldb = KGROUPED ? (int64_t)kp : p.ldb;
  asm volatile("" : "+s"(lda), "+s"(ldb));
  const int64_t ldas = lda / 32, ldbs = ldb / 32;  // scale bytes per A / B row
  const uint8_t* Ab = KGROUPED ? p.A + (int64_t)k_begin * p.M : p.A;
  const uint8_t* Asb = KGROUPED ? p.As + (int64_t)k_begin * p.M / 32 : p.As;
  const uint8_t* Bb0 = KGROUPED ? p.B0 + (int64_t)k_begin * p.N : p.B0;
  const uint8_t* Bsb0 = KGROUPED ? p.B0s + (int64_t)k_begin * p.N / 32 : p.B0s;
  L.k_begin = KGROUPED ? 0 : k_begin;
  L.ldb = (int)ldb;

  // A data and scales: the tile's rows (or gathered token rows; then the
  // descriptors span the whole gather source).
  const bool gath = p.a_rows != nullptr;
  const int64_t tile_rows = min<int64_t>(BM, n_g - m0);
  const uint8_t* abase = uniform_ptr(gath ? p.A : Ab + (row_begin + m0) * lda);
  // A scales: row-major [rows][K/32] for token rows (gathered or permuted
  // by the caller), slab-major [K/128][M][4] for the operands the layer
  // writes itself (h, dG|dU, the weight-gradient operands per group): a
  // row's dword of one slab at row * 4, slabs M * 4 bytes apart.
  // Gathered token rows may bring their scales already slab-major in row
  // order (As_slab); the data rows are still gathered.
  const bool a_slab = KGROUPED || p.As_slab != nullptr || (!gath && (MODE == GEMM_DOWN || MODE == GEMM_DUALK));
  const bool sgath = gath && p.As_slab == nullptr;  // per-row gathered scale loads
  const uint8_t* Asl = p.As_slab ? p.As_slab : Asb;
  const uint8_t* asbase =
      uniform_ptr(sgath ? p.As : a_slab ? Asl + (row_begin + m0) * 4 : Asb + (row_begin + m0) * ldas);
  const uint32_t abytes = __builtin_amdgcn_readfirstlane(gath ? p.a_bytes : (uint32_t)(tile_rows * lda));
  const uint32_t asbytes = __builtin_amdgcn_readfirstlane(
      sgath ? p.as_bytes : a_slab ? (uint32_t)(ldas * p.M - (row_begin + m0) * 4) : (uint32_t)(tile_rows * ldas));
  L.sa_slab = a_slab ? (uint32_t)(p.M * 4) : 0;
  L.ar = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, (int)abytes, 0x00020000);
  L.asr = __builtin_amdgcn_make_buffer_rsrc((void*)asbase, (short)0, (int)asbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int64_t lr0 = i * RPR + lrow;
    const int64_t lr = lr0 < tile_rows ? lr0 : 0;
    const int64_t src = gath ? (int64_t)p.a_rows[row_begin + m0 + lr] : lr;
    L.aoff[i] = (uint32_t)(src * lda) + chunk * 16;
  }
  // Scale loads: waves 0..BM/64-1 fetch 64 A-scale rows each, waves 4..7 fetch
  // 64 B-scale rows each (paired modes: G rows 0-63, 64-127, then U rows).
  constexpr int ASW = BM / 64;
  const bool a_sc = wave < ASW;
  const bool b_sc = wave >= 4;
  uint32_t scoff = 0;
  if (a_sc) {
    const int64_t lr0 = wave * 64 + lane;
    const int64_t lr = lr0 < tile_rows ? lr0 : 0;
    const int64_t src = sgath ? (int64_t)p.a_rows[row_begin + m0 + lr] : lr;
    scoff = (uint32_t)(src * (a_slab ? 4 : ldas));
  }
  const int bi = wave - 4;  // B-scale round of this wave
  const int span = PAIRED ? BN / 2 : BN;
  const int first_row = ntile * span;          // first B row of this N-tile
  const int brows = min(span, p.N - first_row);
  L.brows = brows;
  if (b_sc) {
    const int r = PAIRED ? (bi & 1) * 64 + lane : bi * 64 + lane;
    scoff = (uint32_t)(min(r, brows - 1) * 4);
  }
  L.scoff = scoff;
  // B scales are slab-major: [K/128][G*N][4] for the stacked weights (one
  // matrix of G*N rows; DUALK: each of the two), [Kp/128][N][4] per group for
  // the weight-gradient operands.
  const int gs = KGROUPED ? 1 : p.G;
  const int64_t brow0 = (int64_t)(KGROUPED ? 0 : g) * p.N + first_row;
  const uint8_t* bs0 = Bsb0 + brow0 * 4;
  const uint8_t* bs1 = (PAIRED || DUAL) ? p.B1s + brow0 * 4 : bs0;
  const uint32_t bsbytes = __builtin_amdgcn_readfirstlane((uint32_t)(ldbs * gs * p.N - brow0 * 4));
  L.sb_slab = (uint32_t)(gs * p.N * 4);
  L.bsr0 = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(PAIRED && bi >= 2 ? bs1 : bs0), (short)0,
                                            (int)bsbytes, 0x00020000);
  L.bsr1 = DUAL ? __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(bs1), (short)0, (int)bsbytes, 0x00020000)
                : L.bsr0;
  // B data
  const uint8_t* b0 = Bb0 + (int64_t)g * p.b_stride + first_row * ldb;
  const uint8_t* b1 = (PAIRED || DUAL) ? p.B1 + (int64_t)g * p.b_stride + first_row * ldb : b0;
  const uint32_t bbytes = __builtin_amdgcn_readfirstlane((uint32_t)(brows * ldb));
  L.br0 = __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(PAIRED && ((wave >> 2) & 1) ? b1 : b0), (short)0,
                                           (int)bbytes, 0x00020000);
  L.br1 = DUAL ? __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(b1), (short)0, (int)bbytes, 0x00020000)
               : L.br0;
  L.boff = (uint32_t)((lane >> 3) * ldb) + chunk * 16;
}

// Issue the loads of slab k0 (relative to the tile's K start) into stage st.
template <int BM, int MODE>
__device__ __forceinline__ void mx_issue(const MxArgs& p, const MxLoad<BM>& L, uint8_t* smem, int st, int k0) {
  constexpr int BN = kBN;
  constexpr int RPR = kThreads / 8;
  constexpr int AR = BM / RPR, BR = BN / RPR;
  constexpr int STG = stage_bytes(BM);
  constexpr bool PAIRED = MODE == GEMM_GATEUP || MODE == GEMM_GU;
  constexpr bool DUAL = MODE == GEMM_DUALK;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ldb = L.ldb;
  uint8_t* S = smem + st * STG;
  const int ka = L.k_begin + k0;
#pragma unroll
  for (int i = 0; i < AR; ++i)
    lds_dma<16>(L.ar, S + (i * RPR + wave * 8) * kBKB, L.aoff[i], ka);
  const bool second = DUAL && k0 >= p.k_half;
  const int kb = DUAL ? (second ? k0 - p.k_half : k0) : ka;
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    int r0 = PAIRED ? i * (RPR / 2) + (wave & 3) * 8 : i * RPR + wave * 8;
    r0 = min(r0, L.brows - 8);
    lds_dma<16>(second ? L.br1 : L.br0, S + BM * kBKB + (i * RPR + wave * 8) * kBKB, L.boff, (uint32_t)(r0 * ldb + kb));
  }
  // Scale dwords: row-major operands at K / 32 in the row, slab-major ones
  // at slab * (bytes per slab).
  const uint32_t sa_off = L.sa_slab ? (uint32_t)(ka >> 7) * L.sa_slab : (uint32_t)(ka / 32);
  const uint32_t sb_off = (uint32_t)(kb >> 7) * L.sb_slab;
  if (wave < BM / 64)
    lds_dma<4>(L.asr, S + (BM + BN) * kBKB + wave * 256, L.scoff, sa_off);
  if (wave >= 4)
    lds_dma<4>(second ? L.bsr1 : L.bsr0, S + (BM + BN) * kBKB + BM * 4 + (wave - 4) * 256, L.scoff, sb_off);
}

// One BM x 256 output tile whose load state L is set up.  prefetched: its
// first min(NS, KT) slabs were already issued (by the previous tile).  nxt:
// the next tile of this workgroup (or nullptr), whose first slabs are issued
// once this tile's last slab barrier has freed the LDS ring.
// Background zero fill of the weight gradients of experts without rows
// (K-grouped mode).  The dense [M][N] outputs of those experts are cut into
// 1 KiB chunks; every wave owns a contiguous run of them and stores
// kZeroPerSlab chunks just before each slab it issues inside a K loop, so
// the stores drain under the MFMA work instead of queueing as zero tiles at
// the end of the launch; the wave stores what is left once its tiles are
// done.
constexpr int kZeroPerSlab = 2;
struct ZeroRun {
  const int32_t* empty;  // LDS: ids of the experts without rows
  int slot, off, cpr;    // current expert (index into empty), chunk in it, chunks per expert
  int64_t left;          // chunks still to store
};
__device__ __forceinline__ void zero_chunk(const MxArgs& p, ZeroRun& z, int lane) {
  const int64_t e = z.empty[z.slot];
  int64_t off = (int64_t)z.off * 1024;
  bf16_t* Cg = static_cast<bf16_t*>(p.C);
  if (p.C1 && off >= p.m_split * p.N * 2) {  // split output: chunks never straddle (host-checked)
    Cg = p.C1;
    off -= p.m_split * p.N * 2;
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(Cg + e * p.c_group_stride);
  __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, reinterpret_cast<u32x4*>(base + off + lane * 16));
  if (++z.off == z.cpr) z.off = 0, ++z.slot;
  --z.left;
}

template <int BM, int MODE, int NS>
__device__ __forceinline__ void mx_tile(const MxArgs& p, uint8_t* smem, const MxLoad<BM>& L, int g,
                                        int64_t row_begin, int64_t n_g, int64_t m0, int ntile, int KT,
                                        bool prefetched, bool has_next, const MxLoad<BM>& nxt, int nxt_KT,
                                        ZeroRun* zr = nullptr) {
  constexpr int BN = kBN;
  constexpr int WM = BM / kWavesM, WN = BN / kWavesN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int RPR = kThreads / 8;  // rows per data load round
  constexpr int AR = BM / RPR, BR = BN / RPR;
  constexpr int STG = stage_bytes(BM);
  constexpr int LPS = AR + BR;       // data loads per slab per thread (+1 scale load on most waves)
  constexpr bool PAIRED = MODE == GEMM_GATEUP || MODE == GEMM_GU;
  static_assert(FN == 2, "wave tile");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int64_t tile_rows = min<int64_t>(BM, n_g - m0);
  auto issue = [&](int st, int k0) { mx_issue<BM, MODE>(p, L, smem, st, k0); };
  const bool any_sc = wave < BM / 64 || wave >= 4;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  i32x8 fa[FM], fb[FN];
  int sa[FM], sb[FN];
  auto read_frags = [&](int st, int kk) {
    const uint8_t* S = smem + st * STG;
    // Operand layout of the 32x32x64 MFMA: lane group g = lane / 32 holds
    // K[16g, 16g+16) in its low 16 bytes and K[32+16g, 32+16g+16) in its high
    // 16 bytes; the scale of group g covers K[32g, 32g+32).
    const int c0 = kk * 4 + (lane >> 5), c1 = c0 + 2;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + i * 32 + (lane & 31);
      const u32x4 lo = *reinterpret_cast<const u32x4*>(S + r * kBKB + ((c0 ^ swz(r)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(S + r * kBKB + ((c1 ^ swz(r)) << 4));
      fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WN + j * 32 + (lane & 31);
      const uint8_t* Bb = S + BM * kBKB;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(Bb + r * kBKB + ((c0 ^ swz(r)) << 4));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(Bb + r * kBKB + ((c1 ^ swz(r)) << 4));
      fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  auto read_scales = [&](int st) {
    const uint8_t* S = smem + st * STG + (BM + BN) * kBKB;
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = *reinterpret_cast<const int*>(S + (wm * WM + i * 32 + (lane & 31)) * 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = PAIRED ? (j ? 128 : 0) + wn * 32 + (lane & 31) : wn * WN + j * 32 + (lane & 31);
      sb[j] = *reinterpret_cast<const int*>(S + BM * 4 + r * 4);
    }
  };
  auto mma = [&](int kk) {
    const int sh = 8 * (kk * 2 + (lane >> 5));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0,
                                                                    (sa[i] >> sh) & 0xFF, 0, (sb[j] >> sh) & 0xFF);
  };

  if (!prefetched) {
    wait_vmcnt<0>();
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0)
      if (s0 < KT) issue(s0, s0 * kBKB);
  }
  if (KT >= NS) {
    if (any_sc) wait_vmcnt<(NS - 1) * (LPS + 1)>(); else wait_vmcnt<(NS - 1) * LPS>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  // Keep the first half-slab's MFMAs ahead of the slab barrier: they only feed
  // later MFMAs, and without this pin the compiler sinks them below the
  // barrier, leaving the LDS reads of every slab exposed.
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  // background zero stores (K-grouped mode; the waits below assume one slab in flight)
  constexpr bool ZB = MODE == GEMM_WGRAD && NS == 2;
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % NS;
    read_scales(st);
    read_frags(st, 0);
    mma(0);
    read_frags(st, 1);
    pin_acc();
    mma(1);
    if (kt + NS - 1 < KT) {
      if constexpr (ZB) {
        // The zero stores went out before slab kt + 1's loads, which are the
        // youngest operations in flight: wait for everything (no assumption
        // about the completion order of stores and loads).
        wait_vmcnt<0>();
      } else {
        if (any_sc) wait_vmcnt<(NS - 2) * (LPS + 1)>(); else wait_vmcnt<(NS - 2) * LPS>();
      }
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (kt + NS < KT) {
      if constexpr (ZB) {
        // background zero stores, issued ahead of the next slab's loads
        if (kt + NS < KT - 1 && zr->left >= kZeroPerSlab) {
#pragma unroll
          for (int s = 0; s < kZeroPerSlab; ++s) zero_chunk(p, *zr, lane);
        }
      }
      issue(st, (kt + NS) * kBKB);
    }
  }
  // The ring is free: start the next tile's loads under this epilogue.
  if (has_next) {
#pragma unroll
    for (int s0 = 0; s0 < NS; ++s0)
      if (s0 < nxt_KT) mx_issue<BM, MODE>(p, nxt, smem, s0, s0 * kBKB);
  }

  // Epilogue (32x32 block layout: column lane & 31, rows 8*(v/4) + 4*(lane/32) + v%4).
  int64_t ldc = p.ldc;
  asm volatile("" : "+s"(ldc));
  const int rows_left = (int)tile_rows;
  const int N = p.N;
  if constexpr (MODE == GEMM_DOWN || MODE == GEMM_DUALK || MODE == GEMM_WGRAD) {
    // Plain bf16 output.  One per-lane base pointer; rows step by compile-time
    // multiples of ldc, the two column blocks by an immediate offset.
    // Split K-grouped output: a tile wholly past m_split writes C1; a tile
    // straddling m_split picks the tensor per row (bounds-checked path).
    bf16_t* Cg = static_cast<bf16_t*>(p.C);
    int64_t mrow = row_begin + m0;
    bool straddle = false;
    if (MODE == GEMM_WGRAD && p.C1) {
      if (mrow >= p.m_split) {
        Cg = p.C1;
        mrow -= p.m_split;
      } else {
        straddle = mrow + BM > p.m_split;
      }
    }
    bf16_t* Cb = Cg + (MODE == GEMM_WGRAD ? (int64_t)g * p.c_group_stride : 0) +
                 (mrow + wm * WM + 4 * (lane >> 5)) * ldc + ntile * BN + wn * WN + (lane & 31);
    if (tile_rows == BM && ntile * BN + BN <= N && !straddle) {  // interior tile: no bounds checks
#pragma clang loop unroll(full)
      for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
        for (int v = 0; v < 16; ++v) {
          bf16_t* Cr = Cb + (int64_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * ldc;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            // Weight gradients are not read again by this layer: streaming
            // stores keep them from displacing operand slabs in L2.
            if constexpr (MODE == GEMM_WGRAD) __builtin_nontemporal_store(f32_to_bf16(acc[i][j][v]), &Cr[j * 32]);
            else Cr[j * 32] = f32_to_bf16(acc[i][j][v]);
          }
        }
    } else {
      const int rl0 = wm * WM + 4 * (lane >> 5);
      const int col0 = ntile * BN + wn * WN + (lane & 31);
#pragma clang loop unroll(full)
      for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
        for (int v = 0; v < 16; ++v) {
          const int r = i * 32 + 8 * (v >> 2) + (v & 3);
          if (rl0 + r >= rows_left) continue;
          bf16_t* Cr = Cb + (int64_t)r * ldc;
          if (straddle && mrow + rl0 + r >= p.m_split)  // this row belongs to C1
            Cr = p.C1 + (int64_t)g * p.c_group_stride + (mrow + rl0 + r - p.m_split) * ldc + col0;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (col0 + j * 32 < N) Cr[j * 32] = f32_to_bf16(acc[i][j][v]);
        }
    }
    return;
  }
  if constexpr (MODE == GEMM_SWIGLU_BWD) {
    // dH' -> dG, dU, w h and the partial router-weight gradient <dH', h> per
    // 32-column block.  dG and dU leave in E4M3 twice: along the columns (the
    // gate/up input-gradient GEMM's A operand) and along the routed rows in
    // the expert-blocked transposed layout of the weight-gradient operands
    // (group g: [N][Kp_g] codes at pad_off[g] * N, scales slab-major); w h
    // leaves along the routed rows only (the down weight gradient's operand).
    //
    // The accumulators pass through LDS (the slab ring is idle once the last
    // slab is read), per wave, one 32-row block at a time: element (r, c)
    // of a wave's [PR][64] fp32 region sits at r * 64 + 4 * ((c / 4) ^
    // key(r)) + c % 4; key(r) flips chunk bit 0 with r bit 0 and chunk bit 3
    // with r bits 1 xor 2, which keeps the accumulator-layout writes (rows r,
    // r + 4), the row phase (rows 4m..4m+3, four lanes each) and the column
    // phase (one row, 64 lanes) free of bank conflicts.
    //   Row phase: four lanes share one row's 32-column block, eight columns
    // each (block maxima and sums in two DPP steps, 8- and 16-byte global
    // accesses); each lane writes its eight dG and eight dU, rounded to bf16,
    // back over its eight dH' values (the two 16-byte chunks), and its eight
    // w h in bf16 to a second per-wave [32][64] region (16-byte chunk c of row
    // r at c ^ 4 (r / 2 % 2): rows r, r + 2 share banks).
    //   Column phase: lane (q, pair) takes columns 2 pair, 2 pair + 1 of dG
    // (q = 0) or dU (q = 1) down the 32-row block and writes both columns'
    // 32 codes; lanes 0-31 then do the same for w h.  Rows past the group's
    // end quantize as zeros; the padding rows past the group's last tile are
    // zero-filled by that tile.
    constexpr int PI = 1;                // 32-row blocks per pass
    constexpr int PR = PI * 32;          // rows per pass
    constexpr int ITEMS = PR * FN * 4 / 64;  // (row, block, quarter) items per lane per pass
    constexpr int WREG = PR * 64 * 4 + PR * 64 * 2;  // bytes per wave: fp32 region, then the bf16 w h region
    static_assert(8 * WREG <= (int)kSmemBytes, "staging fits the slab ring");
    // Lane-derived epilogue values are computed here, not hoisted above the
    // K loop where they would hold registers the loop needs.
    int el = lane;
    asm volatile("" : "+v"(el));
    float* stage = reinterpret_cast<float*>(smem + wave * WREG);
    uint32_t* stage_w = reinterpret_cast<uint32_t*>(stage);
    uint32_t* stage_h = reinterpret_cast<uint32_t*>(smem + wave * WREG + PR * 64 * 4);  // [PR][32] dwords
    auto hkey = [](int r) { return ((r >> 1) & 1) << 2; };
    auto skey = [](int r) { return (r & 1) | ((((r >> 2) ^ (r >> 1)) & 1) << 3); };
    const int qt = el & 3;  // row phase: quarter of the block, columns 8 qt .. 8 qt + 7
    const int cq = el >> 5, cp = el & 31;  // column phase: dG / dU, column pair
    const int64_t kp = p.pad_off[g + 1] - p.pad_off[g];
    const int wcol = ntile * BN + wn * WN;  // first of the wave's 64 columns
    const bool wave_cols = wcol < N;        // N is a multiple of 64: all 64 or none
    // This lane's first column in the transposed output, at row 0 of the
    // group (the second column is kp bytes further), and its scale bytes.
    // Group g's block is [2N][kp] at pad_off[g] * 2N: dG^T in its rows
    // [0, N), dU^T in rows [N, 2N) (one weight-gradient operand of 2N rows);
    // scales slab-major, [kp / 128][2N][4] per group, so row rr's block scale
    // of transposed row c sits at (rr / 128) 2N 4 + c 4 + (rr / 32) % 4.
    const int trow = cq * N + wcol + 2 * cp;  // this lane's first row of [dG^T; dU^T]
    uint8_t* tq = p.dgu_t + (int64_t)p.pad_off[g] * 2 * N + (int64_t)trow * kp;
    uint8_t* ts = p.dgu_ts + (int64_t)p.pad_off[g] * 2 * N / 32 + trow * 4;
    auto ts_at = [&](int rr) { return ts + (int64_t)(rr >> 7) * 2 * N * 4 + ((rr >> 5) & 3); };
    // The same for w h (lanes 0-31).
    uint8_t* hq = p.gh_t + (int64_t)p.pad_off[g] * N + (int64_t)(wcol + 2 * cp) * kp;
    uint8_t* hs = p.gh_ts + (int64_t)p.pad_off[g] * N / 32 + (wcol + 2 * cp) * 4;
    auto hs_at = [&](int rr) { return hs + (int64_t)(rr >> 7) * N * 4 + ((rr >> 5) & 3); };
#pragma clang loop unroll(full)
    for (int i0 = 0; i0 < FM; i0 += PI) {
      if (i0) __syncthreads();  // the previous pass's column reads are done
#pragma clang loop unroll(full)
      for (int ii = 0; ii < PI; ++ii)
#pragma clang loop unroll(full)
        for (int v = 0; v < 16; ++v)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int r = ii * 32 + 8 * (v >> 2) + 4 * (el >> 5) + (v & 3);
            const int c = j * 32 + (el & 31);
            stage[r * 64 + (((c >> 2) ^ skey(r)) << 2) + (c & 3)] = acc[i0 + ii][j][v];
          }
      // This pass's G | U and router weights: item k + 1's loads are in flight
      // while item k is processed (the first issued once the pass's
      // accumulators have left their registers).
      u32x4 ngq, nuq;
      float nwr;
      auto load_item = [&](int k) {
        const int rb = (k * 64 + el) >> 2;
        const int r = rb % PR, blk = rb / PR;
        const int tr = wm * WM + i0 * 32 + r;
        const int col = ntile * BN + wn * WN + blk * 32 + 8 * qt;
        ngq = nuq = u32x4{0, 0, 0, 0};
        nwr = 0.0f;
        if (tr < rows_left && col < N) {
          const int64_t grow = row_begin + m0 + tr;
          const int64_t rowoff = grow * (int64_t)(2 * N);
          ngq = *reinterpret_cast<const u32x4*>(p.gu + rowoff + col);
          nuq = *reinterpret_cast<const u32x4*>(p.gu + rowoff + N + col);
          nwr = p.w_row ? p.w_row[grow] : 1.0f;
        }
      };
      load_item(0);
      __syncthreads();
#pragma unroll 1
      for (int k = 0; k < ITEMS; ++k) {
        const int rb = (k * 64 + el) >> 2;
        const int r = rb % PR, blk = rb / PR;
        const int tr = wm * WM + i0 * 32 + r;                    // row in the tile
        const int col = ntile * BN + wn * WN + blk * 32 + 8 * qt;  // first of this lane's 8 columns
        // Rows past the tile end skip their global accesses but keep the
        // quad's reductions in step and stage zeros for the column phase.
        const bool ok = tr < rows_left && col < N;
        const int64_t grow = row_begin + m0 + min(tr, rows_left - 1);
        const int64_t rowoff = grow * (int64_t)(2 * N);  // elements before row grow of the [rows][2N] arrays
        uint32_t* s0 = stage_w + r * 64 + (((blk * 8 + 2 * qt) ^ skey(r)) << 2);
        uint32_t* s1 = stage_w + r * 64 + (((blk * 8 + 2 * qt + 1) ^ skey(r)) << 2);
        const u32x4 gq = ngq, uq = nuq;
        const float wr = nwr;
        if (k + 1 < ITEMS) load_item(k + 1);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(s0), d1 = *reinterpret_cast<const f32x4*>(s1);
        float dg[8], du[8];
        uint32_t hw[4];
        float part = 0.0f;
        uint32_t mg = 0, mu = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t gw = gq[e >> 1], uw = uq[e >> 1];
          const float gv = __uint_as_float((e & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
          const float uv = __uint_as_float((e & 1) ? (uw & 0xFFFF0000u) : (uw << 16));
          const float sg = sigmoid_f32(gv);
          const float sl = gv * sg;
          const float h = sl * uv;
          const float dhp = e < 4 ? d0[e] : d1[e - 4];
          const float dh = wr * dhp;
          dg[e] = dh * uv * sg * (1.0f + gv * (1.0f - sg));
          du[e] = dh * sl;
          part += dhp * h;
          mg = max(mg, __float_as_uint(dg[e]) & 0x7FFFFFFFu);
          mu = max(mu, __float_as_uint(du[e]) & 0x7FFFFFFFu);
          const uint32_t wh = f32_to_bf16(wr * h);
          if (e & 1) hw[e >> 1] |= wh << 16; else hw[e >> 1] = wh;
        }
        // dG, dU in bf16 over this lane's dH', w h to its region (zeros for
        // rows past the end).
        *reinterpret_cast<u32x4*>(s0) = u32x4{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]),
                                              pack_bf16x2(dg[4], dg[5]), pack_bf16x2(dg[6], dg[7])};
        *reinterpret_cast<u32x4*>(s1) = u32x4{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]),
                                              pack_bf16x2(du[4], du[5]), pack_bf16x2(du[6], du[7])};
        *reinterpret_cast<u32x4*>(stage_h + r * 32 + (((blk * 4 + qt) ^ hkey(r)) << 2)) =
            u32x4{hw[0], hw[1], hw[2], hw[3]};
        // Reductions over the quad (the row's 32 columns).
        mg = max(mg, dpp_u32<0xB1>(mg));
        mg = max(mg, dpp_u32<0x4E>(mg));
        mu = max(mu, dpp_u32<0xB1>(mu));
        mu = max(mu, dpp_u32<0x4E>(mu));
        part += dpp_f32<0xB1>(part);
        part += dpp_f32<0x4E>(part);
        if (!ok) continue;
        const int eg = mx_block_exp_bits(mg), eu = mx_block_exp_bits(mu);
        const float ig = mx_inv_scale(eg), iu = mx_inv_scale(eu);

        uint8_t* qrow = p.dguq + rowoff + col;
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2*>(qrow) = u32x2{e4m3x4_rne_sat(dg[0] * ig, dg[1] * ig, dg[2] * ig, dg[3] * ig),
                                                e4m3x4_rne_sat(dg[4] * ig, dg[5] * ig, dg[6] * ig, dg[7] * ig)};
        *reinterpret_cast<u32x2*>(qrow + N) = u32x2{e4m3x4_rne_sat(du[0] * iu, du[1] * iu, du[2] * iu, du[3] * iu),
                                                    e4m3x4_rne_sat(du[4] * iu, du[5] * iu, du[6] * iu, du[7] * iu)};
        if (qt == 0) {
          // dG | dU scales slab-major over the 2N columns, [2N/128][rows][4]
          // (the gate/up input-gradient GEMM's A layout).
          p.dgus[(((int64_t)(col >> 7) * p.M + grow) << 2) + ((col >> 5) & 3)] = (uint8_t)(eg + 127);
          p.dgus[(((int64_t)((N + col) >> 7) * p.M + grow) << 2) + (((N + col) >> 5) & 3)] = (uint8_t)(eu + 127);
          if (p.dg_part) p.dg_part[(rowoff >> 6) + col / 32] = part;
        }
      }
      __syncthreads();  // dG, dU of the pass are staged
      // Column phase: this pass's 32-row blocks along the routed rows.
#pragma unroll
      for (int b = 0; b < PI; ++b) {
        const int rr0 = (int)m0 + wm * WM + i0 * 32 + 32 * b;  // group row of the block's first row
        if (!wave_cols || rr0 >= kp) continue;
        uint32_t x[32];
        uint32_t m0b = 0, m1b = 0;
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const int r = 32 * b + q;
          const int chunk = ((cp >> 4) * 8 + 2 * ((cp & 15) >> 2) + cq) ^ skey(r);
          x[q] = stage_w[r * 64 + (chunk << 2) + (cp & 3)];
          m0b = max(m0b, (x[q] << 16) & 0x7FFFFFFFu);
          m1b = max(m1b, x[q] & 0x7FFF0000u);
        }
        const int e0 = mx_block_exp_bits(m0b), e1 = mx_block_exp_bits(m1b);
        const float i0s = mx_inv_scale(e0), i1s = mx_inv_scale(e1);
        u32x4 c0[2], c1[2];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int q = 4 * w;
          c0[w >> 2][w & 3] = e4m3x4_rne_sat(__uint_as_float(x[q] << 16) * i0s, __uint_as_float(x[q + 1] << 16) * i0s,
                                             __uint_as_float(x[q + 2] << 16) * i0s, __uint_as_float(x[q + 3] << 16) * i0s);
          c1[w >> 2][w & 3] = e4m3x4_rne_sat(__uint_as_float(x[q] & 0xFFFF0000u) * i1s,
                                             __uint_as_float(x[q + 1] & 0xFFFF0000u) * i1s,
                                             __uint_as_float(x[q + 2] & 0xFFFF0000u) * i1s,
                                             __uint_as_float(x[q + 3] & 0xFFFF0000u) * i1s);
        }
        uint8_t* o0 = tq + rr0;
        *reinterpret_cast<u32x4*>(o0) = c0[0];
        *reinterpret_cast<u32x4*>(o0 + 16) = c0[1];
        *reinterpret_cast<u32x4*>(o0 + kp) = c1[0];
        *reinterpret_cast<u32x4*>(o0 + kp + 16) = c1[1];
        uint8_t* s0 = ts_at(rr0);
        s0[0] = (uint8_t)(e0 + 127);
        s0[4] = (uint8_t)(e1 + 127);
        if (el < 32) {  // w h: columns 2 cp, 2 cp + 1
          uint32_t hm0 = 0, hm1 = 0;
#pragma unroll
          for (int q = 0; q < 32; ++q) {
            const int r = 32 * b + q;
            x[q] = stage_h[r * 32 + (((cp >> 2) ^ hkey(r)) << 2) + (cp & 3)];
            hm0 = max(hm0, (x[q] << 16) & 0x7FFFFFFFu);
            hm1 = max(hm1, x[q] & 0x7FFF0000u);
          }
          const int f0 = mx_block_exp_bits(hm0), f1 = mx_block_exp_bits(hm1);
          const float j0s = mx_inv_scale(f0), j1s = mx_inv_scale(f1);
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int q = 4 * w;
            c0[w >> 2][w & 3] =
                e4m3x4_rne_sat(__uint_as_float(x[q] << 16) * j0s, __uint_as_float(x[q + 1] << 16) * j0s,
                               __uint_as_float(x[q + 2] << 16) * j0s, __uint_as_float(x[q + 3] << 16) * j0s);
            c1[w >> 2][w & 3] = e4m3x4_rne_sat(__uint_as_float(x[q] & 0xFFFF0000u) * j1s,
                                               __uint_as_float(x[q + 1] & 0xFFFF0000u) * j1s,
                                               __uint_as_float(x[q + 2] & 0xFFFF0000u) * j1s,
                                               __uint_as_float(x[q + 3] & 0xFFFF0000u) * j1s);
          }
          uint8_t* h0 = hq + rr0;
          *reinterpret_cast<u32x4*>(h0) = c0[0];
          *reinterpret_cast<u32x4*>(h0 + 16) = c0[1];
          *reinterpret_cast<u32x4*>(h0 + kp) = c1[0];
          *reinterpret_cast<u32x4*>(h0 + kp + 16) = c1[1];
          uint8_t* hs0 = hs_at(rr0);
          hs0[0] = (uint8_t)(f0 + 127);
          hs0[4] = (uint8_t)(f1 + 127);
        }
      }
    }
    // Padding rows [m0 + BM, Kp_g) after the group's last tile (a single
    // 64-row tile whose group's row count ends within its first 64 rows of a
    // 128-row padding unit): zero codes and scales.
    if (wm == 0 && wave_cols && m0 + BM < kp && m0 + BM >= n_g) {
      for (int rr = (int)m0 + BM; rr < kp; rr += 32) {
        uint8_t* o0 = tq + rr;
        *reinterpret_cast<u32x4*>(o0) = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(o0 + 16) = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(o0 + kp) = u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4*>(o0 + kp + 16) = u32x4{0, 0, 0, 0};
        uint8_t* s0 = ts_at(rr);
        s0[0] = 0;
        s0[4] = 0;
        if (el < 32) {
          uint8_t* h0 = hq + rr;
          *reinterpret_cast<u32x4*>(h0) = u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>(h0 + 16) = u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>(h0 + kp) = u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>(h0 + kp + 16) = u32x4{0, 0, 0, 0};
          uint8_t* hs0 = hs_at(rr);
          hs0[0] = 0;
          hs0[4] = 0;
        }
      }
    }
    return;
  }
  if constexpr (MODE == GEMM_GATEUP) {
    // h = SiLU(G) * U of column block wn of this tile (lane & 31 the column;
    // lanes 0-31 rows 8 (v / 4) + v % 4, lanes 32-63 four rows further),
    // quantized per row over its 32 columns.  Each lane quad (four adjacent
    // columns) transposes its 4 x 4 block of four consecutive rows, so that a
    // lane holds four adjacent columns of one row: the row's block maximum is
    // the maximum over those four values and over the eight quads of the
    // half-wave that hold the same row (DPP rotations by 4 and 8 inside each
    // 16-lane row, then the half's two rows swapped), and the four codes leave
    // as one dword.  The codes and scales are those of one lane per element.
    uint8_t* C = static_cast<uint8_t*>(p.C);
    const int jq = lane & 3;
    const int colq = ntile * (BN / 2) + wn * 32 + (lane & 28);  // the quad's first column
#pragma clang loop unroll(full)
    for (int i = 0; i < FM; ++i) {
#pragma clang loop unroll(full)
      for (int a = 0; a < 4; ++a) {
        float hv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) hv[k] = silu_f32(acc[i][0][4 * a + k]) * acc[i][1][4 * a + k];
        if (p.gu_out) {  // G | U kept for the backward
          const int col = ntile * (BN / 2) + wn * 32 + (lane & 31);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rl = wm * WM + i * 32 + 8 * a + 4 * (lane >> 5) + k;
            if (rl < rows_left && col < N) {
              const int64_t grow = row_begin + m0 + rl;
              p.gu_out[grow * 2 * N + col] = f32_to_bf16(acc[i][0][4 * a + k]);
              p.gu_out[grow * 2 * N + N + col] = f32_to_bf16(acc[i][1][4 * a + k]);
            }
          }
        }
        quad_transpose4(hv, jq);
        uint32_t mb = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) mb = max(mb, __float_as_uint(hv[k]) & 0x7FFFFFFFu);
        mb = max(mb, dpp_u32<0x124>(mb));  // row_ror:4
        mb = max(mb, dpp_u32<0x128>(mb));  // row_ror:8
        const auto sw = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);
        mb = max((uint32_t)sw[0], (uint32_t)sw[1]);
        const int e = mx_block_exp_bits(mb);
        const float inv = mx_inv_scale(e);
        const uint32_t code = e4m3x4_rne_sat(hv[0] * inv, hv[1] * inv, hv[2] * inv, hv[3] * inv);
        const int rl = wm * WM + i * 32 + 8 * a + 4 * (lane >> 5) + jq;
        if (rl < rows_left && colq < N) {
          const int64_t grow = row_begin + m0 + rl;
          *reinterpret_cast<uint32_t*>(C + grow * ldc + colq) = code;
          // h scales slab-major [I/128][rows][4] (the down GEMM's A layout)
          if ((lane & 28) == 0)
            p.Cs[(((int64_t)(colq >> 7) * p.M + grow) << 2) + ((colq >> 5) & 3)] = (uint8_t)(e + 127);
        }
      }
    }
    return;
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < FM; ++i) {
#pragma clang loop unroll(full)
    for (int v = 0; v < 16; ++v) {
      const int rl = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const bool row_ok = rl < rows_left;
      const int64_t grow = row_begin + m0 + (row_ok ? rl : rows_left - 1);
      if constexpr (MODE == GEMM_GU) {
        const int col = ntile * (BN / 2) + wn * 32 + (lane & 31);
        if (row_ok && col < N) {
          bf16_t* C = static_cast<bf16_t*>(p.C) + grow * ldc;
          C[col] = f32_to_bf16(acc[i][0][v]);
          C[N + col] = f32_to_bf16(acc[i][1][v]);
        }
      }
    }
  }
}


template <int MODE>
__global__ void __launch_bounds__(kThreads, 1) gemm_mxfp8_kernel(MxArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_mx[];
  int32_t* tab = reinterpret_cast<int32_t*>(smem_mx + kSmemBytes);
  const int32_t* t_big = tab;
  const int32_t* t_small = tab + (p.G + 1);
  const int32_t* t_row = tab + 2 * (p.G + 1);
  if (MODE == GEMM_WGRAD) {
    for (int i = threadIdx.x; i <= p.G; i += kThreads) tab[i] = p.k_off[i];
  } else {
    for (int i = threadIdx.x; i <= p.G; i += kThreads) {
      tab[i] = p.big[i];
      tab[p.G + 1 + i] = p.small[i];
      tab[2 * (p.G + 1) + i] = p.row_off[i];
    }
  }
  __syncthreads();
  const int nwg = gridDim.x;
  const int per_xcd = nwg >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  if constexpr (MODE == GEMM_WGRAD) {
    // One output per group, all in big tiles; K range of group g from k_off.
    // Groups without rows come last in the order and get no tiles: their
    // outputs are zero-filled in the background (ZeroRun).  Every tile's
    // first slabs are issued by the previous tile of this workgroup
    // (lookahead).
    const WgradRect rc = wgrad_rect((int)((p.M + kBigM - 1) / kBigM), p.ntiles, xcd);
    const int per_g = rc.bm * rc.bn;
    int32_t* order = tab + (p.G + 1);
    wgrad_order(tab, p.G, order);
    __syncthreads();
    int n_act = 0, hi = p.G;  // groups with rows: a prefix of the order
    while (n_act < hi) {
      const int mid = (n_act + hi) >> 1, g = order[mid];
      if (tab[g + 1] > tab[g]) n_act = mid + 1; else hi = mid;
    }
    n_act = __builtin_amdgcn_readfirstlane(n_act);
    const int tot = n_act * per_g;
    ZeroRun zr;
    {
      const int64_t cpr = p.M * (int64_t)p.N * 2 / 1024;
      const int64_t ztot = (p.G - n_act) * cpr;
      const int64_t nw = (int64_t)nwg * (kThreads / 64);
      const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      const int64_t z0 = uniform_i64(ztot * w / nw), z1 = uniform_i64(ztot * (w + 1) / nw);
      zr.empty = order + n_act;
      zr.cpr = (int)cpr;
      zr.slot = (int)(z0 / cpr);
      zr.off = (int)(z0 - (int64_t)zr.slot * cpr);
      zr.left = z1 - z0;
    }
    auto zero_rest = [&]() {
      const int lane = threadIdx.x & 63;
      while (zr.left > 0) zero_chunk(p, zr, lane);
    };
    struct Job { int g, mt, nt, kb, kt; };
    auto job = [&](int P) {
      Job j;
      const int gi = P / per_g;
      j.g = __builtin_amdgcn_readfirstlane(order[gi]);
      const int r = P - gi * per_g;
      const int rm = r / rc.bn;
      j.mt = __builtin_amdgcn_readfirstlane(rc.mt0 + rm);
      j.nt = __builtin_amdgcn_readfirstlane(rc.nt0 + r - rm * rc.bn);
      j.kb = __builtin_amdgcn_readfirstlane(tab[j.g]);
      j.kt = __builtin_amdgcn_readfirstlane((tab[j.g + 1] - j.kb) / kBKB);
      return j;
    };
    auto pos = [&](int r) { return wgrad_pos(r, slot, per_xcd); };
    int r = 0;
    if (pos(r) >= tot) {
      zero_rest();
      return;
    }
    Job cj = job(pos(r));
    MxLoad<kBigM> cur;
    mx_setup<kBigM, MODE>(p, cur, cj.g, 0, p.M, (int64_t)cj.mt * kBigM, cj.nt, cj.kb, cj.kt * kBKB);
    bool pre = false;
    for (;;) {
      const int rn = r + 1;
      const bool has = pos(rn) < tot;
      Job nj = {0, 0, 0, 0, 0};
      MxLoad<kBigM> nxt;
      if (has) {
        nj = job(pos(rn));
        mx_setup<kBigM, MODE>(p, nxt, nj.g, 0, p.M, (int64_t)nj.mt * kBigM, nj.nt, nj.kb, nj.kt * kBKB);
      }
      mx_tile<kBigM, MODE, 2>(p, smem_mx, cur, cj.g, 0, p.M, (int64_t)cj.mt * kBigM, cj.nt, cj.kt, pre, has, nxt,
                              nj.kt, &zr);
      if (!has) break;
      cur = nxt;
      cj = nj;
      r = rn;
      pre = true;
    }
    zero_rest();
    return;
  }
  const int nbig = t_big[p.G];
  const int nsmall = t_small[p.G];
  const int tb = nbig * p.ntiles;
  const int total = tb + nsmall * p.ntiles;
  const int ts = total - tb;
  const int KT = p.K / kBKB;
  // Tiles run in groups of GN consecutive N-tiles per M-tile, all M-tiles of
  // a group before the next group: an XCD's 32 workgroups share GN B strips
  // and 32 / GN A strips.  The paired gate/up mode (wide K, 16 N-tiles) keeps
  // more B reuse with 4; the modes whose B is one expert's down projection,
  // both dgrad weights or the 8 N-tiles of the SwiGLU backward read each A
  // strip fewer times with 8 (measured 1-3% faster each).
  constexpr int GN = (MODE == GEMM_DOWN || MODE == GEMM_DUALK || MODE == GEMM_SWIGLU_BWD) ? 8 : 4;
  for (int it = 0;; ++it) {
    const int P = it * nwg + xcd * per_xcd + slot;
    if (P >= total) break;
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
    const int32_t* pre = is_big ? t_big : t_small;
    const int g = __builtin_amdgcn_readfirstlane(find_group(pre, p.G, mt));
    const int64_t row_begin = uniform_i64(t_row[g]);
    const int64_t n_g = uniform_i64(t_row[g + 1] - t_row[g]);
    const int nb_g = t_big[g + 1] - t_big[g];
    const int64_t m0 = uniform_i64(is_big ? (int64_t)(mt - pre[g]) * kBigM
                                          : (int64_t)nb_g * kBigM + (int64_t)(mt - pre[g]) * kSmallM);
    const int nt = __builtin_amdgcn_readfirstlane(ntile);
    if (is_big) {
      MxLoad<kBigM> L;
      mx_setup<kBigM, MODE>(p, L, g, row_begin, n_g, m0, nt, 0);
      mx_tile<kBigM, MODE, 2>(p, smem_mx, L, g, row_begin, n_g, m0, nt, KT, false, false, L, 0);
    } else {
      MxLoad<kSmallM> L;
      mx_setup<kSmallM, MODE>(p, L, g, row_begin, n_g, m0, nt, 0);
      mx_tile<kSmallM, MODE, 3>(p, smem_mx, L, g, row_begin, n_g, m0, nt, KT, false, false, L, 0);
    }
    __syncthreads();
  }
}

int num_cus_mx() {
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
hipError_t run_mx(const GemmProblem& q, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mxfp8_kernel<MODE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(kSmemBytes + kTabBytes));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  MxArgs a = {};
  a.A = static_cast<const uint8_t*>(q.A);
  a.As = q.A_scale;
  a.a_rows = q.a_rows;
  a.As_slab = q.A_scale_slab;
  a.a_bytes = (uint32_t)q.a_bytes;
  a.as_bytes = (uint32_t)(q.a_bytes / 32);
  a.lda = q.lda;
  a.row_off = q.row_off;
  a.M = q.M;
  a.G = q.G;
  a.B0 = static_cast<const uint8_t*>(q.B0);
  a.B1 = static_cast<const uint8_t*>(q.B1);
  a.B0s = q.B0_scale;
  a.B1s = q.B1_scale;
  a.b_stride = q.b_group_stride;
  a.N = q.N;
  a.K = q.K;
  constexpr bool paired = MODE == GEMM_GATEUP || MODE == GEMM_GU;
  a.ntiles = paired ? (q.N + kBN / 2 - 1) / (kBN / 2) : (q.N + kBN - 1) / kBN;
  a.ldb = q.ldb ? q.ldb : (MODE == GEMM_DUALK ? q.K / 2 : q.K);
  a.k_half = q.K / 2;
  a.C = q.C;
  a.Cs = q.C_scale;
  a.ldc = q.ldc;
  a.gu = static_cast<const bf16_t*>(q.gu);
  a.w_row = q.w_row;
  a.dgu = static_cast<bf16_t*>(q.dgu);
  a.dguq = q.dgu_q;
  a.dgus = q.dgu_scale;
  a.dgu_t = q.dgu_t;
  a.dgu_ts = q.dgu_t_scale;
  a.gh_t = q.gh_t;
  a.gh_ts = q.gh_t_scale;
  a.pad_off = q.pad_off;
  a.t_ld = q.t_ld;
  a.dg_part = q.dg_part;
  a.k_off = q.k_off;
  a.c_group_stride = q.c_group_stride;
  a.C1 = static_cast<bf16_t*>(q.C1);
  a.m_split = q.m_split;
  a.gu_out = static_cast<bf16_t*>(q.gu_out);
  a.spread_small = MODE == GEMM_DOWN ? 1 : 0;
  if (MODE == GEMM_WGRAD) {
    a.big = a.small = nullptr;
  } else {
    a.big = q.tile_prefix;
    a.small = q.tile_prefix + (q.G + 1);
    mx_tile_prefix_kernel<<<1, 1024, 0, s>>>(q.row_off, q.G, q.tile_prefix, q.tile_prefix + (q.G + 1));
  }
  const int wg = gemm_grid(num_cus_mx());
  gemm_mxfp8_kernel<MODE><<<(unsigned)wg, kThreads, kSmemBytes + kTabBytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace

// Grouped MXFP8 GEMM: row_off and tile_prefix are required except in the
// K-grouped weight-gradient mode (k_off instead); K (each half in DUALK) must
// be whole 128-byte slabs and N whole 64-column blocks.
hipError_t launch_gemm_mxfp8(const GemmProblem& q, hipStream_t s) {
  if (q.N % 64 != 0 || q.G > kMaxGroups) return hipErrorInvalidValue;
  if (q.mode == GEMM_WGRAD) {
    // Outputs dense per group ([M][N] at g * M * N, or with C1 two [M/2][N]
    // halves at g * M/2 * N), cut into whole 1 KiB chunks for the background
    // zero fill of groups without rows (no chunk straddles the halves).
    const int64_t rows_c = q.C1 ? q.m_split : q.M;
    if (!q.k_off || q.G < 1 || q.ldc != q.N || q.c_group_stride != rows_c * (int64_t)q.N ||
        (q.M * (int64_t)q.N * 2) % 1024 != 0 || q.M * (int64_t)q.N * 2 / 1024 > INT32_MAX)
      return hipErrorInvalidValue;
    if (q.C1 && (q.M != 2 * q.m_split || (q.m_split * (int64_t)q.N * 2) % 1024 != 0)) return hipErrorInvalidValue;
    return run_mx<GEMM_WGRAD>(q, s);
  }
  if (!q.row_off || q.K % kBKB != 0) return hipErrorInvalidValue;
  switch (q.mode) {
    case GEMM_GATEUP: return run_mx<GEMM_GATEUP>(q, s);
    case GEMM_DOWN: return run_mx<GEMM_DOWN>(q, s);
    case GEMM_GU: return run_mx<GEMM_GU>(q, s);
    case GEMM_SWIGLU_BWD:
      if (!q.gu || !q.dgu_q || !q.dgu_scale || !q.dgu_t || !q.dgu_t_scale || !q.gh_t || !q.gh_t_scale || !q.pad_off ||
          q.t_ld % 128)
        return hipErrorInvalidValue;
      return run_mx<GEMM_SWIGLU_BWD>(q, s);
    case GEMM_DUALK:
      if ((q.K / 2) % kBKB != 0) return hipErrorInvalidValue;
      return run_mx<GEMM_DUALK>(q, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
