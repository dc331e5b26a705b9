// C ABI of libmoe.so: argument validation, workspace carving and the launch
// sequence of each entry point.  See include/moe.h for the contract.
#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

// Stage-timing hook (moe_trace_events): caller-created events recorded at
// fixed stage boundaries of the fused forward (0) and backward (1).
constexpr int kMaxTrace = 32;
void* g_trace[2][kMaxTrace];
int g_ntrace[2];

void trace(int which, int i, hipStream_t s) {
  if (i < g_ntrace[which] && g_trace[which][i]) (void)hipEventRecord(static_cast<hipEvent_t>(g_trace[which][i]), s);
}

// Cap on the persistent GEMM grids (moe_set_max_workgroups); 0: none.
int g_max_wg = 0;

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(moe_prec prec) { return prec == MOE_F32 ? 4 : 2; }

moe_status check_dims(const moe_dims* D, moe_prec prec) {
  if (!D) return MOE_EINVAL;
  if (prec != MOE_F32 && prec != MOE_BF16 && prec != MOE_MXFP8) return MOE_EINVAL;
  if (D->T < 0 || D->d < 1 || D->E < 1 || D->E > 1024 || D->k < 1 || D->k > 16 || D->k > D->E || D->I < 1 ||
      D->n_shared < 0 || (D->n_shared > 0 && D->I_shared < 1))
    return MOE_EINVAL;
  if (D->T * (int64_t)D->k > INT32_MAX) return MOE_EUNSUPPORTED;
  // GEMM operands are addressed with 32-bit byte offsets from a per-expert
  // (or per-tensor, for gathered token rows) base.
  const int64_t inter = D->n_shared > 0 && D->I_shared > D->I ? D->I_shared : D->I;
  if (D->T * (int64_t)D->d * 4 > UINT32_MAX || D->T * inter * 4 > UINT32_MAX || inter * (int64_t)D->d * 4 > UINT32_MAX)
    return MOE_EUNSUPPORTED;
  if (D->n_shared > 1) return MOE_EUNSUPPORTED;
  if (prec == MOE_F32) {
    if (D->d % 8) return MOE_EUNSUPPORTED;
  } else {
    if (D->d % 64 || D->I % 64 || (D->n_shared > 0 && D->I_shared % 64)) return MOE_EUNSUPPORTED;
    if (prec == MOE_MXFP8 && (D->d % 128 || D->I % 128)) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

// Sequential carving of a caller workspace (or size computation when base is null).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(bytes);
    return p;
  }
};

struct FfnWs {
  int32_t* prefix;
  void* h;
  uint8_t* h_scale;
};

FfnWs carve_ffn(Carver& c, const moe_dims* D, moe_prec prec) {
  const int64_t R = D->T * D->k;
  FfnWs w;
  w.prefix = static_cast<int32_t*>(c.take((size_t)2 * (D->E + 2) * sizeof(int32_t)));
  if (prec == MOE_MXFP8) {
    w.h = c.take((size_t)R * D->I);
    w.h_scale = static_cast<uint8_t*>(c.take((size_t)R * (D->I / 32)));
  } else {
    w.h = c.take((size_t)R * D->I * act_bytes(prec));
    w.h_scale = nullptr;
  }
  return w;
}

void* carve_shared(Carver& c, const moe_dims* D, moe_prec prec) {
  return c.take((size_t)D->T * (D->n_shared ? D->I_shared : 0) * act_bytes(prec));
}

struct FwdWs {
  float* logits;
  int32_t *topk_idx, *counts, *offsets, *row_token, *token_row;
  float* topk_w;
  void* sched;
  void* x_perm;
  uint8_t* x_perm_scale;
  uint8_t* xs_slab;  // MXFP8: the token scales of every routed row, slab-major (the gate/up GEMM's A scales)
  FfnWs ffn;
  void* o_perm;
  void* y_shared;
  void* hs;
};

FwdWs carve_forward(Carver& c, const moe_dims* D, moe_prec prec, const moe_routing* rt) {
  const int64_t T = D->T, R = D->T * D->k;
  FwdWs w;
  auto pick = [&](void* user, size_t bytes) { return user ? (c.take(0), user) : c.take(bytes); };
  w.logits = static_cast<float*>(pick(rt ? rt->logits : nullptr, (size_t)T * D->E * 4));
  w.topk_idx = static_cast<int32_t*>(pick(rt ? rt->topk_idx : nullptr, (size_t)R * 4));
  w.topk_w = static_cast<float*>(pick(rt ? rt->topk_w : nullptr, (size_t)R * 4));
  w.counts = static_cast<int32_t*>(pick(rt ? rt->expert_counts : nullptr, (size_t)D->E * 4));
  w.offsets = static_cast<int32_t*>(pick(rt ? rt->expert_offsets : nullptr, (size_t)(D->E + 1) * 4));
  w.row_token = static_cast<int32_t*>(pick(rt ? rt->row_token : nullptr, (size_t)R * 4));
  w.token_row = static_cast<int32_t*>(pick(rt ? rt->token_row : nullptr, (size_t)R * 4));
  w.sched = c.take(permute_scratch_bytes(T, D->E));
  if (prec == MOE_MXFP8) {  // quantized tokens [T][d] (+ scales); rows are gathered by the GEMM
    w.x_perm = c.take((size_t)T * D->d);
    w.x_perm_scale = static_cast<uint8_t*>(c.take((size_t)T * (D->d / 32)));
    w.xs_slab = static_cast<uint8_t*>(c.take((size_t)R * (D->d / 32)));
  } else {
    w.x_perm = c.take((size_t)R * D->d * act_bytes(prec));
    w.x_perm_scale = nullptr;
    w.xs_slab = nullptr;
  }
  w.ffn = carve_ffn(c, D, prec);
  w.o_perm = c.take((size_t)R * D->d * act_bytes(prec));
  w.y_shared = D->n_shared ? c.take((size_t)T * D->d * act_bytes(prec)) : nullptr;
  w.hs = carve_shared(c, D, prec);
  return w;
}

// Backward scratch.  Rp: K capacity of the expert-padded transposed operands
// of the weight-gradient GEMMs (every expert's rows rounded up to `pad`: 64
// for the bf16 GEMM's K slabs, 128 for the MXFP8 ones).
struct BwdWs {
  int pad;
  int64_t Rp, Tp;
  int32_t* prefix;   // [2(E+2)] GEMM tile prefixes
  int32_t* pad_off;  // [E+1]
  int32_t* single;   // [4] {0, Tp, 0, T}: one-group K range and segment
  float *w_row, *dl, *dl_row;
  void *gu, *dgu, *gh, *da;
  float* dg_part;
  float* router_partial;
  void *xT, *dyT, *ghT, *dguT;  // bf16 transposed operands
  // MXFP8: quantized tokens and output gradients (along d), dG|dU along I, and
  // the transposed operands quantized along the routed-row axis.
  uint8_t *xq, *xqs, *dyq, *dyqs, *dguq, *dguqs;
  uint8_t *xs_slab, *dys_slab;  // token scales of every routed row, slab-major (gathered GEMM A operands)
  uint8_t *xTq, *xTqs, *dyTq, *dyTqs, *ghTq, *ghTqs, *dguTq, *dguTqs;
  void *gus, *dgus, *hs, *dxs, *xTs, *dyTs, *hsT, *dgusT;
};

BwdWs carve_backward(Carver& c, const moe_dims* D, moe_prec prec) {
  const int64_t T = D->T, R = D->T * D->k, d = D->d, I = D->I, Is = D->n_shared ? D->I_shared : 0;
  const bool mx = prec == MOE_MXFP8;
  BwdWs w = {};
  w.pad = mx ? 128 : 64;
  w.Rp = bwd_padded_rows(R, D->E, w.pad);
  w.Tp = (T + w.pad - 1) / w.pad * w.pad;
  auto u8 = [&](size_t n) { return static_cast<uint8_t*>(c.take(n)); };
  w.prefix = static_cast<int32_t*>(c.take((size_t)2 * (D->E + 2) * 4));
  w.pad_off = static_cast<int32_t*>(c.take((size_t)(D->E + 1) * 4));
  w.single = static_cast<int32_t*>(c.take(16));
  w.w_row = static_cast<float*>(c.take((size_t)R * 4));
  w.dl = static_cast<float*>(c.take((size_t)R * 4));
  w.dl_row = static_cast<float*>(c.take((size_t)R * 4));
  w.gu = c.take((size_t)R * 2 * I * 2);
  w.dgu = mx ? nullptr : c.take((size_t)R * 2 * I * 2);  // MXFP8: dG, dU stay in the epilogue
  w.gh = mx ? nullptr : c.take((size_t)R * I * 2);  // MXFP8: w h stays in the epilogue
  w.da = c.take((size_t)R * d * 2);
  w.dg_part = static_cast<float*>(c.take((size_t)R * (I / 32) * 4));
  w.router_partial = static_cast<float*>(c.take((size_t)(w.Rp / 64) * d * 4));
  if (mx) {
    w.xq = u8((size_t)T * d);
    w.xqs = u8((size_t)T * d / 32);
    w.dyq = u8((size_t)T * d);
    w.dyqs = u8((size_t)T * d / 32);
    w.xs_slab = u8((size_t)R * d / 32);
    w.dys_slab = u8((size_t)R * d / 32);
    w.dguq = u8((size_t)R * 2 * I);
    w.dguqs = u8((size_t)R * 2 * I / 32);
    w.xTq = u8((size_t)d * w.Rp);
    w.xTqs = u8((size_t)d * w.Rp / 32);
    w.dyTq = u8((size_t)d * w.Rp);
    w.dyTqs = u8((size_t)d * w.Rp / 32);
    w.ghTq = u8((size_t)I * w.Rp);
    w.ghTqs = u8((size_t)I * w.Rp / 32);
    w.dguTq = u8((size_t)2 * I * w.Rp);
    w.dguTqs = u8((size_t)2 * I * w.Rp / 32);
  } else {
    w.xT = c.take((size_t)d * w.Rp * 2);
    w.dyT = c.take((size_t)d * w.Rp * 2);
    w.ghT = c.take((size_t)I * w.Rp * 2);
    w.dguT = c.take((size_t)2 * I * w.Rp * 2);
  }
  w.gus = c.take((size_t)T * 2 * Is * 2);
  w.dgus = c.take((size_t)T * 2 * Is * 2);
  w.hs = c.take((size_t)T * Is * 2);
  w.dxs = c.take(Is ? (size_t)T * d * 2 : 0);
  w.xTs = c.take(Is ? (size_t)d * w.Tp * 2 : 0);
  w.dyTs = c.take(Is ? (size_t)d * w.Tp * 2 : 0);
  w.hsT = c.take((size_t)Is * w.Tp * 2);
  w.dgusT = c.take((size_t)2 * Is * w.Tp * 2);
  return w;
}

size_t workspace_size(const moe_dims* D, moe_prec prec, int which) {
  Carver c(nullptr);
  switch (which) {
    case 0: carve_forward(c, D, prec, nullptr); break;
    case 1: c.take(permute_scratch_bytes(D->T, D->E)); break;
    case 2: carve_ffn(c, D, prec); break;
    case 3: carve_shared(c, D, prec); break;
    case 4: carve_backward(c, D, prec); break;
    default: return 0;
  }
  return c.used;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

#define MOE_TRY(expr)                  \
  do {                                 \
    moe_status st_ = (expr);           \
    if (st_ != MOE_OK) return st_;     \
  } while (0)

#define MOE_HIP(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return MOE_EHIP;     \
  } while (0)

// ---- launch sequences (arguments already validated) ------------------------

moe_status run_route(const moe_dims* D, moe_prec prec, const void* x, const void* wr, const float* bias,
                     float* logits, int32_t* idx, float* w, hipStream_t s) {
  const bool f32 = prec == MOE_F32;
  MOE_HIP(launch_router_logits(f32, x, wr, bias, logits, w, D->T, D->d, D->E, D->k, s));
  MOE_HIP(launch_topk(f32, logits, x, wr, bias, idx, w, D->T, D->d, D->E, D->k, s));
  return MOE_OK;
}

moe_status run_permute(const moe_dims* D, moe_prec prec, const int32_t* idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* x_perm, uint8_t* x_perm_scale,
                       void* sched, hipStream_t s) {
  MOE_HIP(launch_schedule(idx, D->T, D->E, D->k, counts, offsets, row_token, token_row, sched, s));
  if (x_perm) {
    if (prec == MOE_MXFP8)
      MOE_HIP(launch_dispatch_quant_mx(static_cast<const bf16_t*>(x), token_row, static_cast<uint8_t*>(x_perm),
                                       x_perm_scale, D->T, D->k, D->d, s));
    else
      MOE_HIP(launch_dispatch_rows(x, token_row, x_perm, D->T, D->k, D->d, (int)act_bytes(prec), s));
  }
  return MOE_OK;
}

// Grouped gate/up GEMM with the SwiGLU epilogue into h.
moe_status run_gateup(moe_prec prec, const void* A, const int32_t* a_rows, int64_t a_bytes, int64_t lda,
                      const int32_t* row_off, int64_t M, int G, const void* wg, const void* wu, int d, int I, void* h,
                      int32_t* prefix, hipStream_t s, void* gu_out = nullptr) {
  GemmProblem q = {};
  q.mode = GEMM_GATEUP;
  q.A = A;
  q.a_rows = a_rows;
  q.a_bytes = a_bytes;
  q.lda = lda;
  q.row_off = row_off;
  q.M = M;
  q.G = G;
  q.B0 = wg;
  q.B1 = wu;
  q.b_group_stride = (int64_t)I * d;
  q.N = I;
  q.K = d;
  q.C = h;
  q.ldc = I;
  q.tile_prefix = prefix;
  q.gu_out = gu_out;
  MOE_HIP(prec == MOE_F32 ? launch_gemm_f32(q, s) : launch_gemm_bf16(q, s));
  return MOE_OK;
}

// Grouped down GEMM from h.
moe_status run_down(moe_prec prec, const int32_t* row_off, int64_t M, int G, const void* wd, int d, int I,
                    const void* h, void* out, int32_t* prefix, hipStream_t s) {
  GemmProblem r = {};
  r.mode = GEMM_DOWN;
  r.A = h;
  r.lda = I;
  r.row_off = row_off;
  r.M = M;
  r.G = G;
  r.B0 = wd;
  r.b_group_stride = (int64_t)d * I;
  r.N = d;
  r.K = I;
  r.C = out;
  r.ldc = d;
  r.tile_prefix = prefix;
  MOE_HIP(prec == MOE_F32 ? launch_gemm_f32(r, s) : launch_gemm_bf16(r, s));
  return MOE_OK;
}

// MXFP8 grouped gate/up (h quantized along I in the epilogue) and down.
moe_status run_gateup_mx(const moe_dims* D, const uint8_t* A, const uint8_t* A_scale, const int32_t* a_rows,
                         const int32_t* offsets, const moe_weights* w, uint8_t* h, uint8_t* h_scale, int32_t* prefix,
                         hipStream_t s, void* gu_out = nullptr, const uint8_t* A_scale_slab = nullptr) {
  GemmProblem q = {};
  q.mode = GEMM_GATEUP;
  q.A = A;
  q.A_scale = A_scale;
  q.a_rows = a_rows;
  q.A_scale_slab = A_scale_slab;
  q.a_bytes = a_rows ? D->T * (int64_t)D->d : 0;
  q.lda = D->d;
  q.row_off = offsets;
  q.M = D->T * D->k;
  q.G = D->E;
  q.B0 = w->q_gate;
  q.B1 = w->q_up;
  q.B0_scale = w->q_gate_scale;
  q.B1_scale = w->q_up_scale;
  q.b_group_stride = (int64_t)D->I * D->d;
  q.N = D->I;
  q.K = D->d;
  q.C = h;
  q.C_scale = h_scale;
  q.ldc = D->I;
  q.tile_prefix = prefix;
  q.gu_out = gu_out;
  MOE_HIP(launch_gemm_mxfp8(q, s));
  return MOE_OK;
}

moe_status run_down_mx(const moe_dims* D, const uint8_t* h, const uint8_t* h_scale, const int32_t* offsets,
                       const moe_weights* w, void* o_perm, int32_t* prefix, hipStream_t s) {
  GemmProblem r = {};
  r.mode = GEMM_DOWN;
  r.A = h;
  r.A_scale = h_scale;
  r.lda = D->I;
  r.row_off = offsets;
  r.M = D->T * D->k;
  r.G = D->E;
  r.B0 = w->q_down;
  r.B0_scale = w->q_down_scale;
  r.b_group_stride = (int64_t)D->d * D->I;
  r.N = D->d;
  r.K = D->I;
  r.C = o_perm;
  r.ldc = D->d;
  r.tile_prefix = prefix;
  MOE_HIP(launch_gemm_mxfp8(r, s));
  return MOE_OK;
}

// One SwiGLU FFN over grouped rows: gate/up (+SwiGLU) into h, then down.
moe_status run_ffn_grouped(moe_prec prec, const void* A, const int32_t* a_rows, int64_t a_bytes, int64_t lda,
                           const int32_t* row_off, int64_t M, int G, const void* wg, const void* wu, const void* wd,
                           int d, int I, void* h, void* out, int32_t* prefix, hipStream_t s, void* gu_out = nullptr) {
  MOE_TRY(run_gateup(prec, A, a_rows, a_bytes, lda, row_off, M, G, wg, wu, d, I, h, prefix, s, gu_out));
  return run_down(prec, row_off, M, G, wd, d, I, h, out, prefix, s);
}

moe_status run_expert_ffn(const moe_dims* D, moe_prec prec, const void* A, const uint8_t* A_scale,
                          const int32_t* a_rows, const int32_t* offsets, const moe_weights* w, void* o_perm,
                          const FfnWs& ws, hipStream_t s, bool traced = false, void* gu_out = nullptr,
                          const uint8_t* A_scale_slab = nullptr) {
  if (prec == MOE_MXFP8) {
    MOE_TRY(run_gateup_mx(D, static_cast<const uint8_t*>(A), A_scale, a_rows, offsets, w,
                          static_cast<uint8_t*>(ws.h), ws.h_scale, ws.prefix, s, gu_out, A_scale_slab));
    if (traced) trace(0, 4, s);
    return run_down_mx(D, static_cast<const uint8_t*>(ws.h), ws.h_scale, offsets, w, o_perm, ws.prefix, s);
  }
  const int64_t a_bytes = a_rows ? D->T * (int64_t)D->d * (int64_t)act_bytes(prec) : 0;
  const int64_t R = D->T * D->k;
  MOE_TRY(run_gateup(prec, A, a_rows, a_bytes, D->d, offsets, R, D->E, w->w_gate, w->w_up, D->d, D->I, ws.h,
                     ws.prefix, s, gu_out));
  if (traced) trace(0, 4, s);
  return run_down(prec, offsets, R, D->E, w->w_down, D->d, D->I, ws.h, o_perm, ws.prefix, s);
}

moe_status run_shared_ffn(const moe_dims* D, moe_prec prec, const void* x, const moe_weights* w, void* y_shared,
                          void* hs, hipStream_t s, void* gu_out = nullptr) {
  if (D->T == 0) return MOE_OK;
  if (D->n_shared == 0) {
    MOE_HIP(launch_fill_zero(y_shared, (size_t)D->T * D->d * act_bytes(prec), s));
    return MOE_OK;
  }
  const moe_prec p = prec == MOE_F32 ? MOE_F32 : MOE_BF16;  // shared expert stays bf16 under MXFP8
  return run_ffn_grouped(p, x, nullptr, 0, D->d, nullptr, D->T, 1, w->ws_gate, w->ws_up, w->ws_down, D->d,
                         D->I_shared, hs, y_shared, nullptr, s, gu_out);
}

moe_status check_weights(const moe_dims* D, moe_prec prec, const moe_weights* w, bool routed, bool shared,
                         bool router) {
  if (!w) return MOE_EINVAL;
  if (router && (!w->w_router || !aligned16(w->w_router))) return MOE_EINVAL;
  if (routed) {
    if (prec == MOE_MXFP8) {
      const void* q[] = {w->q_gate, w->q_gate_scale, w->q_up, w->q_up_scale, w->q_down, w->q_down_scale};
      for (const void* p : q)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    } else {
      const void* q[] = {w->w_gate, w->w_up, w->w_down};
      for (const void* p : q)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    }
  }
  if (shared && D->n_shared > 0) {
    const void* q[] = {w->ws_gate, w->ws_up, w->ws_down};
    for (const void* p : q)
      if (!p || !aligned16(p)) return MOE_EINVAL;
  }
  return MOE_OK;
}

bool ptr_ok(const void* p) { return p && aligned16(p); }
bool opt_ok(const void* p) { return !p || aligned16(p); }

// ---- backward ---------------------------------------------------------------

// GEMM descriptor with the fields every backward GEMM sets.
GemmProblem gemm(int mode, const void* A, int64_t lda, const int32_t* row_off, int64_t M, int G, const void* B0,
                 const void* B1, int64_t b_group_stride, int N, int K, void* C, int64_t ldc, int32_t* prefix) {
  GemmProblem q = {};
  q.mode = mode;
  q.A = A;
  q.lda = lda;
  q.row_off = row_off;
  q.M = M;
  q.G = G;
  q.B0 = B0;
  q.B1 = B1;
  q.b_group_stride = b_group_stride;
  q.N = N;
  q.K = K;
  q.C = C;
  q.ldc = ldc;
  q.tile_prefix = prefix;
  return q;
}

// Weight gradients C_g = A[:, K_g] B[:, K_g]^T of every group from the
// transposed operands A [M][ldk], B [N][ldk] over the K ranges k_off.  With
// C1, A stacks two operands of M/2 rows each and rows [M/2, M) of every
// group's result go to C1 (dW_gate and dW_up from [dG^T; dU^T] in one launch,
// reading B = x^T once).
moe_status run_wgrad(const void* A, int64_t M, const void* B, int N, int64_t ldk, const int32_t* k_off, int G,
                     void* C, hipStream_t s, void* C1 = nullptr) {
  GemmProblem q = gemm(GEMM_WGRAD, A, ldk, nullptr, M, G, B, nullptr, 0, N, 64, C, N, nullptr);
  q.ldb = ldk;
  q.k_off = k_off;
  q.c_group_stride = (C1 ? M / 2 : M) * N;
  q.C1 = C1;
  q.m_split = C1 ? M / 2 : 0;
  MOE_HIP(launch_gemm_bf16(q, s));
  return MOE_OK;
}

// MXFP8 weight gradients from the quantized transposed operands
// (A [M][ldk] + scales [M][ldk/32], B [N][ldk] + scales); C1 as in run_wgrad.
moe_status run_wgrad_mx(const uint8_t* A, const uint8_t* As, int64_t M, const uint8_t* B, const uint8_t* Bs, int N,
                        int64_t ldk, const int32_t* k_off, int G, void* C, hipStream_t s, void* C1 = nullptr) {
  GemmProblem q = gemm(GEMM_WGRAD, A, ldk, nullptr, M, G, B, nullptr, 0, N, 128, C, N, nullptr);
  q.A_scale = As;
  q.B0_scale = Bs;
  q.ldb = ldk;
  q.k_off = k_off;
  q.c_group_stride = (C1 ? M / 2 : M) * N;
  q.C1 = C1;
  q.m_split = C1 ? M / 2 : 0;
  MOE_HIP(launch_gemm_mxfp8(q, s));
  return MOE_OK;
}

moe_status check_backward_weights(const moe_dims* D, moe_prec prec, const moe_weights* w, bool router) {
  if (!w) return MOE_EINVAL;
  if (prec == MOE_MXFP8) {
    const void* r[] = {w->q_gate, w->q_gate_scale, w->q_up, w->q_up_scale, w->qt_gate, w->qt_gate_scale,
                       w->qt_up, w->qt_up_scale, w->qt_down, w->qt_down_scale};
    for (const void* p : r)
      if (!ptr_ok(p)) return MOE_EINVAL;
  } else {
    const void* r[] = {w->w_gate, w->w_up, w->wt_gate, w->wt_up, w->wt_down};
    for (const void* p : r)
      if (!ptr_ok(p)) return MOE_EINVAL;
  }
  if (D->n_shared > 0) {
    const void* q[] = {w->ws_gate, w->ws_up, w->wst_gate, w->wst_up, w->wst_down};
    for (const void* p : q)
      if (!ptr_ok(p)) return MOE_EINVAL;
  }
  if (router && !ptr_ok(w->w_router)) return MOE_EINVAL;
  return MOE_OK;
}

moe_status run_backward(const moe_dims* D, const bf16_t* dy, const bf16_t* x, const moe_weights* w,
                        const moe_routing* rt, bf16_t* dx, const moe_grads* g, const BwdWs& b, hipStream_t s) {
  const int64_t T = D->T, R = T * D->k;
  const int d = D->d, I = D->I, E = D->E, k = D->k;
  const bool router = g->dw_router != nullptr;
  const bool mx = b.pad == 128;
  trace(1, 0, s);
  MOE_HIP(launch_pad_offsets(rt->expert_counts, E, T, b.pad, b.pad_off, b.single, s));
  MOE_HIP(launch_row_weight(rt->token_row, rt->topk_w, R, b.w_row, s));
  if (mx) {  // output gradients (and, for the replay, tokens) quantized once along d (row-wise: commutes with the gather)
    MOE_HIP(launch_quantize_mx(dy, T, d, 0, b.dyq, b.dyqs, s));
    MOE_HIP(launch_gather_scales_slab(b.dyqs, rt->row_token, R, d, b.dys_slab, s));
    if (!rt->gu) {
      MOE_HIP(launch_quantize_mx(x, T, d, 0, b.xq, b.xqs, s));
      MOE_HIP(launch_gather_scales_slab(b.xqs, rt->row_token, R, d, b.xs_slab, s));
    }
  }
  trace(1, 1, s);

  // G | U of every routed row: kept by the forward, or replayed here.
  const void* gu = rt->gu ? rt->gu : b.gu;
  GemmProblem q;
  if (!rt->gu) {
  q = gemm(GEMM_GU, mx ? (const void*)b.xq : x, d, rt->expert_offsets, R, E,
                       mx ? (const void*)w->q_gate : w->w_gate, mx ? (const void*)w->q_up : w->w_up, (int64_t)I * d,
                       I, d, b.gu, 2 * I, b.prefix);
  q.a_rows = rt->row_token;
  q.a_bytes = T * (int64_t)d * (mx ? 1 : 2);
  if (mx) {
    q.A_scale = b.xqs;
    q.A_scale_slab = b.xs_slab;
    q.B0_scale = w->q_gate_scale;
    q.B1_scale = w->q_up_scale;
  }
  MOE_HIP(mx ? launch_gemm_mxfp8(q, s) : launch_gemm_bf16(q, s));
  }
  trace(1, 2, s);
  // Reverse combine + down-projection input gradient dH' = dY_perm W_d with
  // the SwiGLU backward and the router-weight partials in the epilogue.
  q = gemm(GEMM_SWIGLU_BWD, mx ? (const void*)b.dyq : dy, d, rt->expert_offsets, R, E,
           mx ? (const void*)w->qt_down : w->wt_down, nullptr, (int64_t)I * d, I, d, b.dgu, 2 * I, b.prefix);
  q.a_rows = rt->row_token;
  q.a_bytes = T * (int64_t)d * (mx ? 1 : 2);
  q.gu = gu;
  q.w_row = b.w_row;
  q.dgu = b.dgu;
  q.h_out = b.gh;
  q.dg_part = b.dg_part;
  if (mx) {
    q.A_scale = b.dyqs;
    q.A_scale_slab = b.dys_slab;
    q.B0_scale = w->qt_down_scale;
    q.dgu_q = b.dguq;
    q.dgu_scale = b.dguqs;
    q.dgu_t = b.dguTq;  // dG^T | dU^T and (w h)^T for the weight gradients, quantized in the epilogue
    q.dgu_t_scale = b.dguTqs;
    q.gh_t = b.ghTq;
    q.gh_t_scale = b.ghTqs;
    q.pad_off = b.pad_off;
    q.t_ld = b.Rp;
  }
  MOE_HIP(mx ? launch_gemm_mxfp8(q, s) : launch_gemm_bf16(q, s));
  trace(1, 3, s);
  MOE_HIP(launch_dg(b.dg_part, I / 32, rt->token_row, rt->topk_w, T, k, g->dtopk_w, router ? b.dl : nullptr,
                    b.dl_row, s));
  trace(1, 4, s);
  // Gate/up input gradient dA = dG W_g + dU W_u (K = 2I over two matrices).
  q = gemm(GEMM_DUALK, mx ? (const void*)b.dguq : b.dgu, 2 * I, rt->expert_offsets, R, E,
           mx ? (const void*)w->qt_gate : w->wt_gate, mx ? (const void*)w->qt_up : w->wt_up, (int64_t)d * I, d, 2 * I,
           b.da, d, b.prefix);
  if (mx) {
    q.A_scale = b.dguqs;
    q.B0_scale = w->qt_gate_scale;
    q.B1_scale = w->qt_up_scale;
  }
  MOE_HIP(mx ? launch_gemm_mxfp8(q, s) : launch_gemm_bf16(q, s));
  trace(1, 5, s);

  const int Is = D->n_shared ? D->I_shared : 0;
  if (Is) {
    if (!rt->gu_shared) {
      q = gemm(GEMM_GU, x, d, nullptr, T, 1, w->ws_gate, w->ws_up, 0, Is, d, b.gus, 2 * Is, nullptr);
      MOE_HIP(launch_gemm_bf16(q, s));
    }
    q = gemm(GEMM_SWIGLU_BWD, dy, d, nullptr, T, 1, w->wst_down, nullptr, 0, Is, d, b.dgus, 2 * Is, nullptr);
    q.gu = rt->gu_shared ? rt->gu_shared : b.gus;
    q.dgu = b.dgus;
    q.h_out = b.hs;
    MOE_HIP(launch_gemm_bf16(q, s));
    q = gemm(GEMM_DUALK, b.dgus, 2 * Is, nullptr, T, 1, w->wst_gate, w->wst_up, 0, d, 2 * Is, b.dxs, d, nullptr);
    MOE_HIP(launch_gemm_bf16(q, s));
  }
  trace(1, 6, s);
  // Reverse dispatch: token-order sum in ascending expert order.
  MOE_HIP(launch_dx(static_cast<const bf16_t*>(b.da), rt->token_row, rt->topk_idx, router ? b.dl : nullptr,
                    static_cast<const bf16_t*>(w->w_router), Is ? static_cast<const bf16_t*>(b.dxs) : nullptr, dx, T,
                    d, k, s));
  trace(1, 7, s);

  // Deferred weight gradients over each expert's whole (padded) row range.
  const bf16_t* gh = static_cast<const bf16_t*>(b.gh);
  const bf16_t* dgu = static_cast<const bf16_t*>(b.dgu);
  const int32_t* off = rt->expert_offsets;
  if (mx) {
    const int64_t Rp = b.Rp;
    // Expert-blocked [cols][Kp_e] operands; dG^T, dU^T and (w h)^T came from
    // the down-dgrad epilogue.
    MOE_HIP(launch_transpose_quant(x, d, d, rt->row_token, off, b.pad_off, E, Rp, b.xTq, b.xTqs, s));
    MOE_HIP(launch_transpose_quant(dy, d, d, rt->row_token, off, b.pad_off, E, Rp, b.dyTq, b.dyTqs, s));
    trace(1, 8, s);
    MOE_TRY(run_wgrad_mx(b.dyTq, b.dyTqs, d, b.ghTq, b.ghTqs, I, Rp, b.pad_off, E, g->dw_down, s));
    trace(1, 9, s);
    // dW_gate and dW_up in one launch over [dG^T; dU^T] (2I rows per expert)
    MOE_TRY(run_wgrad_mx(b.dguTq, b.dguTqs, 2 * I, b.xTq, b.xTqs, d, Rp, b.pad_off, E, g->dw_gate, s, g->dw_up));
    trace(1, 10, s);
  } else {
    MOE_HIP(launch_transpose_rows(x, d, d, rt->row_token, off, b.pad_off, E, b.Rp, static_cast<bf16_t*>(b.xT), s));
    MOE_HIP(launch_transpose_rows(dy, d, d, rt->row_token, off, b.pad_off, E, b.Rp, static_cast<bf16_t*>(b.dyT), s));
    MOE_HIP(launch_transpose_rows(gh, I, I, nullptr, off, b.pad_off, E, b.Rp, static_cast<bf16_t*>(b.ghT), s));
    // [dG | dU] rows -> one [2I][Kp_e] block per expert: dG^T over dU^T
    MOE_HIP(launch_transpose_rows(dgu, 2 * I, 2 * I, nullptr, off, b.pad_off, E, b.Rp, static_cast<bf16_t*>(b.dguT),
                                  s));
    trace(1, 8, s);
    MOE_TRY(run_wgrad(b.dyT, d, b.ghT, I, b.Rp, b.pad_off, E, g->dw_down, s));
    trace(1, 9, s);
    MOE_TRY(run_wgrad(b.dguT, 2 * I, b.xT, d, b.Rp, b.pad_off, E, g->dw_gate, s, g->dw_up));
    trace(1, 10, s);
  }
  if (Is) {
    const int32_t* seg = b.single + 2;
    const bf16_t* dgus = static_cast<const bf16_t*>(b.dgus);
    MOE_HIP(launch_transpose_rows(x, d, d, nullptr, seg, b.single, 1, b.Tp, static_cast<bf16_t*>(b.xTs), s));
    MOE_HIP(launch_transpose_rows(dy, d, d, nullptr, seg, b.single, 1, b.Tp, static_cast<bf16_t*>(b.dyTs), s));
    MOE_HIP(launch_transpose_rows(static_cast<const bf16_t*>(b.hs), Is, Is, nullptr, seg, b.single, 1, b.Tp,
                                  static_cast<bf16_t*>(b.hsT), s));
    MOE_HIP(launch_transpose_rows(dgus, 2 * Is, 2 * Is, nullptr, seg, b.single, 1, b.Tp,
                                  static_cast<bf16_t*>(b.dgusT), s));
    MOE_TRY(run_wgrad(b.dyTs, d, b.hsT, Is, b.Tp, b.single, 1, g->dws_down, s));
    MOE_TRY(run_wgrad(b.dgusT, 2 * Is, b.xTs, d, b.Tp, b.single, 1, g->dws_gate, s, g->dws_up));
  }
  trace(1, 11, s);
  if (router)
    MOE_HIP(launch_router_wgrad(x, rt->row_token, b.dl_row, rt->expert_offsets, b.pad_off, E, d, b.Rp,
                                b.router_partial, g->dw_router, s));
  trace(1, 12, s);
  return MOE_OK;
}

}  // namespace

namespace moe {
int gemm_grid(int num_cus) {
  int wg = (num_cus + 7) / 8 * 8;
  if (g_max_wg > 0 && g_max_wg < wg) wg = g_max_wg / 8 * 8;
  return wg < 8 ? 8 : wg;
}
}  // namespace moe

extern "C" {

moe_status moe_set_max_workgroups(int n) {
  if (n < 0) return MOE_EINVAL;
  g_max_wg = n;
  return MOE_OK;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape or mode not supported by the library";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch or runtime error";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_bytes(const moe_dims* dims, moe_prec prec, int which, size_t* bytes) {
  MOE_TRY(check_dims(dims, prec));
  if (!bytes || which < 0 || which > 4) return MOE_EINVAL;
  *bytes = workspace_size(dims, prec, which);
  return MOE_OK;
}

moe_status moe_route(const moe_dims* dims, moe_prec prec, const void* x, const void* w_router, const float* logit_bias,
                     float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  if (dims->T > 0 && (!ptr_ok(x) || !ptr_ok(w_router) || !ptr_ok(logits) || !ptr_ok(topk_idx) || !ptr_ok(topk_w)))
    return MOE_EINVAL;
  if (!opt_ok(logit_bias)) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;
  return run_route(dims, prec, x, w_router, logit_bias, logits, topk_idx, topk_w, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_dims* dims, moe_prec prec, const int32_t* topk_idx, const void* x,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token, int32_t* token_row,
                       void* x_perm, uint8_t* x_perm_scale, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  if (!ptr_ok(expert_counts) || !ptr_ok(expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0 && (!ptr_ok(topk_idx) || !ptr_ok(row_token) || !ptr_ok(token_row))) return MOE_EINVAL;
  if (x_perm && (!aligned16(x_perm) || !ptr_ok(x) || (prec == MOE_MXFP8 && !ptr_ok(x_perm_scale)))) return MOE_EINVAL;
  if (prec == MOE_MXFP8 && x_perm && dims->d % 32) return MOE_EUNSUPPORTED;
  const size_t need = workspace_size(dims, prec, 1);
  if (need && (!ws || ws_bytes < need)) return MOE_EWORKSPACE;
  if (ws && !aligned16(ws)) return MOE_EINVAL;
  return run_permute(dims, prec, topk_idx, x, expert_counts, expert_offsets, row_token, token_row, x_perm,
                     x_perm_scale, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_quantize_mxfp8_rows_t(const void* src_bf16, int64_t ld_src, int32_t cols, const int32_t* gather,
                                     const int32_t* seg_off, const int32_t* pad_off, int32_t nseg, int64_t p_cap,
                                     uint8_t* dst, uint8_t* dst_scale, void* stream) {
  if (nseg < 1 || nseg > 1024 || cols < 0 || p_cap < 0 || ld_src < cols) return MOE_EINVAL;
  if (cols % 8 || ld_src % 8 || p_cap % 128) return MOE_EUNSUPPORTED;
  if (p_cap == 0 || cols == 0) return MOE_OK;
  if (!ptr_ok(src_bf16) || !opt_ok(gather) || !ptr_ok(seg_off) || !ptr_ok(pad_off) || !ptr_ok(dst) ||
      !ptr_ok(dst_scale))
    return MOE_EINVAL;
  if (p_cap * (int64_t)cols > INT32_MAX * 16ll) return MOE_EUNSUPPORTED;
  MOE_HIP(launch_transpose_quant(static_cast<const bf16_t*>(src_bf16), ld_src, cols, gather, seg_off, pad_off, nseg,
                                 p_cap, dst, dst_scale, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_permute_noalloc(const moe_dims* dims, moe_prec prec, const int32_t* topk_idx, const void* x,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                               int32_t* token_row, void* x_perm, uint8_t* x_perm_scale, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  if (!ptr_ok(expert_counts) || !ptr_ok(expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0 && (!ptr_ok(topk_idx) || !ptr_ok(row_token) || !ptr_ok(token_row))) return MOE_EINVAL;
  if (x_perm && (!aligned16(x_perm) || !ptr_ok(x) || (prec == MOE_MXFP8 && !ptr_ok(x_perm_scale)))) return MOE_EINVAL;
  if (prec == MOE_MXFP8 && x_perm && dims->d % 32) return MOE_EUNSUPPORTED;
  if (permute_scratch_bytes(dims->T, dims->E) > noalloc_scratch_capacity()) return MOE_EWORKSPACE;
  void* sc = nullptr;
  if (dims->T > 0) MOE_HIP(noalloc_scratch(&sc));
  return run_permute(dims, prec, topk_idx, x, expert_counts, expert_offsets, row_token, token_row, x_perm,
                     x_perm_scale, sc, static_cast<hipStream_t>(stream));
}

size_t moe_permute_noalloc_scratch_bytes(void) { return noalloc_scratch_capacity(); }

moe_status moe_expert_ffn(const moe_dims* dims, moe_prec prec, const void* x_perm, const uint8_t* x_perm_scale,
                          const int32_t* expert_offsets, const moe_weights* w, void* o_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  MOE_TRY(check_dims(dims, prec));
  MOE_TRY(check_weights(dims, prec, w, true, false, false));
  if (!ptr_ok(expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0 && (!ptr_ok(x_perm) || !ptr_ok(o_perm))) return MOE_EINVAL;
  if (prec == MOE_MXFP8 && dims->T > 0 && !ptr_ok(x_perm_scale)) return MOE_EINVAL;
  const size_t need = workspace_size(dims, prec, 2);
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;
  Carver c(ws);
  FfnWs f = carve_ffn(c, dims, prec);
  return run_expert_ffn(dims, prec, x_perm, x_perm_scale, nullptr, expert_offsets, w, o_perm, f,
                        static_cast<hipStream_t>(stream));
}

moe_status moe_expert_gate_up(const moe_dims* dims, moe_prec prec, const void* x_perm, const uint8_t* x_perm_scale,
                              const int32_t* expert_offsets, const moe_weights* w, void* h, uint8_t* h_scale, void* ws,
                              size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  MOE_TRY(check_weights(dims, prec, w, true, false, false));
  if (!ptr_ok(expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0 && (!ptr_ok(x_perm) || !ptr_ok(h))) return MOE_EINVAL;
  if (prec == MOE_MXFP8 && dims->T > 0 && (!ptr_ok(x_perm_scale) || !ptr_ok(h_scale))) return MOE_EINVAL;
  const size_t need = workspace_size(dims, prec, 2);
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;
  Carver c(ws);
  FfnWs f = carve_ffn(c, dims, prec);
  if (prec == MOE_MXFP8)
    return run_gateup_mx(dims, static_cast<const uint8_t*>(x_perm), x_perm_scale, nullptr, expert_offsets, w,
                         static_cast<uint8_t*>(h), h_scale, f.prefix, static_cast<hipStream_t>(stream));
  return run_gateup(prec, x_perm, nullptr, 0, dims->d, expert_offsets, dims->T * dims->k, dims->E, w->w_gate,
                    w->w_up, dims->d, dims->I, h, f.prefix, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_down(const moe_dims* dims, moe_prec prec, const void* h, const uint8_t* h_scale,
                           const int32_t* expert_offsets, const moe_weights* w, void* o_perm, void* ws, size_t ws_bytes,
                           void* stream) {
  MOE_TRY(check_dims(dims, prec));
  MOE_TRY(check_weights(dims, prec, w, true, false, false));
  if (!ptr_ok(expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0 && (!ptr_ok(h) || !ptr_ok(o_perm))) return MOE_EINVAL;
  if (prec == MOE_MXFP8 && dims->T > 0 && !ptr_ok(h_scale)) return MOE_EINVAL;
  const size_t need = workspace_size(dims, prec, 2);
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EINVAL;
  if (dims->T == 0) return MOE_OK;
  Carver c(ws);
  FfnWs f = carve_ffn(c, dims, prec);
  if (prec == MOE_MXFP8)
    return run_down_mx(dims, static_cast<const uint8_t*>(h), h_scale, expert_offsets, w, o_perm, f.prefix,
                       static_cast<hipStream_t>(stream));
  return run_down(prec, expert_offsets, dims->T * dims->k, dims->E, w->w_down, dims->d, dims->I, h, o_perm, f.prefix,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_shared_ffn(const moe_dims* dims, moe_prec prec, const void* x, const moe_weights* w, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  MOE_TRY(check_weights(dims, prec, w, false, true, false));
  if (dims->T > 0 && (!ptr_ok(x) || !ptr_ok(y_shared))) return MOE_EINVAL;
  const size_t need = workspace_size(dims, prec, 3);
  if (need && (!ws || ws_bytes < need)) return MOE_EWORKSPACE;
  if (ws && !aligned16(ws)) return MOE_EINVAL;
  Carver c(ws);
  void* hs = carve_shared(c, dims, prec);
  return run_shared_ffn(dims, prec, x, w, y_shared, hs, static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_dims* dims, moe_prec prec, const void* o_perm, const int32_t* token_row,
                       const float* topk_w, const void* y_shared, void* y, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  if (dims->T > 0 && (!ptr_ok(o_perm) || !ptr_ok(token_row) || !ptr_ok(topk_w) || !ptr_ok(y))) return MOE_EINVAL;
  if (!opt_ok(y_shared)) return MOE_EINVAL;
  MOE_HIP(launch_combine(prec == MOE_F32, o_perm, token_row, topk_w, y_shared, y, dims->T, dims->d, dims->k,
                         static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_dims* dims, moe_prec prec, const void* x, const moe_weights* w,
                             const float* logit_bias, void* y, const moe_routing* routing, void* ws, size_t ws_bytes,
                             void* stream) {
  MOE_TRY(check_dims(dims, prec));
  MOE_TRY(check_weights(dims, prec, w, true, true, true));
  if (dims->T > 0 && (!ptr_ok(x) || !ptr_ok(y))) return MOE_EINVAL;
  if (!opt_ok(logit_bias)) return MOE_EINVAL;
  if (routing) {
    const void* f[] = {routing->logits, routing->topk_idx, routing->topk_w, routing->expert_counts,
                       routing->expert_offsets, routing->row_token, routing->token_row, routing->gu,
                       routing->gu_shared};
    for (const void* p : f)
      if (!opt_ok(p)) return MOE_EINVAL;
  }
  const size_t need = workspace_size(dims, prec, 0);
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver c(ws);
  FwdWs f = carve_forward(c, dims, prec, routing);
  if (dims->T == 0) {
    MOE_HIP(launch_schedule(nullptr, 0, dims->E, dims->k, f.counts, f.offsets, nullptr, nullptr, f.sched, s));
    return MOE_OK;
  }
  trace(0, 0, s);
  MOE_TRY(run_route(dims, prec, x, w->w_router, logit_bias, f.logits, f.topk_idx, f.topk_w, s));
  trace(0, 1, s);
  // Dispatch: the schedule places every route; in bf16 the grouped gate/up
  // GEMM then reads its A rows straight from x through row_token (the gather
  // rides in the GEMM's loads and x_perm is never written).
  // In MXFP8 the tokens are quantized once along d (row-wise, so it commutes
  // with the permutation) and the gate/up GEMM gathers the quantized rows.
  const bool fused_gather = prec != MOE_F32;
  MOE_TRY(run_permute(dims, prec, f.topk_idx, x, f.counts, f.offsets, f.row_token, f.token_row,
                      fused_gather ? nullptr : f.x_perm, f.x_perm_scale, f.sched, s));
  if (prec == MOE_MXFP8) {
    MOE_HIP(launch_quantize_mx(static_cast<const bf16_t*>(x), dims->T, dims->d, 0, static_cast<uint8_t*>(f.x_perm),
                               f.x_perm_scale, s));
    MOE_HIP(launch_gather_scales_slab(f.x_perm_scale, f.row_token, dims->T * dims->k, dims->d, f.xs_slab, s));
  }
  trace(0, 2, s);
  // G | U kept for a later backward when the caller provides the buffers
  // (bf16 and MXFP8: their backward consumes them).
  void* keep_gu = routing && prec != MOE_F32 ? routing->gu : nullptr;
  void* keep_gus = routing && prec != MOE_F32 ? routing->gu_shared : nullptr;
  if (dims->n_shared > 0) MOE_TRY(run_shared_ffn(dims, prec, x, w, f.y_shared, f.hs, s, keep_gus));
  trace(0, 3, s);
  if (prec == MOE_MXFP8)
    MOE_TRY(run_expert_ffn(dims, prec, f.x_perm, f.x_perm_scale, f.row_token, f.offsets, w, f.o_perm, f.ffn, s, true,
                           keep_gu, f.xs_slab));
  else if (fused_gather)
    MOE_TRY(run_expert_ffn(dims, prec, x, nullptr, f.row_token, f.offsets, w, f.o_perm, f.ffn, s, true, keep_gu));
  else
    MOE_TRY(run_expert_ffn(dims, prec, f.x_perm, nullptr, nullptr, f.offsets, w, f.o_perm, f.ffn, s, true));
  trace(0, 5, s);
  MOE_HIP(launch_combine(prec == MOE_F32, f.o_perm, f.token_row, f.topk_w, f.y_shared, y, dims->T, dims->d, dims->k,
                         s));
  trace(0, 6, s);
  return MOE_OK;
}

moe_status moe_layer_backward(const moe_dims* dims, moe_prec prec, const void* dy, const void* x,
                              const moe_weights* w, const moe_routing* routing, void* dx, const moe_grads* g, void* ws,
                              size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, prec));
  if (prec == MOE_F32) return MOE_EUNSUPPORTED;
  if (!g || !routing) return MOE_EINVAL;
  MOE_TRY(check_backward_weights(dims, prec, w, g->dw_router != nullptr));
  if (!ptr_ok(g->dw_gate) || !ptr_ok(g->dw_up) || !ptr_ok(g->dw_down) || !opt_ok(g->dw_router)) return MOE_EINVAL;
  if (dims->n_shared > 0 && (!ptr_ok(g->dws_gate) || !ptr_ok(g->dws_up) || !ptr_ok(g->dws_down))) return MOE_EINVAL;
  if (!ptr_ok(routing->expert_counts) || !ptr_ok(routing->expert_offsets)) return MOE_EINVAL;
  if (dims->T > 0) {
    const void* f[] = {dy, x, dx, g->dtopk_w, routing->topk_idx, routing->topk_w, routing->row_token,
                       routing->token_row};
    for (const void* p : f)
      if (!ptr_ok(p)) return MOE_EINVAL;
  }
  if (!opt_ok(routing->gu) || !opt_ok(routing->gu_shared)) return MOE_EINVAL;
  const size_t need = workspace_size(dims, prec, 4);
  if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
  if (!aligned16(ws)) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t E = dims->E, d = dims->d, I = dims->I, Is = dims->n_shared ? dims->I_shared : 0;
  if (dims->T == 0) {  // no tokens: every weight gradient is zero
    MOE_HIP(launch_fill_zero(g->dw_gate, (size_t)(E * I * d * 2), s));
    MOE_HIP(launch_fill_zero(g->dw_up, (size_t)(E * I * d * 2), s));
    MOE_HIP(launch_fill_zero(g->dw_down, (size_t)(E * I * d * 2), s));
    if (Is) {
      MOE_HIP(launch_fill_zero(g->dws_gate, (size_t)(Is * d * 2), s));
      MOE_HIP(launch_fill_zero(g->dws_up, (size_t)(Is * d * 2), s));
      MOE_HIP(launch_fill_zero(g->dws_down, (size_t)(Is * d * 2), s));
    }
    if (g->dw_router) MOE_HIP(launch_fill_zero(g->dw_router, (size_t)(E * d * 4), s));
    return MOE_OK;
  }
  Carver c(ws);
  BwdWs b = carve_backward(c, dims, prec);
  return run_backward(dims, static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(x), w, routing,
                      static_cast<bf16_t*>(dx), g, b, s);
}

moe_status moe_trace_events(int which, void* const* events, int n) {
  if ((which != 0 && which != 1) || n < 0 || n > kMaxTrace || (n > 0 && !events)) return MOE_EINVAL;
  for (int i = 0; i < kMaxTrace; ++i) g_trace[which][i] = i < n ? events[i] : nullptr;
  g_ntrace[which] = n;
  return MOE_OK;
}

moe_status moe_transpose_weights(const void* src, int64_t batch, int64_t rows, int64_t cols, void* dst,
                                 void* stream) {
  if (batch < 0 || rows < 0 || cols < 0) return MOE_EINVAL;
  if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!ptr_ok(src) || !ptr_ok(dst)) return MOE_EINVAL;
  if (batch > 65535 || (rows + 63) / 64 > INT_MAX || (cols + 63) / 64 > 65535) return MOE_EUNSUPPORTED;
  MOE_HIP(launch_transpose_batched(static_cast<const bf16_t*>(src), batch, rows, cols, static_cast<bf16_t*>(dst),
                                   static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_quantize_mxfp8(const void* src_bf16, int64_t rows, int64_t cols, int axis, uint8_t* dst, uint8_t* scale,
                              void* stream) {
  if (rows < 0 || cols < 0 || axis < 0 || axis > 2) return MOE_EINVAL;
  if ((axis == 0 && cols % 32) || (axis == 1 && rows % 32) || (axis == 2 && cols % 128)) return MOE_EINVAL;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!ptr_ok(src_bf16) || !ptr_ok(dst) || !scale) return MOE_EINVAL;
  if (axis != 1 && cols > INT_MAX) return MOE_EUNSUPPORTED;
  MOE_HIP(launch_quantize_mx(static_cast<const bf16_t*>(src_bf16), rows, cols, axis, dst, scale,
                             static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_bf16_mma_tiles(const void* a, const void* b, const float* c, float* d, int64_t n, void* stream) {
  if (n < 0 || n > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (!ptr_ok(a) || !ptr_ok(b) || !c || !d) return MOE_EINVAL;
  MOE_HIP(launch_bf16_mma_tiles(static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b), c, d, n,
                                static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_mx_mma_tiles(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, const uint8_t* b_scale,
                            const float* c, float* d, int64_t n, void* stream) {
  if (n < 0 || n > INT32_MAX) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  if (!ptr_ok(a) || !ptr_ok(b) || !a_scale || !b_scale || !c || !d) return MOE_EINVAL;
  MOE_HIP(launch_mx_mma_tiles(a, a_scale, b, b_scale, c, d, n, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
