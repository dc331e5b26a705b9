/* moe.h - C ABI of the MI355X (gfx950) MoE-layer library, libmoe.so.
 *
 * The operation is the DeepSeek-V3-style mixture-of-experts layer described
 * in the Mixture-of-Kittens blog post ("Overlapping computation and
 * communication in MoE"): a router projection chooses the top-k routed
 * experts of every token with a weight each; every chosen expert runs a
 * SwiGLU feed-forward network (gate and up projections, SwiGLU, down
 * projection); the layer output is the router-weighted sum of the chosen
 * experts' outputs plus the shared experts' outputs (weight 1).
 *
 * Conventions shared by every entry point
 *  - Pointers named in a signature are DEVICE pointers unless stated, and
 *    must be 16-byte aligned.  Matrices are row-major; weights use the
 *    [out][in] layout, stacked per expert.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  The library never allocates device memory, never synchronises
 *    the host and never reads device data on the host.  Scratch memory comes
 *    from the caller's workspace (size from moe_workspace_bytes).
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    any error status nothing has been enqueued (MOE_EHIP: a launch failed,
 *    earlier launches of the same call may have been enqueued) and outputs
 *    are undefined.  No exception crosses this boundary.
 *  - Inputs holding NaN or Inf are outside the contract.
 *  - Results are deterministic: identical inputs give bitwise identical
 *    outputs (no floating-point atomics anywhere).
 *
 * Precision modes (moe_prec)
 *  - MOE_F32:   every tensor fp32.
 *  - MOE_BF16:  activations, weights and outputs bf16; fp32 accumulation;
 *               router logits and weights fp32.
 *  - MOE_MXFP8: like MOE_BF16, but the routed-expert GEMMs take E4M3
 *               operands with one E8M0 scale per 32 elements along K (OCP MX
 *               v1.0); the shared expert and the router stay bf16 (blog post,
 *               "Other features / MXFP8 support").
 *
 * Shape limits: 1 <= k <= min(E, 16), E <= 1024, T >= 0, at most one
 * shared expert.  MOE_F32 needs d % 8 == 0.  MOE_BF16 needs d, I and I_s
 * multiples of 64; MOE_MXFP8 in addition d and I multiples of 128.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* bad argument: dims, NULL or misaligned pointer */
  MOE_EUNSUPPORTED = 2,  /* valid request that the library does not implement */
  MOE_EWORKSPACE = 3,    /* workspace missing or smaller than required */
  MOE_EHIP = 4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 } moe_prec;

/* Layer dimensions (host struct).  T tokens, model dim d, E routed experts,
 * top-k, routed intermediate dim I, n_shared shared experts of intermediate
 * dim I_shared.  R = T*k routed rows. */
typedef struct {
  int64_t T;
  int32_t d, E, k, I, n_shared, I_shared;
} moe_dims;

/* Weights (host struct of device pointers).  Element type: fp32 in MOE_F32,
 * bf16 otherwise.  ws_* are NULL when n_shared == 0.  In MOE_MXFP8 the
 * routed experts are read only from the pre-quantized copies q_* (produced
 * by moe_quantize_mxfp8(axis 2) of the stacked [E*rows][K] matrix along the
 * GEMM's K axis, i.e. along d for gate/up and along I for down: codes
 * [E][rows][K], scales slab-major [K/128][E*rows][4]); w_gate/w_up/w_down
 * may then be NULL. */
typedef struct {
  const void* w_router;                          /* [E][d] */
  const void* w_gate;                            /* [E][I][d] */
  const void* w_up;                              /* [E][I][d] */
  const void* w_down;                            /* [E][d][I] */
  const void* ws_gate;                           /* [S][I_s][d] */
  const void* ws_up;                             /* [S][I_s][d] */
  const void* ws_down;                           /* [S][d][I_s] */
  const uint8_t *q_gate, *q_gate_scale;          /* E4M3 [E][I][d], E8M0 [d/128][E*I][4] */
  const uint8_t *q_up, *q_up_scale;              /* E4M3 [E][I][d], E8M0 [d/128][E*I][4] */
  const uint8_t *q_down, *q_down_scale;          /* E4M3 [E][d][I], E8M0 [I/128][E*d][4] */
  /* Backward only: transposed copies for the input-gradient GEMMs, made
   * once per weight update with moe_transpose_weights (bf16). */
  const void* wt_gate;                           /* [E][d][I] = W_gate[e]^T */
  const void* wt_up;                             /* [E][d][I] = W_up[e]^T */
  const void* wt_down;                           /* [E][I][d] = W_down[e]^T */
  const void* wst_gate;                          /* [S][d][I_s] */
  const void* wst_up;                            /* [S][d][I_s] */
  const void* wst_down;                          /* [S][I_s][d] */
  /* Backward in MOE_MXFP8 only: the transposed routed copies quantized along
   * their rows (the input-gradient GEMMs' K): moe_quantize_mxfp8(axis 2) of
   * wt_gate, wt_up (blocks along I) and wt_down (blocks along d). */
  const uint8_t *qt_gate, *qt_gate_scale;        /* E4M3 [E][d][I], E8M0 [I/128][E*d][4] */
  const uint8_t *qt_up, *qt_up_scale;            /* E4M3 [E][d][I], E8M0 [I/128][E*d][4] */
  const uint8_t *qt_down, *qt_down_scale;        /* E4M3 [E][I][d], E8M0 [d/128][E*I][4] */
} moe_weights;

/* Gradients written by moe_layer_backward (host struct of caller-owned device
 * pointers).  Weight gradients are bf16 in the weights' layouts; the shared
 * ones are NULL when n_shared == 0.  dw_router NULL skips the router chain
 * (then dx has no router term). */
typedef struct {
  void* dw_gate;          /* [E][I][d] */
  void* dw_up;            /* [E][I][d] */
  void* dw_down;          /* [E][d][I] */
  void* dws_gate;         /* [S][I_s][d] */
  void* dws_up;           /* [S][I_s][d] */
  void* dws_down;         /* [S][d][I_s] */
  float* dtopk_w;         /* [T][k] fp32: dL/d topk_w, aligned with topk_idx */
  float* dw_router;       /* [E][d] fp32, or NULL */
} moe_grads;

/* Routing state of one forward pass and the activations kept for a later
 * backward (host struct of caller-owned device pointers).  Any field may be
 * NULL in moe_layer_forward (then it lives in the workspace, or for gu and
 * gu_shared is not kept). */
typedef struct {
  float* logits;          /* [T][E] fp32 */
  int32_t* topk_idx;      /* [T][k] ascending expert id */
  float* topk_w;          /* [T][k] fp32 */
  int32_t* expert_counts; /* [E] */
  int32_t* expert_offsets;/* [E+1] */
  int32_t* row_token;     /* [R] */
  int32_t* token_row;     /* [T][k] */
  void* gu;               /* [R][2I] bf16: gate and up projections G | U of every routed row */
  void* gu_shared;        /* [T][2I_s] bf16: G | U of the shared expert */
} moe_routing;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* Workspace needed by an entry point: which = 0 moe_layer_forward,
 * 1 moe_permute, 2 moe_expert_ffn, 3 moe_shared_ffn, 4 moe_layer_backward.
 * Writes the byte count to *bytes (host pointer).  Pure host computation. */
moe_status moe_workspace_bytes(const moe_dims* dims, moe_prec prec, int which, size_t* bytes);

/* Router projection, top-k selection and normalized weights.
 * Blog post, "Overlapping computation and communication in MoE" (router
 * projection, top-k, a router weight per chosen expert); paper summary
 * section 2.1 ("normalized router weights").
 *   logits[t][e] = fp32(x_t . W_r[e]) + bias[e] (bias optional, fp32 [E]),
 *                  the dot product an fp64 sum of fp32 partial sums over
 *                  64-element K chunks (16 in MOE_F32), rounded once;
 *   topk_idx[t]  = the k largest logits, ties to the smaller id, stored in
 *                  ascending id order;
 *   topk_w[t][j] = softmax of the selected logits.
 * Selection equals the selection on logits recomputed in fp64 (the dot
 * product in fp64, rounded to fp32, plus the bias): a rigorous bound on the
 * computed logits' error (Higham's gamma_64 times the token's largest
 * sum_i |x_i| |W_r[e][i]|, which the logits kernel also accumulates) sets a
 * window around the k-th/(k+1)-th boundary, and every expert inside it is
 * recomputed in fp64 before the selection is redone.  Operands in the bf16
 * subnormal range are outside that statement.  logits, topk_idx and topk_w
 * are outputs owned by the caller; topk_w also carries the per-token bound
 * from the logits kernel to the selection kernel. */
moe_status moe_route(const moe_dims* dims, moe_prec prec, const void* x, const void* w_router,
                     const float* logit_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream);

/* Schedule and dispatch: histogram of routes per expert, exclusive prefix
 * sum as region offsets, and the stable placement of every route into its
 * expert's region (expert-major, token-ascending), then the gather
 * x_perm[r] = x[row_token[r]].
 * Blog post, "Choosing the right communication direction / Scheduling"
 * (count per expert, prefix-sum offsets, re-walk the routes; tokens of an
 * expert land in contiguous rows) and "MXFP8 support" (activation
 * quantization fused into the dispatch).
 *   expert_counts [E], expert_offsets [E+1], row_token [R], token_row [T][k]:
 *   int32 outputs.  x_perm: [R][d] in the activation type, or E4M3 bytes in
 *   MOE_MXFP8 with x_perm_scale E8M0 [R][d/32]; x_perm may be NULL
 *   (schedule only).  ws: workspace of moe_workspace_bytes(which=1). */
moe_status moe_permute(const moe_dims* dims, moe_prec prec, const int32_t* topk_idx, const void* x,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                       int32_t* token_row, void* x_perm, uint8_t* x_perm_scale, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same outputs bit for bit, without a workspace argument.  Its scratch
 * (the schedule's per-block expert histograms, ceil(T/32) * E * 4 bytes)
 * lives in a static device array of moe_permute_noalloc_scratch_bytes()
 * bytes (16 MiB) that each GPU holds from its first call until the process
 * ends; larger requests (T above 131,072 tokens at E = 1024, or above
 * 524,288 at E = 256) return MOE_EWORKSPACE with nothing enqueued.  The
 * call allocates nothing, with no HIP or library allocation, but it looks
 * up the array's device address once per device.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from several host threads) race and give undefined outputs;
 * serialize them.  Nothing in the array needs clearing between calls: the
 * schedule writes every entry it reads. */
moe_status moe_permute_noalloc(const moe_dims* dims, moe_prec prec, const int32_t* topk_idx, const void* x,
                               int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                               int32_t* token_row, void* x_perm, uint8_t* x_perm_scale, void* stream);
size_t moe_permute_noalloc_scratch_bytes(void);

/* Routed expert FFNs on the permuted rows, grouped by expert:
 *   o_perm[r] = (SiLU(a W_g[e]^T) * (a W_u[e]^T)) W_d[e]^T,  a = x_perm[r],
 * for r in [expert_offsets[e], expert_offsets[e+1]).
 * Blog post, "Overlapping computation and communication in MoE" (gate and
 * up projections, SwiGLU, down projection per expert).
 * o_perm: [R][d] output in the activation type (bf16 in MOE_MXFP8).
 * ws: workspace of moe_workspace_bytes(which=2). */
moe_status moe_expert_ffn(const moe_dims* dims, moe_prec prec, const void* x_perm,
                          const uint8_t* x_perm_scale, const int32_t* expert_offsets,
                          const moe_weights* w, void* o_perm, void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them
 * separately (same contract, same workspace which=2):
 *   moe_expert_gate_up: h[r] = SiLU(a W_g[e]^T) * (a W_u[e]^T), h [R][I] in
 *     the activation type (MOE_MXFP8: E4M3 [R][I] quantized in the epilogue
 *     along I, blog post "MXFP8 support": activation quantization fused into
 *     the SwiGLU; h_scale E8M0 slab-major [I/128][R][4], the layout of
 *     moe_quantize_mxfp8 axis 2: byte (c/128, r, (c/32) % 4) is the scale of
 *     the block of row r holding column c);
 *   moe_expert_down: o_perm[r] = h[r] W_d[e]^T (MOE_MXFP8: h and h_scale in
 *     exactly that layout, e.g. moe_quantize_mxfp8(axis 2) of a bf16 h).
 * Blog post, "Scheduling the overlaps": up/gate projections with SwiGLU,
 * then the down projection, per expert. */
moe_status moe_expert_gate_up(const moe_dims* dims, moe_prec prec, const void* x_perm, const uint8_t* x_perm_scale,
                              const int32_t* expert_offsets, const moe_weights* w, void* h, uint8_t* h_scale,
                              void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_down(const moe_dims* dims, moe_prec prec, const void* h, const uint8_t* h_scale,
                           const int32_t* expert_offsets, const moe_weights* w, void* o_perm, void* ws,
                           size_t ws_bytes, void* stream);

/* Shared experts: y_shared[t] = sum_s FFN_s(x_t) in the activation type
 * (bf16 in MOE_MXFP8; the shared expert stays bf16, blog post "MXFP8
 * support").  With n_shared == 0 it writes zeros.
 * ws: workspace of moe_workspace_bytes(which=3). */
moe_status moe_shared_ffn(const moe_dims* dims, moe_prec prec, const void* x, const moe_weights* w,
                          void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* Weighted sum back to token order (blog post footnote to "Overlapping
 * computation and communication in MoE": the weighted sum is the last step):
 *   y[t] = sum_{j ascending expert} topk_w[t][j] * o_perm[token_row[t][j]]
 *          + y_shared[t]
 * accumulated in fp32 in that fixed order, rounded once to the output type.
 * y_shared may be NULL.  Tensors in the activation type (bf16 in MXFP8). */
moe_status moe_combine(const moe_dims* dims, moe_prec prec, const void* o_perm, const int32_t* token_row,
                       const float* topk_w, const void* y_shared, void* y, void* stream);

/* The whole forward: route, schedule and dispatch, shared and routed expert
 * FFNs, weighted sum.  y: [T][d] in the activation type.  routing: optional
 * caller buffers that receive the routing state (NULL or any NULL field:
 * kept in the workspace).  ws: workspace of moe_workspace_bytes(which=0). */
moe_status moe_layer_forward(const moe_dims* dims, moe_prec prec, const void* x, const moe_weights* w,
                             const float* logit_bias, void* y, const moe_routing* routing, void* ws,
                             size_t ws_bytes, void* stream);

/* Backward of the layer for an output gradient dy [T][d] (bf16), given the
 * forward's input x, weights (including the transposed copies wt_* and
 * wst_*) and its routing state (every field of `routing` except logits is
 * required: topk_idx, topk_w, expert_counts, expert_offsets, row_token,
 * token_row).  Writes dx [T][d] bf16 and the gradients in `g`.
 * Blog post, "Scheduling the overlaps" (backward: gather the output
 * gradient to the expert rows, the input-gradient GEMMs with the SwiGLU
 * backward, return the input gradients to token order, then the weight
 * gradients over each expert's whole token range) and "Router weight
 * gradient computation" (dL/dg of a route = <h, dY W_d>, fused into the
 * SwiGLU backward).  G and U come from routing->gu / gu_shared when the
 * forward kept them, else they are recomputed from x (the forward replay of
 * the blog post's "Reversed ring order" section).  Router chain, with the
 * selection held fixed: dl_j = g_j (dg_j - sum_i g_i dg_i) for the selected
 * experts, dW_router = dl^T x, dx += dl W_router.
 * Precision: MOE_BF16 (bf16 operands, fp32 accumulation) and MOE_MXFP8:
 * every routed-expert GEMM takes E4M3 operands with E8M0 scales along its
 * own K (blog post, "MXFP8 support"): dY and x along d, the weights as the
 * q_* (forward replay) and qt_* copies, dG and dU along I (quantized in the
 * SwiGLU-backward epilogue), and the weight-gradient operands along the
 * routed-row axis in blocks of 32 rows of one expert (each expert's rows
 * zero-padded to a multiple of 128); the shared expert and the router stay
 * bf16.  MOE_F32 returns MOE_EUNSUPPORTED.  Every reduction runs in a fixed
 * order (results are bitwise reproducible); experts without rows get exact
 * zero weight gradients.  ws: workspace of moe_workspace_bytes(which=4). */
moe_status moe_layer_backward(const moe_dims* dims, moe_prec prec, const void* dy, const void* x,
                              const moe_weights* w, const moe_routing* routing, void* dx, const moe_grads* g,
                              void* ws, size_t ws_bytes, void* stream);

/* dst[b][c][r] = src[b][r][c] for bf16 src [batch][rows][cols]: the
 * transposed weight copies of the backward (W_gate^T, W_up^T, W_down^T),
 * made once per weight update.  src and dst must not overlap. */
moe_status moe_transpose_weights(const void* src, int64_t batch, int64_t rows, int64_t cols, void* dst,
                                 void* stream);

/* Stage-timing hook for profiling (host state of the library, not
 * thread-safe).  events: n <= 32 caller-created hipEvent_t handles (host
 * array); the fused entry points then record events[i] on their stream at
 * stage boundary i, so that elapsed times between consecutive events give
 * each stage's device time.  n = 0 disables.  Boundaries:
 *   which = 0, moe_layer_forward: 0 start, 1 routed (router + top-k),
 *     2 scheduled (+ MXFP8 token quantization), 3 shared FFN done,
 *     4 routed gate/up done, 5 routed down done, 6 combine done;
 *   which = 1, moe_layer_backward: 0 start, 1 prepared (padded offsets, row
 *     weights, MXFP8 quantization of dY, and of x for the replay), 2 G|U
 *     replayed (when the forward did not keep them), 3 down dgrad
 *     + SwiGLU backward done, 4 router-weight gradients done, 5 gate/up dgrad
 *     done, 6 shared-expert input gradient done, 7 dx done, 8 transposes done,
 *     9 dW_down done, 10 dW_gate and dW_up done (one launch), 11 shared
 *     weight gradients done, 12 router gradient done. */
moe_status moe_trace_events(int which, void* const* events, int n);

/* Tuning knob (host state of the library, process-wide, not thread-safe):
 * caps the persistent grids of the grouped GEMMs at n workgroups (rounded
 * down to a multiple of 8, the XCD count, and at least 8), e.g. to leave
 * compute units to other work; n = 0 restores one workgroup per compute
 * unit.  Results are bitwise identical for every n: which workgroup runs a
 * tile, and in which order, never changes a tile's arithmetic (blog post,
 * "Determinism").  Takes effect for calls enqueued afterwards. */
moe_status moe_set_max_workgroups(int n);

/* MX quantization of a bf16 matrix src [rows][cols] (OCP MX v1.0; blog post
 * "MXFP8 support": a quantization kernel pre-quantizes the weights).
 * axis = 0: one block per 32 consecutive elements of a row (cols % 32 == 0):
 *   dst [rows][cols] E4M3, scale [rows][cols/32] E8M0.
 * axis = 1: one block per 32 consecutive rows of a column (rows % 32 == 0):
 *   dst [rows][cols] E4M3, scale [rows/32][cols] E8M0.
 * axis = 2: the blocks of axis 0 (cols % 128 == 0) with the scales stored
 *   slab-major for the grouped GEMMs: scale [cols/128][rows][4], byte
 *   (c/128, r, (c/32) % 4) for the block of row r holding column c (the four
 *   block scales of one row's 128-column slab form one dword, and a slab's
 *   dwords are contiguous over the rows).
 * Per block: e = the smallest integer with max |v| / 2^e <= 448 (the finest
 * power-of-two scale that leaves the block maximum unclipped), clamped to
 * [-127, 127] (-127 for an all-zero block); element = v / 2^e rounded to
 * nearest-even E4M3, sign kept; scale byte = e + 127.  Every MX operand the
 * library quantizes itself (tokens, h, gradients) uses the same rule. */
moe_status moe_quantize_mxfp8(const void* src_bf16, int64_t rows, int64_t cols, int axis, uint8_t* dst,
                              uint8_t* scale, void* stream);

/* Routed-row-axis MX quantization of a weight-gradient operand (the K axis
 * of the MXFP8 weight-gradient GEMMs is the routed rows; blog post, "MXFP8
 * support": quantization fused into the grouped GEMMs).  For every group e in
 * [0, nseg): rows r in [seg_off[e], seg_off[e+1]) of a bf16 matrix (row r is
 * src row gather[r] when gather is not NULL, else src row r; ld_src elements
 * between rows), transposed into a [cols][Kp_e] block of E4M3 codes at byte
 * pad_off[e] * cols of dst, Kp_e = pad_off[e+1] - pad_off[e] (a multiple of
 * 128, at least the group's row count; positions past the group's rows hold
 * zeros), quantized in blocks of 32 consecutive positions of one column with
 * the scale rule of moe_quantize_mxfp8.  Scales slab-major per group:
 * [Kp_e/128][cols][4] at byte pad_off[e] * cols / 32, byte (p/128) * cols * 4
 * + c * 4 + (p/32) % 4 of the block for position p of column c.  This is the
 * layout moe_layer_backward builds for x and dY in MOE_MXFP8.
 * seg_off, pad_off: device int32 [nseg+1]; gather: device int32 or NULL;
 * p_cap: a multiple of 128, at least pad_off[nseg] (sizes the launch); cols
 * a multiple of 8; dst and dst_scale hold p_cap * cols and p_cap * cols / 32
 * bytes. */
moe_status moe_quantize_mxfp8_rows_t(const void* src_bf16, int64_t ld_src, int32_t cols, const int32_t* gather,
                                     const int32_t* seg_off, const int32_t* pad_off, int32_t nseg, int64_t p_cap,
                                     uint8_t* dst, uint8_t* dst_scale, void* stream);

/* The matrix-core operation under every MXFP8 GEMM of the library, one per
 * tile (blog post "MXFP8 support": the routed experts' GEMMs take E4M3
 * operands with one E8M0 scale per 32 elements along K; OCP MX v1.0).  For
 * each tile t in [0, n): d[t] = c[t] + A[t] B[t]^T, with A[t] and B[t]
 * [32][64] E4M3 codes (row-major, K contiguous; a and b hold n * 2048 bytes,
 * 16-byte aligned), a_scale[t] and b_scale[t] [32][2] E8M0 codes (the scale
 * of K[32j, 32j+32) of row i at byte 64t + 2i + j), c[t] and d[t] [32][32]
 * fp32 row-major (n * 4096 bytes each; d may alias c).  Each tile is one
 * gfx950 v_mfma_scale_f32_32x32x64_f8f6f4 with its operands in the lanes
 * where the grouped GEMMs put them, so the rounding of that instruction,
 * which those GEMMs inherit, can be measured and tested.  Device pointers;
 * n = 0 is a no-op; EINVAL for n < 0 or above INT32_MAX, a null pointer, or
 * a or b not 16-byte aligned. */
moe_status moe_mx_mma_tiles(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, const uint8_t* b_scale,
                            const float* c, float* d, int64_t n, void* stream);

/* The bf16 matrix-core operation under the bf16 grouped GEMMs and the router
 * logits (blog post "MoE layer benchmarks": the layers run in bf16; the
 * router's exact selection relies on a bound of this instruction's
 * accumulation error).  For each tile t in [0, n): d[t] = c[t] + A[t] B[t]^T,
 * with A[t] and B[t] [32][16] bf16 (row-major, K contiguous; a and b hold
 * n * 1024 bytes, 16-byte aligned), c[t] and d[t] [32][32] fp32 row-major
 * (d may alias c).  Each tile is one gfx950 v_mfma_f32_32x32x16_bf16 with its
 * operands in the lanes where the bf16 GEMMs put them.  Device pointers;
 * n = 0 is a no-op; EINVAL for n < 0 or above INT32_MAX, a null pointer, or
 * a or b not 16-byte aligned. */
moe_status moe_bf16_mma_tiles(const void* a, const void* b, const float* c, float* d, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif
