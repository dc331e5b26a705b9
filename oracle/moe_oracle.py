"""CPU oracle of the DeepSeek-V3-style MoE layer (test infrastructure).

This module is test infrastructure, not part of the product: only the tests,
the package smoke check and the CPU-baseline leg of the benchmark import it.
It shares no code with the GPU library and never calls it.

It is the plain definition of what the layer computes, in float64 (numpy),
with no blocking, fusion or reordering beyond what the definition states.
Library primitives (matrix products, sorts) serve as single steps.

Sources (the pages of the Mixture-of-Kittens paper and blog post):
  * blog post "Mixture-of-Kittens", section "Overlapping computation and
    communication in MoE": a router projection picks the top-k routed experts
    and a router weight for each; every selected expert runs up and gate
    projections, SwiGLU and a down projection; the layer combines shared and
    routed expert outputs with the router weights;
  * paper summary, section 2.1 "MoE and Expert Parallelism": shared and
    selected routed-expert FFNs are applied to every token and their outputs
    summed using normalized router weights;
  * blog post, section "Choosing the right communication direction /
    Scheduling": the pull schedule counts routes per local expert, takes an
    exclusive prefix sum as region offsets and re-walks the routes to write
    the table whose row index is the destination row (no sorting);
  * blog post, footnote to the same section: the weighted reduction is the
    separate last step ("weighted sum");
  * blog post, "Other features / MXFP8 support": routed experts in MXFP8,
    shared expert stays BF16; block format from "Microscaling Data Formats for
    Deep Learning" (cited by the paper), read as OCP MX v1.0 E4M3 elements
    with one E8M0 scale per 32 elements; the scale is the smallest power of
    two that keeps the block maximum unclipped (see mx_scale_exponent);
  * blog post, "Other features / Router weight gradient computation": the
    router-weight gradient is the inner product of the SwiGLU activation and
    the down-projection input gradient.

Readings where the pages are garbled or silent (the layer equation did not
survive extraction):
  * router weights: softmax over the selected k logits (the full softmax
    restricted to the top-k and renormalized; the full denominator cancels);
  * top-k ties: the smaller expert id wins; selected ids are stored ascending;
  * the shared expert is added with weight 1;
  * SwiGLU applies SiLU to the gate projection and multiplies by the up
    projection;
  * the routed rows are laid out expert-major, token-ascending inside each
    expert (the pull-schedule walk with a single source rank).

Parity status of every function is pinned by tests (tests/test_oracle_*.py);
nothing here is "parity unpinned".
"""
import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Router: projection, top-k, normalized weights
# --------------------------------------------------------------------------
def router_logits(x, w_router, bias=None):
    """Router projection logits[t][e] = x_t . W_r[e] (+ b_e).

    Blog post, "Overlapping computation and communication in MoE" (a router
    projection per token).  Each dot product is formed in float64 and rounded
    once to fp32; an optional fp32 logit bias is then added in fp32.
    x: [T][d], w_router: [E][d] (float64 holding the stored values).
    """
    logits = (np.asarray(x, F64) @ np.asarray(w_router, F64).T).astype(F32)
    if bias is not None:
        logits = (logits + np.asarray(bias, F32)).astype(F32)
    return logits


def topk_route(logits, k):
    """Top-k expert ids per token, ascending by id.

    Blog post, "Overlapping computation and communication in MoE": the router
    selects the top-k routed experts.  Order: larger logit first, equal
    logits resolved towards the smaller expert id; the k winners are then
    stored in ascending id order.
    """
    logits = np.asarray(logits, F32)
    T, E = logits.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> sort by -logit, then by id.
    order = np.lexsort((ids, -logits.astype(F64)), axis=-1)
    top = np.sort(order[:, :k], axis=1)
    return top.astype(np.int32)


def renormalized_weights(logits, topk_idx):
    """Normalized router weights g[t][j] over the selected experts.

    Paper summary, section 2.1 ("normalized router weights"): softmax of the
    selected logits, g_j = exp(l_j - m) / sum_i exp(l_i - m) with m the largest
    selected logit; computed in float64, rounded once to fp32.
    """
    sel = np.take_along_axis(np.asarray(logits, F64), np.asarray(topk_idx, np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return (e / e.sum(axis=1, keepdims=True)).astype(F32)


# --------------------------------------------------------------------------
# Schedule (pull-schedule algorithm with one source rank = counting sort)
# --------------------------------------------------------------------------
def schedule(topk_idx, E):
    """Counts, region offsets and the row table of the routed rows.

    Blog post, "Choosing the right communication direction / Scheduling":
    (1) count the routes of every expert; (2) exclusive prefix sum of the
    counts gives each expert's region offset; (3) walk the routes again
    (token-major, then route slot) and give each route the next free row of
    its expert's region.  With a single source rank the schedule table entry
    of a row is the source token index.

    Returns counts[E], offsets[E+1], row_token[R] (row -> token) and
    token_row[T][k] (route -> row), all int32.
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[topk_idx[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    row_token = np.zeros(T * k, dtype=np.int64)
    token_row = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = topk_idx[t, j]
            r = cursor[e]
            cursor[e] += 1
            row_token[r] = t
            token_row[t, j] = r
    return (counts.astype(np.int32), offsets.astype(np.int32), row_token.astype(np.int32),
            token_row.astype(np.int32))


def permute(x, row_token):
    """Dispatch on one device: routed row r holds token row_token[r].

    Blog post, "Scheduling": tokens of an expert land in contiguous rows so
    that the expert-grouped GEMMs need no further reordering.
    """
    return np.asarray(x)[np.asarray(row_token, np.int64)]


# --------------------------------------------------------------------------
# Expert FFN (SwiGLU)
# --------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, F64)))


def swiglu_ffn(a, w_gate, w_up, w_down):
    """FFN(a) = (SiLU(a W_g^T) * (a W_u^T)) W_d^T, all in float64.

    Blog post, "Overlapping computation and communication in MoE": up and
    gate projections, a SwiGLU activation, a down projection.
    a: [n][d], w_gate, w_up: [I][d], w_down: [d][I].  Returns (out, G, U, h).
    """
    a = np.asarray(a, F64)
    G = a @ np.asarray(w_gate, F64).T
    U = a @ np.asarray(w_up, F64).T
    h = silu(G) * U
    return h @ np.asarray(w_down, F64).T, G, U, h


# --------------------------------------------------------------------------
# Weighted sum and the whole layer
# --------------------------------------------------------------------------
def combine(o_perm, token_row, topk_w, y_shared=None):
    """y_t = sum over the token's experts in ascending id of g * O[row] (+ shared).

    Blog post footnote to "Overlapping computation and communication in MoE":
    the weighted sum is the last step.  Accumulated in float64.
    """
    o_perm = np.asarray(o_perm, F64)
    token_row = np.asarray(token_row, np.int64)
    g = np.asarray(topk_w, F64)
    T, k = token_row.shape
    y = np.zeros((T, o_perm.shape[1]), dtype=F64) if y_shared is None else np.array(y_shared, F64)
    for j in range(k):
        y += g[:, j:j + 1] * o_perm[token_row[:, j]]
    return y


def shared_ffn(x, ws_gate, ws_up, ws_down):
    """Sum of the shared experts' FFNs (weight 1 each), float64 [T][d]."""
    x = np.asarray(x, F64)
    y = np.zeros_like(x)
    for s in range(0 if ws_gate is None else len(ws_gate)):
        y += swiglu_ffn(x, ws_gate[s], ws_up[s], ws_down[s])[0]
    return y


def layer_forward(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, k):
    """The MoE layer forward: route, schedule, expert FFNs, weighted sum.

    Returns a dict with logits, topk_idx, topk_w, counts, offsets, row_token,
    token_row, o_perm (float64), y_shared (float64) and y (float64).
    w_gate/w_up: [E][I][d], w_down: [E][d][I]; shared: [S][I_s][d] etc.
    """
    E = len(w_router)
    logits = router_logits(x, w_router, bias)
    idx = topk_route(logits, k)
    g = renormalized_weights(logits, idx)
    counts, offsets, row_token, token_row = schedule(idx, E)
    a = permute(np.asarray(x, F64), row_token)
    o_perm = np.zeros_like(a)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            o_perm[lo:hi] = swiglu_ffn(a[lo:hi], w_gate[e], w_up[e], w_down[e])[0]
    y_shared = shared_ffn(x, ws_gate, ws_up, ws_down)
    y = combine(o_perm, token_row, g, y_shared)
    return dict(logits=logits, topk_idx=idx, topk_w=g, counts=counts, offsets=offsets,
                row_token=row_token, token_row=token_row, o_perm=o_perm, y_shared=y_shared, y=y)


def token_forward(x_t, idx_t, g_t, expert_weights, shared_weights):
    """Forward of one token given its routing: sum_j g_j FFN_{e_j}(x_t) + shared.

    Used to check samples of workloads too large for a full oracle run; the
    arithmetic is that of ``layer_forward`` restricted to one token.
    expert_weights(e) -> (w_gate[e], w_up[e], w_down[e]) in float64.
    """
    x_t = np.asarray(x_t, F64)[None, :]
    y = np.zeros(x_t.shape[1], dtype=F64)
    for e, g in zip(idx_t, g_t):
        wg, wu, wd = expert_weights(int(e))
        y += float(g) * swiglu_ffn(x_t, wg, wu, wd)[0][0]
    for wg, wu, wd in shared_weights:
        y += swiglu_ffn(x_t, wg, wu, wd)[0][0]
    return y


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------
def silu_grad(z):
    """d SiLU / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    s = sigmoid(z)
    z = np.asarray(z, F64)
    return s * (1.0 + z * (1.0 - s))


def ffn_backward(a, w_gate, w_up, w_down, dout):
    """Gradients of FFN(a) for an output gradient dout (all float64).

    Returns dA, dW_gate, dW_up, dW_down and h, dH (the down-projection input
    gradient).  The weight gradients sum over the rows of a in row order.
    """
    a = np.asarray(a, F64)
    G = a @ np.asarray(w_gate, F64).T
    U = a @ np.asarray(w_up, F64).T
    sg = silu(G)
    h = sg * U
    dout = np.asarray(dout, F64)
    dH = dout @ np.asarray(w_down, F64)
    dG = dH * U * silu_grad(G)
    dU = dH * sg
    dA = dG @ np.asarray(w_gate, F64) + dU @ np.asarray(w_up, F64)
    return dA, dG.T @ a, dU.T @ a, dout.T @ h, h, dH


def layer_backward(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, k, dy,
                   with_router=True):
    """Gradients of the MoE layer for an output gradient dy.

    Per route (t, e) with weight g: dO = g dY_t; the router-weight gradient
    dg = <dY_t, O> equals <h, dY_t W_d> (blog post, "Router weight gradient
    computation": inner product of the SwiGLU activation and the
    down-projection input gradient).  dX sums each token's routed input
    gradients and the shared expert's.  Router chain (selection treated as
    constant): dl_i = g_i (dg_i - sum_j g_j dg_j) for selected i, else 0;
    dW_r = dl^T x and dX += dl W_r.
    """
    fw = layer_forward(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, k)
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    E = len(w_router)
    T, d = x.shape
    idx, g = fw["topk_idx"], fw["topk_w"].astype(F64)
    offsets, row_token, token_row = fw["offsets"], fw["row_token"], fw["token_row"]
    R = T * k
    # route weight of every routed row
    g_row = np.zeros(R, dtype=F64)
    for t in range(T):
        for j in range(k):
            g_row[token_row[t, j]] = g[t, j]
    a = permute(x, row_token)
    dy_perm = permute(dy, row_token)
    dA_perm = np.zeros((R, d), dtype=F64)
    dg_row = np.zeros(R, dtype=F64)
    dWg = np.zeros(np.shape(w_gate), dtype=F64)
    dWu = np.zeros(np.shape(w_up), dtype=F64)
    dWd = np.zeros(np.shape(w_down), dtype=F64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        dout = g_row[lo:hi, None] * dy_perm[lo:hi]
        dA, dWg[e], dWu[e], dWd[e], h, dH = ffn_backward(a[lo:hi], w_gate[e], w_up[e], w_down[e], dout)
        dA_perm[lo:hi] = dA
        # unscaled down-projection input gradient dH' = dH / g
        dHp = dy_perm[lo:hi] @ np.asarray(w_down[e], F64)
        dg_row[lo:hi] = np.sum(h * dHp, axis=1)
    dx = np.zeros((T, d), dtype=F64)
    for j in range(k):
        dx += dA_perm[token_row[:, j]]
    S = 0 if ws_gate is None else len(ws_gate)
    dWsg = np.zeros(np.shape(ws_gate), dtype=F64) if S else None
    dWsu = np.zeros(np.shape(ws_up), dtype=F64) if S else None
    dWsd = np.zeros(np.shape(ws_down), dtype=F64) if S else None
    for s in range(S):
        dA, dWsg[s], dWsu[s], dWsd[s], _, _ = ffn_backward(x, ws_gate[s], ws_up[s], ws_down[s], dy)
        dx += dA
    dg = dg_row[token_row]
    out = dict(fw=fw, dx=dx, dw_gate=dWg, dw_up=dWu, dw_down=dWd, dtopk_w=dg,
               dws_gate=dWsg, dws_up=dWsu, dws_down=dWsd)
    if with_router:
        dl = np.zeros((T, E), dtype=F64)
        inner = np.sum(g * dg, axis=1, keepdims=True)
        dsel = g * (dg - inner)
        np.put_along_axis(dl, idx.astype(np.int64), dsel, axis=1)
        out["dlogits"] = dl
        out["dw_router"] = dl.T @ x
        out["dx"] = dx + dl @ np.asarray(w_router, F64)
    return out


# --------------------------------------------------------------------------
# MXFP8 (OCP MX v1.0: E4M3 elements, one E8M0 scale per 32-element block)
# --------------------------------------------------------------------------
E4M3_MAX = 448.0
E4M3_EMAX = 8            # exponent of the largest normal, 448 = 1.75 * 2^8
E4M3_MIN_NORMAL_EXP = -6
MX_BLOCK = 32


def e4m3_round(v):
    """Round float64 values to the E4M3FN grid: nearest, ties to even,
    subnormals kept (quantum 2^-9 below 2^-6), saturating at +-448."""
    v = np.asarray(v, F64)
    a = np.abs(v)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - 3)            # 3 mantissa bits
    q = np.rint(a / quantum) * quantum        # np.rint: ties to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, v)


def e4m3_encode(q):
    """Bit patterns (uint8) of values already on the E4M3FN grid."""
    q = np.asarray(q, F64)
    sign = (np.signbit(q)).astype(np.uint32) << 7
    a = np.abs(q)
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** E4M3_MIN_NORMAL_EXP
    # normal: a = (1 + m/8) 2^e, field = e + 7 ; subnormal: a = m/8 2^-6
    m_norm = np.rint(np.where(normal, a / np.ldexp(1.0, e) - 1.0, 0.0) * 8).astype(np.uint32)
    m_sub = np.rint(a / 2.0 ** -9).astype(np.uint32)
    field = np.where(normal, (e + 7).astype(np.int64), 0).astype(np.uint32)
    mant = np.where(normal, m_norm, m_sub)
    return (sign | (field << 3) | mant).astype(np.uint8)


def e4m3_decode(bits):
    """float64 values of E4M3FN bit patterns (0x7F / 0xFF are NaN)."""
    b = np.asarray(bits, np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    f = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(f == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, f - 7))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return s * val


def mx_scale_exponent(amax):
    """Shared block exponent: the smallest integer e with amax / 2^e <= 448,
    i.e. the finest power-of-two scale at which the block's largest magnitude
    is still an E4M3 value without clipping; clamped to [-127, 127] (the E8M0
    range); an all-zero block takes -127 (E8M0 code 0).

    Reading: the pages fix the format (E4M3 elements, one power-of-two E8M0
    scale per 32 elements; blog post "MXFP8 support") but not how an encoder
    picks the scale.  The MX paper's rule, floor(log2 amax) - 8, maps a block
    maximum with mantissa above 1.75 past 448, where it is clipped by up to
    12.5%; this rule never clips and is otherwise the same (it is one larger
    exactly when that happens).
    """
    amax = np.asarray(amax, F64)
    pos = amax > 0
    _, ex = np.frexp(np.where(pos, amax, 1.0))      # amax = m 2^ex, m in [0.5, 1)
    e = ex - 1 - E4M3_EMAX                          # floor(log2 amax) - 8: amax / 2^e in [256, 512)
    e = e + (np.where(pos, amax, 0.0) > E4M3_MAX * np.ldexp(1.0, e))   # past 448: one step coarser
    e = np.clip(e, -127, 127)
    return np.where(pos, e, -127).astype(np.int64)


def mx_quantize(v, axis=-1):
    """MX-quantize along `axis` (length a multiple of 32).

    Returns (codes uint8 E4M3 bits, same shape as v) and (scales uint8 E8M0
    codes, with the axis length divided by 32).  Elements are v / 2^e_s
    rounded to E4M3 (ties to even; saturation is reached only where the
    scale is clamped at the top of the E8M0 range).
    """
    v = np.moveaxis(np.asarray(v, F64), axis, -1)
    n = v.shape[-1]
    assert n % MX_BLOCK == 0
    blocks = v.reshape(*v.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    e_s = mx_scale_exponent(np.max(np.abs(blocks), axis=-1))
    q = e4m3_round(blocks / np.ldexp(1.0, e_s)[..., None])
    codes = e4m3_encode(q).reshape(v.shape)
    scales = (e_s + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes, scales, axis=-1):
    """float64 values of an MX tensor (inverse of the encoding, not of rounding)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64) - 127
    vals = e4m3_decode(c).reshape(*c.shape[:-1], c.shape[-1] // MX_BLOCK, MX_BLOCK)
    out = (vals * np.ldexp(1.0, s)[..., None]).reshape(c.shape)
    return np.moveaxis(out, -1, axis)
