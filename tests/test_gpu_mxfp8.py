"""GPU parity of the MXFP8 forward: the quantizer and the quantizing
dispatch bit-exact against the oracle's MX quantizer; routed-expert MXFP8
GEMMs and the whole layer within 3e-2 of a quantization-aware float64 model
(the oracle's quantizer at the path's quantization points, exact arithmetic
otherwise: the kernels' own error), and on the small shapes element by
element: G and U, every scale and code of h, and the down projection each
within a bound derived from the matrix cores' measured accumulation
(tests/mma_rules.py); held to the stated 6e-2
(max|d|/max|ref|) against the float64 oracle of the unquantized layer, an
expected failure only where MX rounding alone exceeds it."""
import numpy as np
import pytest

import gen
from oracle import moe_oracle as O
from tests.moe_parity import TOL, HostProblem, check_mx_bound, device_problem, rel_err, rms_rel, to_np
from tests.mma_rules import mx_dot

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


SMALL = {
    "mx_ragged": gen.Dims("mx_ragged", 300, 256, 16, 4, 256, 1, 128, "mxfp8", 0.0),
    "mx_skew_noshared": gen.Dims("mx_skew_noshared", 513, 384, 32, 8, 128, 0, 0, "mxfp8", 1.2),
    "mx_k1": gen.Dims("mx_k1", 77, 128, 4, 1, 128, 1, 64, "mxfp8", 0.0),
    "mx_kE": gen.Dims("mx_kE", 64, 128, 8, 8, 128, 0, 0, "mxfp8", 0.0),
    "mx_E1": gen.Dims("mx_E1", 130, 128, 1, 1, 128, 0, 0, "mxfp8", 0.0),
    # the ABI's limits: E = 1024 experts, k = 16
    "mx_max_E_k": gen.Dims("mx_max_E_k", 300, 128, 1024, 16, 128, 1, 64, "mxfp8", 1.2),
    "mx_one_token": gen.Dims("mx_one_token", 1, 256, 16, 4, 256, 1, 128, "mxfp8", 0.0),
}


@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_bit_exact(axis):
    import mixture_experts_layer_prefix_amd as M
    D = gen.Dims("q", 64, 192, 8, 2, 96, 0, 0, "bf16", 0.0)
    p = gen.Problem(D)
    w = p.device("w_down").reshape(-1, D.I)  # [E*d][I] = [1536][96]
    q, s = M.quantize_mxfp8(w, axis)
    # ABI axis 0 = blocks of 32 consecutive elements of a row = numpy axis 1
    rq, rs = O.mx_quantize(p.host("w_down").reshape(-1, D.I), axis=1 - axis)
    assert np.array_equal(to_np(q), rq) and np.array_equal(to_np(s), rs)


def test_quantizer_slab_major_bit_exact():
    """axis 2: the blocks of axis 0 with the scales slab-major [cols/128][rows][4]
    (the grouped GEMMs' weight layout): the same codes, and the oracle's
    [rows][cols/32] scales regrouped by 128-column slab."""
    import mixture_experts_layer_prefix_amd as M
    D = gen.Dims("q2", 64, 256, 8, 2, 128, 0, 0, "bf16", 0.0)
    p = gen.Problem(D)
    w = p.device("w_gate").reshape(-1, D.d)  # [E*I][d] = [1024][256]
    q, s = M.quantize_mxfp8(w, 2)
    rq, rs = O.mx_quantize(p.host("w_gate").reshape(-1, D.d), axis=1)
    rows = rq.shape[0]
    assert tuple(s.shape) == (D.d // 128, rows, 4)
    assert np.array_equal(to_np(q), rq)
    assert np.array_equal(to_np(s), rs.reshape(rows, D.d // 128, 4).transpose(1, 0, 2))


def mx_round(v, axis=-1):
    """Values after an MX quantize/dequantize round trip (oracle quantizer)."""
    q, sc = O.mx_quantize(v, axis=axis)
    return O.mx_dequantize(q, sc, axis=axis)


def e4m3_quantum(a):
    """Spacing of the E4M3 grid at magnitudes a: 3 mantissa bits above 2^-6,
    the fixed subnormal step 2^-9 below."""
    _, ex = np.frexp(np.maximum(np.asarray(a, np.float64), 2.0 ** O.E4M3_MIN_NORMAL_EXP))
    return np.ldexp(1.0, ex - 1 - 3)


def check_gate_up_elementwise(p, D, ref, gu, h, h_scale):
    """Element-wise bounds on the MXFP8 gate/up GEMM and its epilogue, each
    derived from the arithmetic (G, U from MX-rounded x and weights, exact
    products, the matrix cores' accumulation as bounded by mx_dot):
      G, U (kept in bf16): |G_k - G| <= 2^-8 max(|G_k|, |G|) + mx_dot's bound;
      h = silu(G) U, evaluated in fp32 from the fp32 G and U: within dh of the
        exact value (silu is 1.1-Lipschitz; 2^-16 relative covers exp,
        reciprocal and product rounding);
      each 32-element scale: the block-exponent rule applied to some block
        maximum within the band [max(|h| - dh), max(|h| + dh)];
      each code at its block's scale: within half an E4M3 step plus dh of h,
        i.e. round-to-nearest of a value in h's band.
    Which of two codes a value in the band takes, and which of two scales at a
    boundary, is left open: both are correct roundings of a correctly
    accumulated fp32 value.  Returns the decoded h and the counts of such
    open decisions (codes, scales) taken differently from float64."""
    a = mx_round(p.host("x"))[ref["row_token"]]
    off = ref["offsets"]
    R, I = D.R, D.I
    G, U, dG, dU = (np.zeros((R, I)) for _ in range(4))
    for e in range(D.E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        wg, wu = mx_round(p.host_expert("w_gate", e)), mx_round(p.host_expert("w_up", e))
        G[lo:hi], dG[lo:hi] = mx_dot(a[lo:hi], wg)
        U[lo:hi], dU[lo:hi] = mx_dot(a[lo:hi], wu)
    for name, k, m, dm in (("G", gu[:, :I], G, dG), ("U", gu[:, I:], U, dU)):
        over = np.abs(k - m) - (2.0 ** -8 * np.maximum(np.abs(k), np.abs(m)) + dm)
        assert np.all(over <= 0), "%s off by %.3e beyond its bound at %s" % (
            name, over.max(), np.unravel_index(np.argmax(over), over.shape))
    sc = h_scale.transpose(1, 0, 2).reshape(R, I // 32)
    h_dec, h64 = check_mx_h(G, U, dG, dU, h, sc)
    qm, sm = O.mx_quantize(h64)
    return h_dec, int(np.sum(qm != h)), int(np.sum(sm != sc))


def check_mx_h(G, U, dG, dU, codes, scales):
    """h = silu(G) U quantized by the gate/up epilogue, on any [n][c] set of
    rows and whole 32-column blocks: G, U (float64, exact from the MX-rounded
    operands) and their accumulation bounds dG, dU, the kernel's E4M3 codes
    [n][c] and E8M0 scales [n][c/32].  Each scale must be the block rule's
    exponent for some block maximum within h's band, each code within half an
    E4M3 step plus the band of h.  Returns the decoded h and the float64 h."""
    n, c = G.shape
    s = O.silu(G)
    h64 = s * U
    dh = 1.1 * dG * (np.abs(U) + dU) + (np.abs(s) + 1.1 * dG) * dU + 2.0 ** -16 * (np.abs(s) + 1.1 * dG) * (np.abs(U) + dU)
    sc = np.asarray(scales).astype(np.int64)
    blk = lambda v: v.reshape(n, c // 32, 32)
    e_lo = O.mx_scale_exponent(np.max(np.maximum(blk(np.abs(h64) - dh), 0.0), axis=-1)) + 127
    e_hi = O.mx_scale_exponent(np.max(blk(np.abs(h64) + dh), axis=-1)) + 127
    bad = (sc < e_lo) | (sc > e_hi)
    assert not bad.any(), "h scale outside the admissible range at %s" % (np.argwhere(bad)[:5],)
    step = np.ldexp(1.0, np.repeat(sc - 127, 32, axis=1))
    h_dec = O.e4m3_decode(codes) * step
    half = 0.5 * e4m3_quantum(np.maximum(np.abs(h_dec), np.abs(h64) + dh) / step) * step
    over = np.abs(h_dec - h64) - (half + dh)
    assert np.all(over <= 0), "h code off by %.3e beyond half a step plus its band at %s" % (
        over.max(), np.unravel_index(np.argmax(over), over.shape))
    return h_dec, h64


def check_down_elementwise(p, D, ref, h_dec, o_perm):
    """o_perm (bf16) against the exact product of the kernel's own decoded h
    and the MX-rounded W_down: within half a bf16 ulp plus mx_dot's bound on
    the matrix cores' accumulation over I."""
    off = ref["offsets"]
    o, do = np.zeros((D.R, D.d)), np.zeros((D.R, D.d))
    for e in range(D.E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        wd = mx_round(p.host_expert("w_down", e))
        o[lo:hi], do[lo:hi] = mx_dot(h_dec[lo:hi], wd)
    over = np.abs(o_perm - o) - (2.0 ** -8 * np.maximum(np.abs(o_perm), np.abs(o)) + do)
    assert np.all(over <= 0), "o_perm off by %.3e beyond its bound at %s" % (
        over.max(), np.unravel_index(np.argmax(over), over.shape))


def quantized_expert_outputs(p, D, ref):
    """float64 expert outputs with every routed GEMM operand MX-rounded along
    its K axis (x and W_gate/W_up along d, h and W_down along I): the
    arithmetic the MXFP8 path performs, without its fp32 accumulation."""
    a = mx_round(p.host("x"))[ref["row_token"]]
    o = np.zeros((D.R, D.d))
    off = ref["offsets"]
    for e in range(D.E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        wg, wu, wd = (mx_round(p.host_expert(n, e)) for n in ("w_gate", "w_up", "w_down"))
        h = O.silu(a[lo:hi] @ wg.T) * (a[lo:hi] @ wu.T)
        o[lo:hi] = mx_round(h) @ wd.T
    return o


@pytest.mark.parametrize("name", list(SMALL))
def test_small_mxfp8_layer(name):
    check_mxfp8_layer(SMALL[name], strict=True)


def check_mxfp8_layer(D, strict):
    """One small MXFP8 layer: routing, the quantizing dispatch and the
    staged/fused equalities bit-exact; y within 3e-2 of the quantization-aware
    model; G, U, every h scale and code and o_perm element by element; the
    combine against a float64 sum.  strict: also the stated 6e-2 bound
    against the float64 oracle (an expected failure where the quantized
    operands alone exceed it)."""
    import mixture_experts_layer_prefix_amd as M
    name = D.name
    say("[case]", name, D)
    ref = HostProblem(D).oracle_forward()
    p, t, md, w = device_problem(D)
    wq = M.prepare_mxfp8(w, md)
    # quantizing dispatch: bit-exact against the oracle quantizer on gathered rows
    _, idx, tw = M.route(t["x"], t["w_router"], md, "mxfp8", bias=t["bias"])
    assert np.array_equal(to_np(idx), ref["topk_idx"])
    counts, offsets, row_token, token_row, xq, xs = M.permute(idx, t["x"], md, "mxfp8")
    rq, rs = O.mx_quantize(p.host("x")[ref["row_token"]], axis=-1)
    assert np.array_equal(to_np(xq), rq) and np.array_equal(to_np(xs), rs)
    # routed experts through the staged entry points
    h, hs = M.expert_gate_up(xq, xs, offsets, wq, md, "mxfp8")
    o_perm = M.expert_down(h, hs, offsets, wq, md, "mxfp8")
    e_o = rel_err(to_np(o_perm), ref["o_perm"])
    o_perm2 = M.expert_ffn(xq, xs, offsets, wq, md, "mxfp8")
    assert torch.equal(o_perm, o_perm2)
    # fused forward
    y, routing = M.layer_forward(t["x"], wq, md, "mxfp8", bias=t["bias"])
    e_y = rel_err(to_np(y), ref["y"])
    # Against the same arithmetic on MX-rounded operands (float64): only fp32
    # accumulation and h-quantization decisions at rounding boundaries differ.
    oq = quantized_expert_outputs(p, D, ref)
    yq = O.combine(oq, ref["token_row"], ref["topk_w"], ref["y_shared"])
    e_qo, e_qy = rel_err(to_np(o_perm), oq), rel_err(to_np(y), yq)
    say("   mxfp8 y vs exact %.3e (rms %.3e); vs MX-rounded operands: y %.3e, o_perm %.3e (o_perm vs exact %.3e)"
        % (e_y, rms_rel(to_np(y), ref["y"]), e_qy, e_qo, e_o))
    # o_perm is held element by element below: a max-norm bar on it fails where
    # one h code next to a rounding boundary legitimately went the other way
    # (a 128-term row moved by a fifth of an E4M3 step)
    assert e_qy <= 3e-2
    # a second run, keeping G | U: bitwise the same output
    y2, routing2 = M.layer_forward(t["x"], wq, md, "mxfp8", bias=t["bias"], keep_gu=True)
    assert torch.equal(y, y2)
    # element by element: G and U, every h scale and code, and o_perm against
    # the exact product of the kernel's own h, each within its derived bound
    h_dec, n_codes, n_scales = check_gate_up_elementwise(p, D, ref, to_np(routing2["gu"][:D.R]).astype(np.float64),
                                                         to_np(h), to_np(hs))
    check_down_elementwise(p, D, ref, h_dec, to_np(o_perm).astype(np.float64))
    say("   element-wise bounds hold; rounding decisions inside the fp32 band taken unlike float64: "
        "%d of %d h codes, %d of %d scales" % (n_codes, D.R * D.I, n_scales, D.R * D.I // 32))
    # the layer forward equals the staged entry points bit for bit (expert
    # FFNs, shared FFN, moe_combine)
    y_sh = M.shared_ffn(t["x"], wq, md, "mxfp8") if D.S else None
    y_st = M.combine(o_perm, token_row, tw, y_sh, md, "mxfp8")
    assert torch.equal(y, y_st), "moe_layer_forward differs from the staged entry points"
    # combine of the GPU's own expert outputs against a float64 weighted sum of them
    y_c_ref = O.combine(to_np(o_perm), ref["token_row"], to_np(tw), to_np(y_sh) if D.S else None)
    assert rel_err(to_np(y_st), y_c_ref) <= 4e-3
    # Against the exact layer: the stated 6e-2 bound (an expected failure
    # where MX rounding of the operands alone already exceeds it).
    if strict:
        check_mx_bound({"y": (e_y, rel_err(yq, ref["y"])), "o_perm": (e_o, rel_err(oq, ref["o_perm"]))}, name)


def test_expert_down_takes_quantizer_layout():
    """moe_expert_down reads h and h_scale in the layout of
    moe_quantize_mxfp8(axis 2) (scales slab-major [I/128][R][4]), the layout
    moe_expert_gate_up writes: a bf16 h from the generator quantized by that
    entry point gives the oracle's product of the dequantized operands to
    fp32-accumulation accuracy; and the h_scale written by
    moe_expert_gate_up, read in that layout, dequantizes h to within the
    MX rounding of the exact SwiGLU output."""
    import mixture_experts_layer_prefix_amd as M
    D = gen.Dims("mx_down_layout", 300, 256, 8, 2, 384, 0, 0, "mxfp8", 0.0)
    say("[case] h layout", D)
    ref = HostProblem(D).oracle_forward()
    p, t, md, w = device_problem(D)
    wq = M.prepare_mxfp8(w, md)
    off = torch.as_tensor(ref["offsets"], device="cuda")
    # h from the generator's dy stream ([T][d] reshaped to [R][I] rows)
    hb = gen.Problem(gen.Dims("hsrc", D.R, D.I, 1, 1, 128, 0, 0, "bf16", 0.0)).device("dy")
    hq, hs = M.quantize_mxfp8(hb, 2)
    o = M.expert_down(hq, hs, off, wq, md, "mxfp8")
    h_host = gen.Problem(gen.Dims("hsrc", D.R, D.I, 1, 1, 128, 0, 0, "bf16", 0.0)).host("dy")
    hd = mx_round(h_host)
    want = np.zeros((D.R, D.d))
    for e in range(D.E):
        lo, hi = ref["offsets"][e], ref["offsets"][e + 1]
        want[lo:hi] = hd[lo:hi] @ mx_round(p.host_expert("w_down", e)).T
    e_o = rel_err(to_np(o), want)
    say("   down of quantizer-made h: %.3e" % e_o)
    assert e_o <= 1e-2   # bf16 output rounding (2^-9) and fp32 accumulation only
    # the gate/up epilogue's h and scales decode, in that layout, to the exact
    # SwiGLU output within MX rounding
    counts, offsets, row_token, token_row, xq, xs = M.permute(torch.as_tensor(ref["topk_idx"], device="cuda"),
                                                              t["x"], md, "mxfp8")
    h, h_scale = M.expert_gate_up(xq, xs, offsets, wq, md, "mxfp8")
    assert tuple(h_scale.shape) == (D.I // 128, D.R, 4)
    sc = to_np(h_scale).transpose(1, 0, 2).reshape(D.R, D.I // 32)
    h_dec = O.mx_dequantize(to_np(h), sc, axis=-1)
    a = p.host("x")[ref["row_token"]]
    h_exact = np.zeros((D.R, D.I))
    for e in range(D.E):
        lo, hi = ref["offsets"][e], ref["offsets"][e + 1]
        h_exact[lo:hi] = O.swiglu_ffn(a[lo:hi], *(p.host_expert(n, e) for n in ("w_gate", "w_up", "w_down")))[3]
    e_h = rel_err(h_dec, h_exact)
    say("   gate/up h decoded slab-major vs exact SwiGLU: %.3e" % e_h)
    assert e_h <= 1e-1   # three MX roundings (x, weights, h); a wrong layout gives O(1)


