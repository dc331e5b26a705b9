"""Token granularity of the layer calls, through the C ABI (one GPU's reading
of the blog post's granularity study, where a batch is processed in chunks of
512 to 32,768 tokens).

A layer call over T tokens and calls over consecutive chunks of those tokens
must give the same per-token results bit for bit: the logits, the selected
experts and their weights, the output y, dX and dL/dg.  Every one of them
depends only on the token's own rows: the router and expert GEMMs accumulate
each output row over K in an order that does not depend on the other rows of
its tile, the MX quantization of tokens, h, dY, dG and dU runs along each row,
and the weighted sums run over the token's own experts in ascending order.
The weight gradients of a call cover its own tokens; summed over the chunks
they match the whole call's within bf16 rounding of each chunk's result (bf16;
the MXFP8 weight-gradient operands are quantized in 32-row blocks of one
expert's rows, which chunking regroups, so only the per-token results are
compared there).  The forward with G|U kept and the backward's replay of them
are compared bitwise in the backward tests."""
import pytest

import gen
from tests.moe_parity import device_problem, rel_err, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    # ragged last chunk; Zipf-skewed routing leaves some experts empty in a chunk
    "n2_bf16": (gen.Dims("n2_bf16", 1100, 512, 16, 4, 320, 1, 192, "bf16", 1.2, backward=True), (512, 512, 76)),
    "n2_mxfp8": (gen.Dims("n2_mxfp8", 1100, 512, 16, 4, 384, 1, 192, "mxfp8", 1.2, backward=True), (256, 768, 76)),
    "n2_mxfp8_noshared_k1": (gen.Dims("n2_mxfp8_k1", 600, 256, 8, 1, 256, 0, 0, "mxfp8", 0.0, backward=True),
                             (1, 64, 535)),
}

PER_TOKEN = ("logits", "topk_idx", "topk_w")


def say(*a):
    print(*a, flush=True)


def layer_call(D, fw, bw, x, dy, bias, T):
    import mixture_experts_layer_prefix_amd as M
    md = M.Dims(T, D.d, D.E, D.k, D.I, D.S, D.Is)
    f = M.ForwardPlan(md, D.prec, keep_gu=True)
    y = f.run(x, fw, bias).clone()
    b = M.BackwardPlan(md, D.prec)
    dx, grads = b.run(dy, x, bw, f.routing)
    torch.cuda.synchronize()
    return (y, {n: f.routing[n].clone() for n in PER_TOKEN}, dx.clone(),
            {n: v.clone() for n, v in grads.items()})


@pytest.mark.parametrize("name", list(CASES))
def test_chunked_calls_match_whole_call(name):
    import mixture_experts_layer_prefix_amd as M
    D, sizes = CASES[name]
    assert sum(sizes) == D.T
    say("[case]", name, D, "chunks", sizes)
    p, t, md, w = device_problem(D)
    x, dy, bias = t["x"], p.device("dy"), t["bias"]
    if D.prec == "mxfp8":
        fw = M.prepare_mxfp8(w, md)
        bw = M.prepare_backward(fw, mxfp8=True)
    else:
        fw = w
        bw = M.prepare_backward(w)
    y, rt, dx, grads = layer_call(D, fw, bw, x, dy, bias, D.T)
    parts, t0 = [], 0
    for c in sizes:
        parts.append(layer_call(D, fw, bw, x[t0:t0 + c], dy[t0:t0 + c], bias, c))
        t0 += c
    assert torch.equal(torch.cat([q[0] for q in parts]), y)
    for n in PER_TOKEN:
        assert torch.equal(torch.cat([q[1][n] for q in parts]), rt[n]), n
    assert torch.equal(torch.cat([q[2] for q in parts]), dx)
    assert torch.equal(torch.cat([q[3]["dtopk_w"] for q in parts]), grads["dtopk_w"])
    say("   per-token results of %d chunked calls bit-identical to the whole call" % len(sizes))
    if D.prec != "bf16":
        return
    for n, v in grads.items():
        if n == "dtopk_w":
            continue
        tot = sum(q[3][n].float() for q in parts)
        e = rel_err(to_np(tot), to_np(v.float()))
        say("   %s: chunk sum vs whole %.2e" % (n, e))
        assert e <= (1e-4 if n == "dw_router" else 1e-2), (n, e)
