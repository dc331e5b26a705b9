"""Determinism regardless of how the work is scheduled (blog post,
"Determinism": the floating-point order is fixed, so results are bitwise
reproducible): the whole layer, forward and backward, gives the same bits
whether the persistent GEMM grids span every compute unit or are capped at
64 or 16 workgroups (moe_set_max_workgroups), which changes which workgroup
runs each tile and the order tiles are taken in."""
import pytest

import gen
from tests.moe_parity import device_problem

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "det_bf16": gen.Dims("det_bf16", 2100, 512, 16, 4, 320, 1, 192, "bf16", 1.2, backward=True),
    "det_mxfp8": gen.Dims("det_mxfp8", 2100, 512, 16, 4, 384, 1, 256, "mxfp8", 1.2, backward=True),
}


def say(*a):
    print(*a, flush=True)


def run_layer(D, p, t, md, w, dy):
    import mixture_experts_layer_prefix_amd as M
    y, routing = M.layer_forward(t["x"], w, md, D.prec, bias=t["bias"], keep_gu=True)
    dx, grads = M.layer_backward(dy, t["x"], w, routing, md, D.prec)
    torch.cuda.synchronize()
    out = {"y": y.clone(), "dx": dx.clone()}
    out.update({n: v.clone() for n, v in grads.items()})
    out.update({n: routing[n].clone() for n in ("topk_idx", "topk_w", "row_token")})
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_bitwise_identical_across_grid_sizes(name):
    import mixture_experts_layer_prefix_amd as M
    from mixture_experts_layer_prefix_amd import _lib as L
    D = CASES[name]
    say("[case]", name, D)
    p, t, md, w = device_problem(D)
    if D.prec == "mxfp8":
        w = M.prepare_mxfp8(w, md)
    w = M.prepare_backward(w, mxfp8=D.prec == "mxfp8")
    dy = p.device("dy")
    try:
        ref = run_layer(D, p, t, md, w, dy)
        for cap in (64, 16):
            L.call("moe_set_max_workgroups", cap)
            got = run_layer(D, p, t, md, w, dy)
            for n, v in ref.items():
                assert torch.equal(got[n], v), "%s differs with the grid capped at %d workgroups" % (n, cap)
            say("   grid capped at %d workgroups: every output bitwise equal" % cap)
    finally:
        L.call("moe_set_max_workgroups", 0)
