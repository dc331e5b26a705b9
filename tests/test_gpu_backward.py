"""GPU parity of the layer backward (bf16) against the oracle, through the C
ABI: dx (with and without the router chain), the router-weight gradients
dL/dg, every routed and shared weight gradient and the router weight
gradient.  Bars: max|d|/max|ref| <= 2e-2 per tensor; experts without rows
get exact zero gradients; repeated runs are bitwise identical.

Small shapes are checked in full against the oracle's layer backward; the
DeepSeek-V3-shaped layer on sampled tokens (dx, dg), on the router weight
gradient rows of two ragged experts, and on sampled intermediate columns of
every expert's weight gradients (every row of each expert) and of the shared
expert's, each sample exact per-element math."""
import numpy as np
import pytest

import gen
from oracle import moe_oracle as O
from tests.moe_parity import (TOL, HostProblem, device_problem, expert_wgrad_columns, rel_err, rms_rel,
                              sampled_backward, shared_weights, to_np)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SMALL = {
    "bwd_ragged": gen.Dims("bwd_ragged", 300, 256, 16, 4, 192, 1, 128, "bf16", 0.0, backward=True),
    "bwd_skew_noshared": gen.Dims("bwd_skew_noshared", 513, 192, 32, 8, 128, 0, 0, "bf16", 1.2, backward=True),
    "bwd_k1": gen.Dims("bwd_k1", 77, 64, 4, 1, 64, 1, 64, "bf16", 0.0, backward=True),
    "bwd_kE": gen.Dims("bwd_kE", 64, 128, 8, 8, 64, 1, 64, "bf16", 0.0, backward=True),
    "bwd_E1": gen.Dims("bwd_E1", 130, 128, 1, 1, 64, 0, 0, "bf16", 0.0, backward=True),
    "bwd_tiles": gen.Dims("bwd_tiles", 1100, 512, 8, 2, 320, 1, 192, "bf16", 0.0, backward=True),
    # the ABI's limits: E = 1024 experts, k = 16
    "bwd_max_E_k": gen.Dims("bwd_max_E_k", 300, 128, 1024, 16, 64, 1, 64, "bf16", 1.2, backward=True),
    "bwd_one_token": gen.Dims("bwd_one_token", 1, 256, 16, 4, 192, 1, 128, "bf16", 0.0, backward=True),
}


def say(*a):
    print(*a, flush=True)


def forward_and_backward(D, router_grad=True):
    import mixture_experts_layer_prefix_amd as M
    p, t, md, w = device_problem(D)
    dy = p.device("dy")
    wb = M.prepare_backward(w)
    _, routing = M.layer_forward(t["x"], w, md, D.prec, bias=t["bias"])
    dx, grads = M.layer_backward(dy, t["x"], wb, routing, md, D.prec, router_grad=router_grad)
    torch.cuda.synchronize()
    return p, t, md, wb, dy, routing, dx, grads


def test_transpose_weights_exact():
    import mixture_experts_layer_prefix_amd as M
    g = torch.Generator().manual_seed(0)
    for shape in ((3, 64, 128), (2, 100, 37), (1, 1, 5)):
        a = torch.randn(shape, generator=g).to(torch.bfloat16).cuda()
        assert torch.equal(M.transpose_weights(a), a.transpose(1, 2).contiguous())


@pytest.mark.parametrize("name", list(SMALL))
def test_small_backward_full(name):
    D = SMALL[name]
    say("[case]", name, D)
    hp = HostProblem(D)
    a = hp.full()
    dy_h = hp.p.host("dy")
    ref = O.layer_backward(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"], a["w_down"], a["ws_gate"],
                           a["ws_up"], a["ws_down"], D.k, dy_h, with_router=True)
    p, t, md, wb, dy, routing, dx, grads = forward_and_backward(D)
    fw = ref["fw"]
    assert np.array_equal(to_np(routing["topk_idx"]), fw["topk_idx"])
    errs = {}
    pairs = [("dx", dx, ref["dx"]), ("dtopk_w", grads["dtopk_w"], ref["dtopk_w"]),
             ("dw_gate", grads["dw_gate"], ref["dw_gate"]), ("dw_up", grads["dw_up"], ref["dw_up"]),
             ("dw_down", grads["dw_down"], ref["dw_down"]), ("dw_router", grads["dw_router"], ref["dw_router"])]
    if D.S:
        pairs += [("dws_gate", grads["dws_gate"], ref["dws_gate"]), ("dws_up", grads["dws_up"], ref["dws_up"]),
                  ("dws_down", grads["dws_down"], ref["dws_down"])]
    for n, got, want in pairs:
        errs[n] = rel_err(to_np(got), want)
    say("   rel err " + ", ".join("%s %.2e" % kv for kv in errs.items()))
    say("   rms dx %.2e dw_gate %.2e" % (rms_rel(to_np(dx), ref["dx"]), rms_rel(to_np(grads["dw_gate"]),
                                                                                 ref["dw_gate"])))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
    # experts without rows: exact zeros
    empty = np.nonzero(fw["counts"] == 0)[0]
    if len(empty):
        sel = torch.as_tensor(empty, dtype=torch.long, device=dx.device)
        for n in ("dw_gate", "dw_up", "dw_down"):
            assert torch.count_nonzero(grads[n][sel]) == 0, n
    # without the router chain: dx lacks the router term, the rest is unchanged
    ref_nr = O.layer_backward(a["x"], a["w_router"], a["bias"], a["w_gate"], a["w_up"], a["w_down"], a["ws_gate"],
                              a["ws_up"], a["ws_down"], D.k, dy_h, with_router=False)
    import mixture_experts_layer_prefix_amd as M
    dx2, grads2 = M.layer_backward(dy, t["x"], wb, routing, md, D.prec, router_grad=False)
    e_nr = rel_err(to_np(dx2), ref_nr["dx"])
    say("   dx without router chain %.2e" % e_nr)
    assert e_nr <= TOL["bf16"]
    assert torch.equal(grads2["dw_gate"], grads["dw_gate"]) and torch.equal(grads2["dtopk_w"], grads["dtopk_w"])
    # determinism
    dx3, grads3 = M.layer_backward(dy, t["x"], wb, routing, md, D.prec, router_grad=True)
    assert torch.equal(dx3, dx)
    for n in grads:
        assert torch.equal(grads3[n], grads[n]), n
    # G | U kept by the forward: the same bits as the backward's own replay
    _, routing4 = M.layer_forward(t["x"], wb, md, D.prec, bias=t["bias"], keep_gu=True)
    assert "gu" in routing4
    dx4, grads4 = M.layer_backward(dy, t["x"], wb, routing4, md, D.prec, router_grad=True)
    assert torch.equal(dx4, dx)
    for n in grads:
        assert torch.equal(grads4[n], grads[n]), n


def test_backward_no_tokens():
    import mixture_experts_layer_prefix_amd as M
    D = gen.Dims("bwd_empty", 0, 128, 8, 2, 64, 1, 64, "bf16", 0.0)
    p, t, md, w = device_problem(D)
    wb = M.prepare_backward(w)
    routing = dict(topk_idx=torch.empty(0, 2, dtype=torch.int32, device="cuda"),
                   topk_w=torch.empty(0, 2, device="cuda"),
                   expert_counts=torch.zeros(8, dtype=torch.int32, device="cuda"),
                   expert_offsets=torch.zeros(9, dtype=torch.int32, device="cuda"),
                   row_token=torch.empty(1, dtype=torch.int32, device="cuda"),
                   token_row=torch.empty(0, 2, dtype=torch.int32, device="cuda"))
    plan = M.BackwardPlan(md, "bf16")
    for v in plan.grads.values():
        v.fill_(1.0)
    dx, grads = plan.run(t["x"], t["x"], wb, routing)
    torch.cuda.synchronize()
    for n, v in grads.items():
        if v.numel():
            assert torch.count_nonzero(v) == 0, n


def test_dsv3_backward_sampled():
    """DeepSeek-V3-shaped bf16 backward (T=8192, Zipf-skewed routing)."""
    check_backward_sampled(gen.get_config("c3a"))


def check_backward_sampled(D, ntok=128, seed=11):
    """Two backward runs bitwise equal; dx and dL/dg of ntok seeded tokens
    plus every token of the smallest non-empty expert and of one expert with
    64 to 256 rows; the router weight gradient rows of those experts; the
    weight gradients of every non-empty expert on 16 seeded intermediate
    columns each (all of the expert's rows), one error per tensor; the shared
    expert's weight gradients on sampled columns (all tokens).  Each sample is
    exact per-element oracle math."""
    import mixture_experts_layer_prefix_amd as M
    from tests.moe_parity import gather_wgrad, pick_tokens, router_wgrad_rows, sampled_eval, wgrad_columns
    say("[case] %s backward sampled" % D.name, D)
    p, t, md, wb, dy, routing, dx, grads = forward_and_backward(D)
    dx2, grads2 = M.layer_backward(dy, t["x"], wb, routing, md, D.prec, router_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx)
    for n in grads:
        assert torch.equal(grads2[n], grads[n]), n
    del dx2, grads2
    hp = HostProblem(D)
    ref_rt = hp.routing()
    idx, g = ref_rt["topk_idx"], ref_rt["topk_w"]
    assert np.array_equal(to_np(routing["topk_idx"]), idx)
    tokens, experts = pick_tokens(ref_rt, D.T, ntok, seed)
    res = sampled_eval(hp, tokens, idx, g, backward=True)
    tk = torch.as_tensor(tokens, device=dx.device)
    errs = {"dx": rel_err(to_np(dx[tk]), res["dx"]), "dtopk_w": rel_err(to_np(grads["dtopk_w"][tk]), res["dg"])}
    ex = router_wgrad_rows(hp, experts, tokens, idx, res["dl"])
    errs["dw_router"] = rel_err(to_np(grads["dw_router"][torch.as_tensor(experts, device=dx.device)]), ex)
    samples = wgrad_columns(hp, ref_rt, 16, seed)
    gw = gather_wgrad(grads, samples)
    for n, lst in samples.items():
        errs[n] = rel_err(gw[n], np.concatenate([v[2].ravel() for v in lst]))
        per = []
        for e, cols, ev, _ in lst:
            c = torch.as_tensor(cols, device=dx.device)
            gv = to_np(grads[n][e][:, c] if n == "dw_down" else grads[n][e][c])
            per.append((rel_err(gv, ev), e, int(ref_rt["counts"][e])))
        say("   %s worst expert: %.3e (expert %d, %d rows)" % ((n,) + max(per)))
    counts = ref_rt["counts"]
    empty = np.nonzero(counts == 0)[0]
    if len(empty):
        sel = torch.as_tensor(empty, device=dx.device)
        for n in ("dw_gate", "dw_up", "dw_down"):
            assert torch.count_nonzero(grads[n][sel]) == 0, n
    if D.S:
        # shared-expert weight gradients on sampled intermediate columns (all tokens)
        rng = np.random.default_rng(seed + 1)
        cols = np.sort(rng.choice(D.Is, size=4, replace=False))
        wg, wu, wd = shared_weights(hp.p, D)
        _, dWg, dWu, dWd, _, _ = O.ffn_backward(hp.p.host("x"), wg[cols], wu[cols], wd[:, cols], hp.p.host("dy"))
        c = torch.as_tensor(cols, device=dx.device)
        errs["dws_gate"] = rel_err(to_np(grads["dws_gate"][0][c]), dWg)
        errs["dws_up"] = rel_err(to_np(grads["dws_up"][0][c]), dWu)
        errs["dws_down"] = rel_err(to_np(grads["dws_down"][0][:, c]), dWd)
    say("   %d sampled tokens (experts %s with %s rows): %s" % (
        len(tokens), experts, [int(counts[e]) for e in experts], ", ".join("%s %.2e" % kv for kv in errs.items())))
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
