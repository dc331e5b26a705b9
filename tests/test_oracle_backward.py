"""Pins of the oracle's backward: central finite differences in float64 with
the routing held fixed, a torch.autograd cross-check of the whole chain
(router included, selection held fixed), the router-weight-gradient identity
and exact zeros for experts that receive no tokens."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O


def make(rng, T=6, d=8, E=4, k=2, I=5, S=1, Is=4):
    x = rng.standard_normal((T, d))
    ws = dict(
        wr=rng.standard_normal((E, d)) / np.sqrt(d),
        wg=rng.standard_normal((E, I, d)) / np.sqrt(d), wu=rng.standard_normal((E, I, d)) / np.sqrt(d),
        wd=rng.standard_normal((E, d, I)) / np.sqrt(I),
        sg=rng.standard_normal((S, Is, d)) / np.sqrt(d), su=rng.standard_normal((S, Is, d)) / np.sqrt(d),
        sd=rng.standard_normal((S, d, Is)) / np.sqrt(Is))
    dy = rng.standard_normal((T, d))
    return x, ws, dy, k


def fixed_routing_loss(x, w, dy, fw):
    """<dy, y> with the oracle's routing (ids, weights, rows) held fixed."""
    a = O.permute(x, fw["row_token"])
    o = np.zeros_like(a)
    off = fw["offsets"]
    for e in range(len(w["wg"])):
        if off[e + 1] > off[e]:
            o[off[e]:off[e + 1]] = O.swiglu_ffn(a[off[e]:off[e + 1]], w["wg"][e], w["wu"][e], w["wd"][e])[0]
    y = O.combine(o, fw["token_row"], fw["topk_w"], O.shared_ffn(x, w["sg"], w["su"], w["sd"]))
    return float(np.sum(y * dy))


def test_finite_differences_fixed_routing():
    rng = np.random.default_rng(12)
    x, w, dy, k = make(rng)
    out = O.layer_backward(x, w["wr"], None, w["wg"], w["wu"], w["wd"], w["sg"], w["su"], w["sd"], k, dy,
                           with_router=False)
    fw = out["fw"]
    h = 1e-6

    def fd(arr, idx, f):
        old = arr[idx]
        arr[idx] = old + h
        lp = f()
        arr[idx] = old - h
        lm = f()
        arr[idx] = old
        return (lp - lm) / (2 * h)

    loss = lambda: fixed_routing_loss(x, w, dy, fw)
    pts = [(0, 0), (3, 5), (5, 7)]
    for p in pts:
        assert abs(fd(x, p, loss) - out["dx"][p]) < 1e-7 * max(1, abs(out["dx"][p]))
    for name, key in [("wg", "dw_gate"), ("wu", "dw_up"), ("wd", "dw_down"), ("sg", "dws_gate"),
                      ("su", "dws_up"), ("sd", "dws_down")]:
        arr = w[name]
        for flat in (0, arr.size // 2, arr.size - 1):
            p = np.unravel_index(flat, arr.shape)
            assert abs(fd(arr, p, loss) - out[key][p]) < 1e-7 * max(1, abs(out[key][p])), (name, p)
    # router-weight gradient: derivative of the loss in each weight g[t][j]
    g = fw["topk_w"].astype(np.float64)
    fw64 = dict(fw, topk_w=g)
    for t, j in [(0, 0), (2, 1), (5, 0)]:
        lossg = lambda: fixed_routing_loss(x, w, dy, fw64)
        assert abs(fd(g, (t, j), lossg) - out["dtopk_w"][t, j]) < 1e-7


def test_router_weight_gradient_identity():
    rng = np.random.default_rng(13)
    x, w, dy, k = make(rng, T=10, E=5, k=3)
    out = O.layer_backward(x, w["wr"], None, w["wg"], w["wu"], w["wd"], w["sg"], w["su"], w["sd"], k, dy)
    fw = out["fw"]
    # dg = <dY_t, O_row> (output side) equals <h, dY_t W_d> (computed inside)
    via_o = np.einsum("tkd,td->tk", fw["o_perm"][fw["token_row"]], dy)
    assert np.allclose(out["dtopk_w"], via_o, rtol=1e-12, atol=1e-12)


def test_torch_autograd_cross_check():
    rng = np.random.default_rng(14)
    x, w, dy, k = make(rng, T=7, d=8, E=5, k=2, I=6, S=1, Is=3)
    out = O.layer_backward(x, w["wr"], None, w["wg"], w["wu"], w["wd"], w["sg"], w["su"], w["sd"], k, dy)
    idx = torch.from_numpy(out["fw"]["topk_idx"].astype(np.int64))
    tt = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True) for n, v in w.items()}
    xt = torch.tensor(x, requires_grad=True)
    logits = xt @ tt["wr"].T
    g = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    g.retain_grad()
    y = torch.zeros_like(xt)
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(idx[t, j])
            hh = F.silu(xt[t] @ tt["wg"][e].T) * (xt[t] @ tt["wu"][e].T)
            y[t] = y[t] + g[t, j] * (hh @ tt["wd"][e].T)
    for s in range(len(w["sg"])):
        y = y + (F.silu(xt @ tt["sg"][s].T) * (xt @ tt["su"][s].T)) @ tt["sd"][s].T
    (y * torch.from_numpy(dy)).sum().backward()
    # oracle weights are rounded to fp32: allow for that in the comparison
    tol = dict(rtol=2e-6, atol=2e-6)
    assert np.allclose(out["dx"], xt.grad.numpy(), **tol)
    for n, key in [("wg", "dw_gate"), ("wu", "dw_up"), ("wd", "dw_down"), ("sg", "dws_gate"),
                   ("su", "dws_up"), ("sd", "dws_down"), ("wr", "dw_router")]:
        assert np.allclose(out[key], tt[n].grad.numpy(), **tol), key
    assert np.allclose(out["dtopk_w"], g.grad.numpy(), **tol)


def test_empty_experts_get_exact_zero_gradients():
    rng = np.random.default_rng(15)
    x, w, dy, k = make(rng, T=8, E=6, k=1)
    bias = np.array([0, 0, -100, 0, -100, -100], dtype=np.float32)
    out = O.layer_backward(x, w["wr"], bias, w["wg"], w["wu"], w["wd"], w["sg"], w["su"], w["sd"], k, dy)
    for e in (2, 4, 5):
        assert out["fw"]["counts"][e] == 0
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(out[key][e] == 0.0)
    assert np.all(out["dw_router"][[2, 4, 5]] == 0.0)
