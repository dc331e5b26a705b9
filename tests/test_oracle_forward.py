"""Pins of the oracle's layer forward: a hand-worked example, a brute-force
dense evaluation (every token through every expert, masked by its routing),
and special cases that reduce to library routines."""
import json
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, T, d, E, k, I, S, Is):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / np.sqrt(d)
    wg = rng.standard_normal((E, I, d)) / np.sqrt(d)
    wu = rng.standard_normal((E, I, d)) / np.sqrt(d)
    wd = rng.standard_normal((E, d, I)) / np.sqrt(I)
    sg = rng.standard_normal((S, Is, d)) / np.sqrt(d)
    su = rng.standard_normal((S, Is, d)) / np.sqrt(d)
    sd = rng.standard_normal((S, d, Is)) / np.sqrt(Is)
    return x, wr, wg, wu, wd, sg, su, sd


def torch_swiglu(a, wg, wu, wd):
    a, wg, wu, wd = (torch.from_numpy(np.asarray(v, np.float64)) for v in (a, wg, wu, wd))
    return (F.silu(F.linear(a, wg)) * F.linear(a, wu)) @ wd.T


def test_golden_layer_example():
    g = json.load(open(os.path.join(GOLD, "layer_example.json")))
    a = {k: np.array(v, dtype=np.float64) for k, v in g.items() if isinstance(v, list)}
    out = O.layer_forward(a["x"], a["w_router"], None, a["w_gate"], a["w_up"], a["w_down"],
                          a["ws_gate"], a["ws_up"], a["ws_down"], g["k"])
    assert np.allclose(out["y"], a["y"], rtol=1e-15, atol=0)


def test_silu_matches_torch():
    z = np.linspace(-60, 60, 2001)
    assert np.allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)
    g = torch.from_numpy(z).requires_grad_()
    F.silu(g).sum().backward()
    assert np.allclose(O.silu_grad(z), g.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_dense_masked_brute_force():
    """y_t = sum_e mask_te * g_te * FFN_e(x_t) + shared, every expert on every token."""
    rng = np.random.default_rng(6)
    for (T, d, E, k, I, S) in [(16, 8, 4, 2, 6, 1), (33, 12, 7, 3, 5, 0), (20, 8, 5, 5, 4, 2)]:
        x, wr, wg, wu, wd, sg, su, sd = rand_layer(rng, T, d, E, k, I, S, 6)
        out = O.layer_forward(x, wr, None, wg, wu, wd, sg, su, sd, k)
        lg = out["logits"].astype(np.float64)
        y = np.zeros((T, d))
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
            z = np.exp(lg[t, order] - lg[t, order].max())
            gw = dict(zip(order, (z / z.sum()).astype(np.float32).astype(np.float64)))  # stored fp32
            for e in range(E):
                mask = gw.get(e, 0.0)
                y[t] += mask * torch_swiglu(x[t:t + 1], wg[e], wu[e], wd[e]).numpy()[0]
            for s in range(S):
                y[t] += torch_swiglu(x[t:t + 1], sg[s], su[s], sd[s]).numpy()[0]
        assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-12)
        # per-token path used for large workloads agrees with the full layer
        ew = lambda e: (wg[e], wu[e], wd[e])
        for t in (0, T - 1):
            yt = O.token_forward(x[t], out["topk_idx"][t], out["topk_w"][t], ew, list(zip(sg, su, sd)))
            assert np.allclose(yt, out["y"][t], rtol=1e-6, atol=1e-6)


def test_single_expert_is_plain_swiglu():
    rng = np.random.default_rng(7)
    x, wr, wg, wu, wd, sg, su, sd = rand_layer(rng, 10, 8, 1, 1, 5, 0, 1)
    out = O.layer_forward(x, wr, None, wg, wu, wd, sg, su, sd, 1)
    assert np.allclose(out["y"], torch_swiglu(x, wg[0], wu[0], wd[0]).numpy(), rtol=1e-13, atol=1e-13)


def test_gate_takes_the_silu():
    # gate and up differ: only SiLU(gate) * up matches
    rng = np.random.default_rng(8)
    a = rng.standard_normal((4, 6))
    wg, wu, wd = rng.standard_normal((3, 6)), rng.standard_normal((3, 6)), rng.standard_normal((6, 3))
    got = O.swiglu_ffn(a, wg, wu, wd)[0]
    assert np.allclose(got, torch_swiglu(a, wg, wu, wd).numpy(), rtol=1e-13)
    assert not np.allclose(got, torch_swiglu(a, wu, wg, wd).numpy(), rtol=1e-3)


def test_all_experts_selected_is_full_softmax_mixture():
    rng = np.random.default_rng(9)
    T, d, E, I = 12, 8, 4, 5
    x, wr, wg, wu, wd, sg, su, sd = rand_layer(rng, T, d, E, E, I, 0, 1)
    out = O.layer_forward(x, wr, None, wg, wu, wd, sg, su, sd, E)
    p = scipy.special.softmax(x @ wr.T, axis=1)
    y = sum(p[:, e:e + 1] * torch_swiglu(x, wg[e], wu[e], wd[e]).numpy() for e in range(E))
    assert np.allclose(out["y"], y, rtol=1e-6, atol=1e-7)  # logits rounded to fp32


def test_zero_down_projection_leaves_shared_expert():
    rng = np.random.default_rng(10)
    x, wr, wg, wu, wd, sg, su, sd = rand_layer(rng, 9, 8, 4, 2, 5, 1, 7)
    out = O.layer_forward(x, wr, None, wg, wu, np.zeros_like(wd), sg, su, sd, 2)
    assert np.array_equal(out["y"], torch_swiglu(x, sg[0], su[0], sd[0]).numpy()) or \
        np.allclose(out["y"], torch_swiglu(x, sg[0], su[0], sd[0]).numpy(), rtol=1e-14, atol=0)
    assert np.all(out["o_perm"] == 0)


def test_bias_changes_selection_and_weights():
    # the logit bias enters both the selection and the softmax
    x = np.array([[1.0, 0.0]])
    wr = np.array([[1.0, 0.0], [0.5, 0.0], [0.0, 0.0]])
    b = np.array([0.0, 0.0, 2.0], dtype=np.float32)
    lg = O.router_logits(x, wr, b)
    idx = O.topk_route(lg, 2)
    assert idx.tolist() == [[0, 2]]
    w = O.renormalized_weights(lg, idx)
    assert np.allclose(w, [[1 / (1 + np.e), np.e / (1 + np.e)]], rtol=1e-7)
