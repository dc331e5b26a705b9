"""Pins of the oracle's router: projection rounding, top-k with its tie rule,
and the normalized weights."""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(row, k):
    """The unique k-subset whose every member beats every non-member under
    (larger logit, then smaller id)."""
    E = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    winners = [s for s in itertools.combinations(range(E), k)
               if all(beats(a, b) for a in s for b in range(E) if b not in s)]
    assert len(winners) == 1
    return list(winners[0])


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for E, k in [(4, 1), (5, 2), (6, 3), (8, 2), (8, 8), (7, 6)]:
        logits = rng.integers(-2, 3, size=(40, E)).astype(np.float32)  # many ties
        got = O.topk_route(logits, k)
        for t in range(40):
            assert list(got[t]) == brute_topk(logits[t], k)


def test_topk_matches_torch_topk_without_ties():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((500, 64)).astype(np.float32)
    ref = torch.topk(torch.from_numpy(logits), 6, dim=1).indices.sort(dim=1).values.numpy()
    assert np.array_equal(O.topk_route(logits, 6), ref)


def test_golden_router_example():
    g = json.load(open(os.path.join(GOLD, "router_example.json")))
    logits = np.array(g["logits"], dtype=np.float32)
    idx = O.topk_route(logits, g["k"])
    assert idx.tolist() == g["topk_idx"]
    w = O.renormalized_weights(logits, idx)
    assert np.allclose(w, np.array(g["topk_w"], dtype=np.float32), rtol=0, atol=1e-7)


def test_weights_invariants():
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((300, 32)) * 3).astype(np.float32)
    for k in (1, 2, 8, 32):
        idx = O.topk_route(logits, k)
        w = O.renormalized_weights(logits, idx)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 4 * np.finfo(np.float32).eps)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 32:  # every expert selected: the full softmax
            ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
            assert np.allclose(w, ref, rtol=1e-6, atol=0)
    # shift invariance of the restricted softmax (logits on a 2^-10 grid so
    # the fp32 shift is exact)
    q = (np.round(logits * 1024) / 1024).astype(np.float32)
    idx = O.topk_route(q, 4)
    assert np.allclose(O.renormalized_weights(q + np.float32(8.0), idx),
                       O.renormalized_weights(q, idx), rtol=2.5e-7, atol=0)


def test_logits_round_once_then_add_bias_in_fp32():
    # x . w = 2^24 + 1 exactly: rounds (ties to even) to 2^24 in fp32; adding
    # a bias of 1 in fp32 ties back to 2^24.  Adding the bias before rounding
    # would give 2^24 + 2.
    x = np.array([[2.0 ** 24, 1.0]])
    w = np.array([[1.0, 1.0], [1.0, 0.0]])
    lg = O.router_logits(x, w)
    assert lg.dtype == np.float32 and lg[0, 0] == np.float32(2 ** 24)
    lb = O.router_logits(x, w, bias=np.array([1.0, 0.0], dtype=np.float32))
    assert lb[0, 0] == np.float32(2 ** 24)
    # and the dot product itself is exact before the single rounding
    x2 = np.array([[1.0, 2.0 ** -30, -1.0]])
    assert O.router_logits(x2, np.ones((1, 3)))[0, 0] == np.float32(2.0 ** -30)
