"""Pins of the oracle's schedule (counting sort) and permutation."""
import json
import os

import numpy as np

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_schedule_example():
    g = json.load(open(os.path.join(GOLD, "schedule_example.json")))
    c, off, rt, tr = O.schedule(np.array(g["topk_idx"]), g["E"])
    assert c.tolist() == g["counts"] and off.tolist() == g["offsets"]
    assert rt.tolist() == g["row_token"] and tr.tolist() == g["token_row"]


def test_schedule_invariants_and_stable_sort():
    rng = np.random.default_rng(4)
    for T, E, k in [(1, 1, 1), (37, 5, 2), (200, 16, 4), (64, 8, 8)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        idx = O.topk_route(logits, k)
        c, off, rt, tr = O.schedule(idx, E)
        assert c.sum() == T * k and off[0] == 0 and np.array_equal(np.diff(off), c)
        # library stable sort of the routes by (expert, token)
        routes = sorted(((int(idx[t, j]), t, j) for t in range(T) for j in range(k)))
        assert rt.tolist() == [t for (_, t, _) in routes]
        for r, (e, t, j) in enumerate(routes):
            assert tr[t, j] == r and off[e] <= r < off[e + 1]
        for e in range(E):
            assert np.all(np.diff(rt[off[e]:off[e + 1]]) > 0)


def test_permute_round_trip_is_exact():
    rng = np.random.default_rng(5)
    T, E, k, d = 50, 6, 3, 7
    x = rng.standard_normal((T, d))
    idx = O.topk_route(rng.standard_normal((T, E)).astype(np.float32), k)
    _, _, rt, tr = O.schedule(idx, E)
    xp = O.permute(x, rt)
    for j in range(k):
        assert np.array_equal(xp[tr[:, j]], x)
