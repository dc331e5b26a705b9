"""Seeded random small layer shapes through the small-shape parity checks:
bf16 forward (every entry point) and backward in full, fp32 forward, and the
MXFP8 forward (bit-exact routing and quantizing dispatch, element-wise G, U,
h and o_perm bounds); ragged token counts (1 to 700), 1 to 130 experts, k up
to 16, with and without the shared expert and the Zipf router skew.  Every
case is exact oracle math; the MXFP8 shapes are not held to the 6e-2 bound
against the unquantized oracle, which at these sizes measures the format."""
import random

import pytest

import gen
import tests.test_gpu_backward as B
import tests.test_gpu_forward as F
import tests.test_gpu_mxfp8 as MF

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def random_dims(seed, prec):
    rng = random.Random(seed)
    step, inter = {"bf16": (64, 64), "f32": (8, 8), "mxfp8": (128, 128)}[prec]
    E = rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 130])
    k = rng.randint(1, min(E, 16))
    T = rng.choice([1, 2, 31, 64, 65, 127, 200, 333, 512, 700])
    d = step * rng.randint(1, 4 if prec == "bf16" else 16)
    I = inter * rng.randint(1, 3)
    S = rng.randint(0, 1)
    Is = min(inter, 64) * rng.randint(1, 3) if S else 0
    return gen.Dims("rand_%s_%d" % (prec, seed), T, d, E, k, I, S, Is, prec, rng.choice([0.0, 1.2]),
                    seed=rng.randint(1, 10**6))


CASES = [("bf16", s) for s in range(12)] + [("f32", 100 + s) for s in range(6)]


@pytest.mark.parametrize("prec,seed", CASES)
def test_random_shape_forward(prec, seed):
    D = random_dims(seed, prec)
    F.SMALL[D.name] = D
    try:
        F.test_small_layer_every_entry_point(D.name)
    finally:
        del F.SMALL[D.name]


@pytest.mark.parametrize("seed", [s for p, s in CASES if p == "bf16"])
def test_random_shape_backward(seed):
    D = random_dims(seed, "bf16")
    B.SMALL[D.name] = D
    try:
        B.test_small_backward_full(D.name)
    finally:
        del B.SMALL[D.name]


@pytest.mark.parametrize("seed", range(200, 210))
def test_random_shape_mxfp8_forward(seed):
    MF.check_mxfp8_layer(random_dims(seed, "mxfp8"), strict=False)
