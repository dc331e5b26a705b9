"""The seeded input generator: Philox4x32-10 against its published
known-answer vectors (Salmon et al., SC'11, Random123 distribution), the bf16
rounding against torch's conversion, and the distribution recipe."""
import numpy as np
import pytest
import torch

import gen


@pytest.mark.parametrize("ctr,key,expect", [
    ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
    ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
    ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
     [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
])
def test_philox_known_answers(ctr, key, expect):
    assert list(gen.host_philox(ctr, key)) == expect


def test_bf16_rounding_matches_torch():
    f = gen.host_fill(0, 200_000, 7, 3, 1.2247, bf16=False)
    b = gen.host_fill(0, 200_000, 7, 3, 1.2247, bf16=True)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_distribution_and_slices():
    p = gen.Problem(gen.get_config("c1"))
    x = p.host_flat("x", 0, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    w = p.host_expert("w_gate", 3)
    assert abs(w.std() * np.sqrt(p.dims.d) - 1.0) < 2e-2
    # random access: a slice equals the same elements of a longer fill
    full = p.host_flat("w_down", 0, 5000)
    assert np.array_equal(full[1234:2345], p.host_flat("w_down", 1234, 1111))
    rows = p.host_rows("x", [5, 2])
    assert np.array_equal(rows[1], p.host_flat("x", 2 * p.dims.d, p.dims.d))


def test_zipf_bias_recipe():
    p = gen.Problem(gen.get_config("c3a"))
    b = p.logit_bias().astype(np.float64)
    pi = p.expert_permutation()
    assert sorted(pi) == list(range(256))
    probs = np.exp(b)
    assert abs(probs.sum() - 1.0) < 1e-5
    # rank r expert has probability proportional to r^-1.2
    ranked = probs[pi]
    assert np.all(np.diff(ranked) < 0)
    assert abs(ranked[0] / ranked[1] - 2 ** 1.2) < 1e-4
    assert gen.Problem(gen.get_config("c1")).logit_bias() is None
