"""moe_permute_noalloc, the entry point that allocates nothing (its scratch
is a static device array), through the C ABI: the same outputs bit for bit
as moe_permute on the same inputs, on consecutive calls whose second is
smaller (the array keeps the first call's contents), at the array's
capacity, in bf16 and MXFP8, and requests beyond the capacity rejected."""
import ctypes

import numpy as np
import pytest

import gen
from tests.moe_parity import device_problem

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def routed(D):
    import mixture_experts_layer_prefix_amd as M
    p, t, md, w = device_problem(D)
    _, idx, _ = M.route(t["x"], t["w_router"], md, D.prec, bias=t["bias"])
    return md, t["x"], idx


def compare(D):
    import mixture_experts_layer_prefix_amd as M
    md, x, idx = routed(D)
    want = M.permute(idx, x, md, D.prec)
    out = tuple(None if v is None else torch.full_like(v, 0x55 if v.dtype == torch.uint8 else -7) for v in want)
    got = M.permute_noalloc(idx, x, md, D.prec, out)
    torch.cuda.synchronize()
    for n, a, b in zip(("counts", "offsets", "row_token", "token_row", "x_perm", "x_perm_scale"), got, want):
        if b is None:
            assert a is None, n
            continue
        assert torch.equal(a, b), "%s differs from moe_permute" % n
    say("   %s: T=%d E=%d k=%d equal to moe_permute (max rows per expert %d)"
        % (D.name, D.T, D.E, D.k, int(want[0].max())))


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_noalloc_matches_permute_on_consecutive_calls(prec):
    big = gen.Dims("na_big", 3000, 256, 64, 6, 128, 0, 0, prec, 1.2)
    small = gen.Dims("na_small", 700, 256, 64, 6, 128, 0, 0, prec, 0.0)
    compare(big)
    compare(small)
    compare(big)


def test_noalloc_at_capacity_then_smaller():
    """ceil(T/32) * E * 4 bytes equal to the 16 MiB array, then a small call."""
    import mixture_experts_layer_prefix_amd as M
    cap = M._lib.lib().moe_permute_noalloc_scratch_bytes()
    T = cap // (1024 * 4) * 32
    compare(gen.Dims("na_cap", T, 64, 1024, 2, 64, 0, 0, "bf16", 1.2))
    compare(gen.Dims("na_after", 257, 64, 1024, 16, 64, 0, 0, "bf16", 0.0))


def test_noalloc_rejects_beyond_capacity():
    import mixture_experts_layer_prefix_amd as M
    from mixture_experts_layer_prefix_amd import _lib as L
    cap = L.lib().moe_permute_noalloc_scratch_bytes()
    T = cap // (1024 * 4) * 32 + 1
    d = M.Dims(T, 64, 1024, 2, 64)
    buf = torch.empty(16, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    st = L.lib().moe_permute_noalloc(ctypes.byref(d.c()), L.PREC["bf16"], p, p, p, p, p, p, None, None, None)
    assert st == L.MOE_EWORKSPACE
