"""The C ABI on the host: the library loads, exports every entry point that
include/moe.h declares, and rejects bad arguments with the documented
status before any device work (these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_prefix_amd as M
from mixture_experts_layer_prefix_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared()
    assert len(names) >= 9
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.exported_symbols(), n


def test_status_strings():
    for s in range(5):
        assert L.status_str(s).startswith("MOE_")


def dims(**kw):
    base = dict(T=16, d=128, E=8, k=2, I=64, S=1, Is=64)
    base.update(kw)
    return M.Dims(**base)


def ws_status(d, prec="bf16", which=0):
    n = ctypes.c_size_t(0)
    return L.lib().moe_workspace_bytes(ctypes.byref(d.c()), L.PREC[prec], which, ctypes.byref(n)), n.value


@pytest.mark.parametrize("bad,status", [
    (dict(k=0), L.MOE_EINVAL), (dict(k=9), L.MOE_EINVAL), (dict(E=0), L.MOE_EINVAL), (dict(E=2000), L.MOE_EINVAL),
    (dict(T=-1), L.MOE_EINVAL), (dict(d=0), L.MOE_EINVAL), (dict(k=17, E=32), L.MOE_EINVAL),
    (dict(d=96), L.MOE_EUNSUPPORTED), (dict(I=100), L.MOE_EUNSUPPORTED), (dict(S=2), L.MOE_EUNSUPPORTED),
])
def test_dims_validation(bad, status):
    assert ws_status(dims(**bad))[0] == status


def test_workspace_sizes_grow_with_tokens():
    s0, n0 = ws_status(dims(T=16))
    s1, n1 = ws_status(dims(T=4096))
    assert s0 == s1 == L.MOE_OK and n1 > n0 > 0
    assert ws_status(dims(), "bf16", 7)[0] == L.MOE_EINVAL


def test_entry_points_reject_null_and_small_workspace_before_device_work():
    lib = L.lib()
    d = dims()
    st = lib.moe_route(ctypes.byref(d.c()), L.MOE_BF16, None, None, None, None, None, None, None)
    assert st == L.MOE_EINVAL
    fake = 1 << 20  # aligned host address: never dereferenced, validation fails first
    w = M.Weights(w_router=None).c()
    st = lib.moe_layer_forward(ctypes.byref(d.c()), L.MOE_BF16, fake, ctypes.byref(w), None, fake, None, fake,
                               16, None)
    assert st == L.MOE_EINVAL
    st = lib.moe_permute(ctypes.byref(d.c()), L.MOE_BF16, fake, fake, fake, fake, fake, fake, None, None, None, 0,
                         None)
    assert st == L.MOE_EWORKSPACE
    st = lib.moe_combine(ctypes.byref(d.c()), L.MOE_BF16, fake + 8, fake, fake, None, fake, None)
    assert st == L.MOE_EINVAL
    st = lib.moe_quantize_mxfp8(fake, 10, 33, 0, fake, fake, None)
    assert st == L.MOE_EINVAL


def test_backward_validation_before_device_work():
    lib = L.lib()
    d = dims()
    fake = 1 << 20
    w = M.Weights(w_router=None).c()
    g = L.moe_grads()
    rt = L.moe_routing()
    # fp32 and MXFP8 backward are not built
    for prec in (L.MOE_F32, L.MOE_MXFP8):
        st = lib.moe_layer_backward(ctypes.byref(d.c()), prec, fake, fake, ctypes.byref(w), ctypes.byref(rt), fake,
                                    ctypes.byref(g), fake, 1 << 40, None)
        assert st == L.MOE_EUNSUPPORTED
    # missing transposed weights / gradients / routing
    st = lib.moe_layer_backward(ctypes.byref(d.c()), L.MOE_BF16, fake, fake, ctypes.byref(w), ctypes.byref(rt), fake,
                                ctypes.byref(g), fake, 1 << 40, None)
    assert st == L.MOE_EINVAL
    st = lib.moe_layer_backward(ctypes.byref(d.c()), L.MOE_BF16, fake, fake, ctypes.byref(w), None, fake, None, fake,
                                1 << 40, None)
    assert st == L.MOE_EINVAL
    # complete arguments but a small workspace
    names = [n for n, _ in L.moe_weights._fields_]
    w_full = L.moe_weights(**{n: fake for n in names})
    g_full = L.moe_grads(**{n: fake for n, _ in L.moe_grads._fields_})
    rt_full = L.moe_routing(**{n: fake for n, _ in L.moe_routing._fields_})
    st = lib.moe_layer_backward(ctypes.byref(d.c()), L.MOE_BF16, fake, fake, ctypes.byref(w_full),
                                ctypes.byref(rt_full), fake, ctypes.byref(g_full), fake, 64, None)
    assert st == L.MOE_EWORKSPACE
    # misaligned gradient pointer
    g_bad = L.moe_grads(**{n: fake for n, _ in L.moe_grads._fields_})
    g_bad.dw_up = fake + 2
    st = lib.moe_layer_backward(ctypes.byref(d.c()), L.MOE_BF16, fake, fake, ctypes.byref(w_full),
                                ctypes.byref(rt_full), fake, ctypes.byref(g_bad), fake, 1 << 40, None)
    assert st == L.MOE_EINVAL
    assert ws_status(d, "bf16", 4)[0] == L.MOE_OK and ws_status(d, "bf16", 4)[1] > 0
    assert lib.moe_transpose_weights(fake, -1, 4, 4, fake, None) == L.MOE_EINVAL
    assert lib.moe_transpose_weights(None, 1, 4, 4, fake, None) == L.MOE_EINVAL
    assert lib.moe_transpose_weights(None, 0, 4, 4, None, None) == L.MOE_OK
    # the matrix-core tile entry point: count, null and alignment checks on the host
    assert lib.moe_mx_mma_tiles(fake, fake, fake, fake, fake, fake, -1, None) == L.MOE_EINVAL
    assert lib.moe_mx_mma_tiles(fake, fake, fake, fake, fake, fake, 1 << 31, None) == L.MOE_EINVAL
    assert lib.moe_mx_mma_tiles(fake, None, fake, fake, fake, fake, 1, None) == L.MOE_EINVAL
    assert lib.moe_mx_mma_tiles(fake + 8, fake, fake, fake, fake, fake, 1, None) == L.MOE_EINVAL
    assert lib.moe_mx_mma_tiles(None, None, None, None, None, None, 0, None) == L.MOE_OK
    assert lib.moe_bf16_mma_tiles(fake, fake, fake, fake, -1, None) == L.MOE_EINVAL
    assert lib.moe_bf16_mma_tiles(fake, None, fake, fake, 1, None) == L.MOE_EINVAL
    assert lib.moe_bf16_mma_tiles(fake + 8, fake, fake, fake, 1, None) == L.MOE_EINVAL
    assert lib.moe_bf16_mma_tiles(None, None, None, None, 0, None) == L.MOE_OK


def test_permute_noalloc_rejects_beyond_its_scratch_on_the_host():
    """moe_permute_noalloc refuses a schedule whose block histograms exceed
    its static scratch (MOE_EWORKSPACE) before any device work: the pointers
    here are never dereferenced."""
    cap = L.lib().moe_permute_noalloc_scratch_bytes()
    assert cap == 16 << 20
    fake = 0x100000
    for T, E in ((cap // (1024 * 4) * 32 + 1, 1024), (cap // (256 * 4) * 32 + 1, 256)):
        d = M.Dims(T, 64, E, 2, 64)
        st = L.lib().moe_permute_noalloc(ctypes.byref(d.c()), L.PREC["bf16"], fake, fake, fake, fake, fake, fake,
                                        None, None, None)
        assert st == L.MOE_EWORKSPACE, (T, E, st)
    d = M.Dims(16, 64, 8, 2, 64)
    st = L.lib().moe_permute_noalloc(ctypes.byref(d.c()), L.PREC["bf16"], fake, fake, None, fake, fake, fake,
                                    None, None, None)
    assert st == L.MOE_EINVAL
