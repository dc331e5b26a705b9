"""ctypes binding of libmoe.so (argument marshalling only).

Every entry point of include/moe.h is exposed under the same name.  The
library is loaded from this package directory; if it is missing the import
of any op fails loudly (there is no fallback path).
"""
import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8 = range(3)
PREC = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("I_shared", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
        "q_gate", "q_gate_scale", "q_up", "q_up_scale", "q_down", "q_down_scale",
        "wt_gate", "wt_up", "wt_down", "wst_gate", "wst_up", "wst_down",
        "qt_gate", "qt_gate_scale", "qt_up", "qt_up_scale", "qt_down", "qt_down_scale")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down", "dtopk_w", "dw_router")]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "row_token", "token_row", "gu",
        "gu_shared")]


_P = ctypes.c_void_p
_DIMS = ctypes.POINTER(moe_dims)
_SIGS = {
    "moe_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "moe_workspace_bytes": ([_DIMS, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "moe_route": ([_DIMS, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_permute": ([_DIMS, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_permute_noalloc": ([_DIMS, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_permute_noalloc_scratch_bytes": ([], ctypes.c_size_t),
    "moe_expert_ffn": ([_DIMS, ctypes.c_int, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P, ctypes.c_size_t, _P],
                       ctypes.c_int),
    "moe_expert_gate_up": ([_DIMS, ctypes.c_int, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P, _P,
                            ctypes.c_size_t, _P], ctypes.c_int),
    "moe_expert_down": ([_DIMS, ctypes.c_int, _P, _P, _P, ctypes.POINTER(moe_weights), _P, _P, ctypes.c_size_t, _P],
                        ctypes.c_int),
    "moe_shared_ffn": ([_DIMS, ctypes.c_int, _P, ctypes.POINTER(moe_weights), _P, _P, ctypes.c_size_t, _P],
                       ctypes.c_int),
    "moe_combine": ([_DIMS, ctypes.c_int, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_layer_forward": ([_DIMS, ctypes.c_int, _P, ctypes.POINTER(moe_weights), _P, _P,
                           ctypes.POINTER(moe_routing), _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_layer_backward": ([_DIMS, ctypes.c_int, _P, _P, ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing),
                            _P, ctypes.POINTER(moe_grads), _P, ctypes.c_size_t, _P], ctypes.c_int),
    "moe_set_max_workgroups": ([ctypes.c_int], ctypes.c_int),
    "moe_trace_events": ([ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int], ctypes.c_int),
    "moe_transpose_weights": ([_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P], ctypes.c_int),
    "moe_quantize_mxfp8": ([_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _P, _P, _P], ctypes.c_int),
    "moe_quantize_mxfp8_rows_t": ([_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                   _P, _P, _P], ctypes.c_int),
    "moe_mx_mma_tiles": ([_P, _P, _P, _P, _P, _P, ctypes.c_int64, _P], ctypes.c_int),
    "moe_bf16_mma_tiles": ([_P, _P, _P, _P, ctypes.c_int64, _P], ctypes.c_int),
}

_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so not found at %s: build it with __graft_entry__.build()" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def status_str(code):
    return lib().moe_status_str(code).decode()


def call(name, *args):
    """Call an entry point; raise MoeError on a non-OK status."""
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st, status_str(st))
    return st


def exported_symbols():
    return list(_SIGS)
