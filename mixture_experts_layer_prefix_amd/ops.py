"""Torch-facing wrappers of the C ABI: allocate outputs and workspaces with
torch (device memory only), pass raw pointers and the current HIP stream.
No arithmetic of the layer happens here."""
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import PREC, call, moe_dims, moe_grads, moe_routing, moe_weights


@dataclass(frozen=True)
class Dims:
    T: int
    d: int
    E: int
    k: int
    I: int
    S: int = 0
    Is: int = 0

    def c(self):
        return moe_dims(self.T, self.d, self.E, self.k, self.I, self.S, self.Is if self.S else 0)

    @property
    def R(self):
        return self.T * self.k


@dataclass
class Weights:
    w_router: torch.Tensor
    w_gate: Optional[torch.Tensor] = None
    w_up: Optional[torch.Tensor] = None
    w_down: Optional[torch.Tensor] = None
    ws_gate: Optional[torch.Tensor] = None
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None
    q_gate: Optional[torch.Tensor] = None
    q_gate_scale: Optional[torch.Tensor] = None
    q_up: Optional[torch.Tensor] = None
    q_up_scale: Optional[torch.Tensor] = None
    q_down: Optional[torch.Tensor] = None
    q_down_scale: Optional[torch.Tensor] = None
    wt_gate: Optional[torch.Tensor] = None
    wt_up: Optional[torch.Tensor] = None
    wt_down: Optional[torch.Tensor] = None
    wst_gate: Optional[torch.Tensor] = None
    wst_up: Optional[torch.Tensor] = None
    wst_down: Optional[torch.Tensor] = None
    qt_gate: Optional[torch.Tensor] = None
    qt_gate_scale: Optional[torch.Tensor] = None
    qt_up: Optional[torch.Tensor] = None
    qt_up_scale: Optional[torch.Tensor] = None
    qt_down: Optional[torch.Tensor] = None
    qt_down_scale: Optional[torch.Tensor] = None

    def c(self):
        w = moe_weights()
        for name, _ in moe_weights._fields_:
            t = getattr(self, name)
            setattr(w, name, t.data_ptr() if t is not None else None)
        return w


def _p(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _act_dtype(prec):
    return torch.float32 if prec == "f32" else torch.bfloat16


def workspace_bytes(dims: Dims, prec: str, which: int) -> int:
    n = ctypes.c_size_t(0)
    call("moe_workspace_bytes", ctypes.byref(dims.c()), PREC[prec], which, ctypes.byref(n))
    return n.value


def _workspace(dims, prec, which, device):
    n = workspace_bytes(dims, prec, which)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device), n


def route(x, w_router, dims: Dims, prec: str, bias=None):
    dev = x.device
    logits = torch.empty(dims.T, dims.E, dtype=torch.float32, device=dev)
    idx = torch.empty(dims.T, dims.k, dtype=torch.int32, device=dev)
    w = torch.empty(dims.T, dims.k, dtype=torch.float32, device=dev)
    call("moe_route", ctypes.byref(dims.c()), PREC[prec], _p(x), _p(w_router), _p(bias), _p(logits), _p(idx), _p(w),
         _stream())
    return logits, idx, w


def permute(topk_idx, x, dims: Dims, prec: str, gather=True):
    dev = topk_idx.device
    counts = torch.empty(dims.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(dims.E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(dims.R, 1), dtype=torch.int32, device=dev)
    token_row = torch.empty(dims.T, dims.k, dtype=torch.int32, device=dev)
    x_perm = scale = None
    if gather:
        if prec == "mxfp8":
            x_perm = torch.empty(dims.R, dims.d, dtype=torch.uint8, device=dev)
            scale = torch.empty(dims.R, dims.d // 32, dtype=torch.uint8, device=dev)
        else:
            x_perm = torch.empty(dims.R, dims.d, dtype=_act_dtype(prec), device=dev)
    ws, n = _workspace(dims, prec, 1, dev)
    call("moe_permute", ctypes.byref(dims.c()), PREC[prec], _p(topk_idx), _p(x), _p(counts), _p(offsets),
         _p(row_token), _p(token_row), _p(x_perm), _p(scale), _p(ws), n, _stream())
    return counts, offsets, row_token[:dims.R], token_row, x_perm, scale


def permute_noalloc(topk_idx, x, dims: Dims, prec: str, out):
    """moe_permute_noalloc into caller-allocated outputs: out = (counts,
    offsets, row_token, token_row, x_perm, x_perm_scale) as permute returns
    them (x_perm and x_perm_scale may be None).  Allocates nothing."""
    counts, offsets, row_token, token_row, x_perm, scale = out
    call("moe_permute_noalloc", ctypes.byref(dims.c()), PREC[prec], _p(topk_idx), _p(x), _p(counts), _p(offsets),
         _p(row_token), _p(token_row), _p(x_perm), _p(scale), _stream())
    return out


def expert_ffn(x_perm, x_perm_scale, offsets, weights: Weights, dims: Dims, prec: str):
    dev = offsets.device
    o_perm = torch.empty(dims.R, dims.d, dtype=_act_dtype(prec), device=dev)
    ws, n = _workspace(dims, prec, 2, dev)
    w = weights.c()
    call("moe_expert_ffn", ctypes.byref(dims.c()), PREC[prec], _p(x_perm), _p(x_perm_scale), _p(offsets),
         ctypes.byref(w), _p(o_perm), _p(ws), n, _stream())
    return o_perm


def expert_gate_up(x_perm, x_perm_scale, offsets, weights: Weights, dims: Dims, prec: str, ws=None):
    dev = offsets.device
    if prec == "mxfp8":
        h = torch.empty(dims.R, dims.I, dtype=torch.uint8, device=dev)
        # slab-major scales [I/128][R][4] (moe_quantize_mxfp8 axis 2 layout)
        h_scale = torch.empty(dims.I // 128, dims.R, 4, dtype=torch.uint8, device=dev)
    else:
        h = torch.empty(dims.R, dims.I, dtype=_act_dtype(prec), device=dev)
        h_scale = None
    if ws is None:
        ws, n = _workspace(dims, prec, 2, dev)
    else:
        n = ws.numel()
    w = weights.c()
    call("moe_expert_gate_up", ctypes.byref(dims.c()), PREC[prec], _p(x_perm), _p(x_perm_scale), _p(offsets),
         ctypes.byref(w), _p(h), _p(h_scale), _p(ws), n, _stream())
    return h, h_scale


def expert_down(h, h_scale, offsets, weights: Weights, dims: Dims, prec: str, ws=None):
    dev = offsets.device
    o_perm = torch.empty(dims.R, dims.d, dtype=_act_dtype(prec), device=dev)
    if ws is None:
        ws, n = _workspace(dims, prec, 2, dev)
    else:
        n = ws.numel()
    w = weights.c()
    call("moe_expert_down", ctypes.byref(dims.c()), PREC[prec], _p(h), _p(h_scale), _p(offsets), ctypes.byref(w),
         _p(o_perm), _p(ws), n, _stream())
    return o_perm


def shared_ffn(x, weights: Weights, dims: Dims, prec: str):
    y_shared = torch.empty(dims.T, dims.d, dtype=_act_dtype(prec), device=x.device)
    ws, n = _workspace(dims, prec, 3, x.device)
    w = weights.c()
    call("moe_shared_ffn", ctypes.byref(dims.c()), PREC[prec], _p(x), ctypes.byref(w), _p(y_shared), _p(ws), n,
         _stream())
    return y_shared


def combine(o_perm, token_row, topk_w, y_shared, dims: Dims, prec: str):
    y = torch.empty(dims.T, dims.d, dtype=_act_dtype(prec), device=token_row.device)
    call("moe_combine", ctypes.byref(dims.c()), PREC[prec], _p(o_perm), _p(token_row), _p(topk_w), _p(y_shared), _p(y),
         _stream())
    return y


def combine_into(o_perm, token_row, topk_w, y_shared, dims: Dims, prec: str, y):
    """moe_combine into a caller-allocated y."""
    call("moe_combine", ctypes.byref(dims.c()), PREC[prec], _p(o_perm), _p(token_row), _p(topk_w), _p(y_shared), _p(y),
         _stream())
    return y


class ForwardPlan:
    """Pre-allocated output, routing buffers and workspace of one forward
    configuration, so that repeated calls allocate nothing."""

    def __init__(self, dims: Dims, prec: str, device="cuda", keep_routing=True, keep_gu=False):
        """keep_gu: also keep the gate/up projections G | U (routed and shared)
        for a later backward, which then skips their recomputation."""
        self.dims, self.prec = dims, prec
        T, E, k = dims.T, dims.E, dims.k
        self.y = torch.empty(T, dims.d, dtype=_act_dtype(prec), device=device)
        self.routing = None
        self.rt = None
        if keep_routing:
            self.routing = dict(
                logits=torch.empty(T, E, dtype=torch.float32, device=device),
                topk_idx=torch.empty(T, k, dtype=torch.int32, device=device),
                topk_w=torch.empty(T, k, dtype=torch.float32, device=device),
                expert_counts=torch.empty(E, dtype=torch.int32, device=device),
                expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
                row_token=torch.empty(max(dims.R, 1), dtype=torch.int32, device=device),
                token_row=torch.empty(T, k, dtype=torch.int32, device=device))
            if keep_gu:
                self.routing["gu"] = torch.empty(max(dims.R, 1), 2 * dims.I, dtype=torch.bfloat16, device=device)
                if dims.S:
                    self.routing["gu_shared"] = torch.empty(T, 2 * dims.Is, dtype=torch.bfloat16, device=device)
            self.rt = moe_routing(**{n: t.data_ptr() for n, t in self.routing.items()})
        self.ws, self.ws_bytes = _workspace(dims, prec, 0, device)
        self.cdims = dims.c()

    def run(self, x, weights: Weights, bias=None):
        w = weights.c()
        call("moe_layer_forward", ctypes.byref(self.cdims), PREC[self.prec], _p(x), ctypes.byref(w), _p(bias),
             _p(self.y), ctypes.byref(self.rt) if self.rt is not None else None, _p(self.ws), self.ws_bytes,
             _stream())
        return self.y


def layer_forward(x, weights: Weights, dims: Dims, prec: str, bias=None, keep_routing=True, keep_gu=False):
    plan = ForwardPlan(dims, prec, x.device, keep_routing, keep_gu)
    y = plan.run(x, weights, bias)
    return y, plan.routing


def quantize_mxfp8(src, axis):
    rows, cols = src.shape
    dst = torch.empty(rows, cols, dtype=torch.uint8, device=src.device)
    if axis == 0:
        scale = torch.empty(rows, cols // 32, dtype=torch.uint8, device=src.device)
    elif axis == 2:  # slab-major [cols/128][rows][4] (the grouped GEMMs' weight layout)
        scale = torch.empty(cols // 128, rows, 4, dtype=torch.uint8, device=src.device)
    else:
        scale = torch.empty(rows // 32, cols, dtype=torch.uint8, device=src.device)
    call("moe_quantize_mxfp8", _p(src), rows, cols, axis, _p(dst), _p(scale), _stream())
    return dst, scale


def quantize_mxfp8_rows_t(src, seg_off, pad_off, gather=None):
    """moe_quantize_mxfp8_rows_t: the routed-row-axis MX quantization of a
    weight-gradient operand.  src [rows][cols] bf16; seg_off, pad_off int32
    [nseg+1] device tensors (pad_off: multiples of 128).  Returns the codes
    (p_cap * cols bytes) and scales (p_cap * cols / 32 bytes), p_cap =
    pad_off's last entry rounded to 128, as flat uint8 tensors."""
    cols = src.shape[1]
    p_cap = int(pad_off[-1].item())
    p_cap = (p_cap + 127) // 128 * 128
    dst = torch.empty(max(p_cap * cols, 16), dtype=torch.uint8, device=src.device)
    scale = torch.empty(max(p_cap * cols // 32, 16), dtype=torch.uint8, device=src.device)
    call("moe_quantize_mxfp8_rows_t", _p(src), src.stride(0), cols, _p(gather), _p(seg_off), _p(pad_off),
         seg_off.numel() - 1, p_cap, _p(dst), _p(scale), _stream())
    return dst[:p_cap * cols], scale[:p_cap * cols // 32]


def mx_mma_tiles(a, a_scale, b, b_scale, c):
    """moe_mx_mma_tiles: d[t] = c[t] + A[t] B[t]^T per tile through one
    scaled matrix-core operation.  a, b uint8 [n][32][64] E4M3 codes; a_scale,
    b_scale uint8 [n][32][2] E8M0 codes; c float32 [n][32][32].  Returns d."""
    n = a.shape[0]
    assert a.shape == (n, 32, 64) and b.shape == (n, 32, 64) and c.shape == (n, 32, 32)
    assert a_scale.shape == (n, 32, 2) and b_scale.shape == (n, 32, 2)
    assert a.dtype == b.dtype == a_scale.dtype == b_scale.dtype == torch.uint8 and c.dtype == torch.float32
    a, b, a_scale, b_scale, c = (t.contiguous() for t in (a, b, a_scale, b_scale, c))
    d = torch.empty_like(c)
    call("moe_mx_mma_tiles", _p(a), _p(a_scale), _p(b), _p(b_scale), _p(c), _p(d), n, _stream())
    return d


def bf16_mma_tiles(a, b, c):
    """moe_bf16_mma_tiles: d[t] = c[t] + A[t] B[t]^T per tile through one bf16
    matrix-core operation.  a, b bfloat16 [n][32][16]; c float32 [n][32][32].
    Returns d."""
    n = a.shape[0]
    assert a.shape == (n, 32, 16) and b.shape == (n, 32, 16) and c.shape == (n, 32, 32)
    assert a.dtype == b.dtype == torch.bfloat16 and c.dtype == torch.float32
    a, b, c = a.contiguous(), b.contiguous(), c.contiguous()
    d = torch.empty_like(c)
    call("moe_bf16_mma_tiles", _p(a), _p(b), _p(c), _p(d), n, _stream())
    return d


def prepare_mxfp8(weights: Weights, dims: Dims) -> Weights:
    """Weights with the routed experts pre-quantized for MOE_MXFP8 (blocks
    along each GEMM's K: d for gate/up, I for down)."""
    E, d, I = dims.E, dims.d, dims.I
    qg, sg = quantize_mxfp8(weights.w_gate.reshape(E * I, d), 2)
    qu, su = quantize_mxfp8(weights.w_up.reshape(E * I, d), 2)
    qd, sd = quantize_mxfp8(weights.w_down.reshape(E * d, I), 2)
    return Weights(w_router=weights.w_router, w_gate=weights.w_gate, w_up=weights.w_up, w_down=weights.w_down,
                   ws_gate=weights.ws_gate, ws_up=weights.ws_up, ws_down=weights.ws_down,
                   q_gate=qg, q_gate_scale=sg, q_up=qu, q_up_scale=su, q_down=qd, q_down_scale=sd)


def transpose_weights(w):
    """[batch][rows][cols] bf16 -> [batch][cols][rows] (moe_transpose_weights)."""
    b, r, c = w.shape
    out = torch.empty(b, c, r, dtype=w.dtype, device=w.device)
    call("moe_transpose_weights", _p(w), b, r, c, _p(out), _stream())
    return out


def prepare_backward(weights: Weights, mxfp8=False) -> Weights:
    """Weights with the transposed copies the backward's input-gradient GEMMs
    read (made once per weight update); with mxfp8 also their MX-quantized
    forms (blocks along the rows of the transposed copies: I for W_gate^T and
    W_up^T, d for W_down^T)."""
    import dataclasses
    t = {"wt_gate": weights.w_gate, "wt_up": weights.w_up, "wt_down": weights.w_down,
         "wst_gate": weights.ws_gate, "wst_up": weights.ws_up, "wst_down": weights.ws_down}
    out = dataclasses.replace(weights, **{n: (transpose_weights(v) if v is not None else None) for n, v in t.items()})
    if mxfp8:
        q = {}
        for n in ("gate", "up", "down"):
            wt = getattr(out, "wt_" + n)
            codes, scale = quantize_mxfp8(wt.reshape(-1, wt.shape[-1]), 2)
            q["qt_" + n] = codes.reshape(wt.shape)
            q["qt_%s_scale" % n] = scale
        out = dataclasses.replace(out, **q)
    return out


class BackwardPlan:
    """Pre-allocated gradients and workspace of one backward configuration."""

    def __init__(self, dims: Dims, prec: str, device="cuda", router_grad=True):
        self.dims, self.prec = dims, prec
        T, d, E, k, I = dims.T, dims.d, dims.E, dims.k, dims.I
        bf = torch.bfloat16  # gradients are bf16 in both bf16 and MXFP8 modes
        self.dx = torch.empty(T, d, dtype=bf, device=device)
        self.grads = dict(
            dw_gate=torch.empty(E, I, d, dtype=bf, device=device),
            dw_up=torch.empty(E, I, d, dtype=bf, device=device),
            dw_down=torch.empty(E, d, I, dtype=bf, device=device),
            dtopk_w=torch.empty(T, k, dtype=torch.float32, device=device))
        if dims.S:
            self.grads.update(dws_gate=torch.empty(dims.S, dims.Is, d, dtype=bf, device=device),
                              dws_up=torch.empty(dims.S, dims.Is, d, dtype=bf, device=device),
                              dws_down=torch.empty(dims.S, d, dims.Is, dtype=bf, device=device))
        if router_grad:
            self.grads["dw_router"] = torch.empty(E, d, dtype=torch.float32, device=device)
        self.g = moe_grads(**{n: t.data_ptr() for n, t in self.grads.items()})
        self.ws, self.ws_bytes = _workspace(dims, prec, 4, device)
        self.cdims = dims.c()

    def run(self, dy, x, weights: Weights, routing):
        w = weights.c()
        rt = moe_routing(**{n: t.data_ptr() for n, t in routing.items()})
        call("moe_layer_backward", ctypes.byref(self.cdims), PREC[self.prec], _p(dy), _p(x), ctypes.byref(w),
             ctypes.byref(rt), _p(self.dx), ctypes.byref(self.g), _p(self.ws), self.ws_bytes, _stream())
        return self.dx, self.grads


def layer_backward(dy, x, weights: Weights, routing, dims: Dims, prec: str, router_grad=True):
    plan = BackwardPlan(dims, prec, dy.device, router_grad)
    return plan.run(dy, x, weights, routing)


FWD_STAGES = ("route", "schedule", "shared_ffn", "gate_up", "down", "combine")
BWD_STAGES = ("prepare", "replay_gate_up", "down_dgrad_swiglu", "router_weight_grad", "gate_up_dgrad",
              "shared_dgrad", "dx", "transposes", "wgrad_down", "wgrad_gate_up", "shared_wgrad", "router_grad")


class StageTimer:
    """Per-stage device times of the fused forward (which=0) or backward
    (which=1) from events the library records at its stage boundaries
    (moe_trace_events): one event set per call, read after the calls."""

    def __init__(self, which, calls):
        self.which = which
        self.names = FWD_STAGES if which == 0 else BWD_STAGES
        self.sets = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]
                     for _ in range(calls)]
        for evs in self.sets:  # create the underlying HIP events
            for e in evs:
                e.record()
        torch.cuda.synchronize()
        self.used = 0

    def arm(self, i):
        """Record the next traced call into event set i."""
        evs = self.sets[i]
        arr = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
        call("moe_trace_events", self.which, arr, len(evs))
        self.used = max(self.used, i + 1)

    def disarm(self):
        call("moe_trace_events", self.which, None, 0)

    def mean_ms(self):
        torch.cuda.synchronize()
        out = dict.fromkeys(self.names, 0.0)
        for evs in self.sets[:self.used]:
            for k, n in enumerate(self.names):
                out[n] += evs[k].elapsed_time(evs[k + 1]) / self.used
        return out
