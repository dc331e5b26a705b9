"""MI355X-native (gfx950) hot path of a DeepSeek-V3-style MoE layer.

The compute runs in hand-written HIP kernels inside libmoe.so (C ABI in
include/moe.h); this package only marshals torch tensors (device memory and
the current stream) into those calls.
"""
from . import _lib  # noqa: F401
from .ops import (Dims, Weights, ForwardPlan, route, permute, permute_noalloc, expert_ffn, expert_gate_up, expert_down,  # noqa: F401
                  shared_ffn, combine, combine_into, layer_forward, quantize_mxfp8, quantize_mxfp8_rows_t, prepare_mxfp8, workspace_bytes,
                  BackwardPlan, layer_backward, transpose_weights, prepare_backward, StageTimer,
                  mx_mma_tiles, bf16_mma_tiles)
