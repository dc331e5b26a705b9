"""Seeded synthetic inputs for the MoE layer, shared by the oracle side and
the GPU side.

This package holds no arithmetic of the MoE layer.  It produces the input
tensors (activations, router and expert weights, the output gradient and the
skewed-routing logit bias) from a counter-based generator, Philox4x32-10,
implemented once in ``philox4x32.h`` and compiled both for the host (gcc,
``libmoegen_host.so``) and for the device (hipcc, ``libmoegen_dev.so``).
Because the generator is counter-based, any slice of any tensor can be
regenerated on the host without materialising the rest, which is how the
oracle side checks samples of the largest workloads.
"""
from .configs import CONFIGS, Dims, get_config  # noqa: F401
from .problem import Problem, STREAMS  # noqa: F401
from ._lib import host_fill, host_philox, host_u32, device_fill, bf16_bits_to_f64, build  # noqa: F401
