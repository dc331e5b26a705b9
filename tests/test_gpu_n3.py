"""GPU parity at the other layer shapes the Mixture-of-Kittens blog post
benchmarks ("MoE layer benchmarks": Kimi K2.7 Code, GLM-5.2, Qwen3.5-397B-A17B
and DeepSeek-V4-Pro), through the C ABI, with the checks and bars of the
DeepSeek-V3-shaped tests:
  * whole layers on one GPU (T=8192, Zipf-skewed routing, one shared expert):
    bf16 and MXFP8 forward on sampled tokens with bit-exact routing, bf16
    backward of all four and the MXFP8 backward of GLM-5.2 on sampled tokens
    and weight-gradient columns of every expert;
  * one GPU's share of the post's EP-64 runs (the E/64 local experts and the
    2,048·k rows they receive, gen/configs.py): MXFP8 backward on sampled
    tokens and weight-gradient columns.
Every sample is exact per-element oracle math (the MXFP8 ones also against the
quantization-aware model)."""
import pytest

import gen
from gen.configs import SHAPES

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

WHOLE = [n for n in SHAPES if n != "dsv3"]


@pytest.fixture(autouse=True)
def release_cached_memory():
    """Each case allocates tens of GB of weights: hand the previous case's
    cached blocks back first."""
    torch.cuda.empty_cache()
    yield


@pytest.mark.parametrize("name", WHOLE)
def test_whole_layer_bf16_forward_sampled(name):
    from tests.test_gpu_forward import check_forward_sampled
    check_forward_sampled(gen.get_config(name), 128)


@pytest.mark.parametrize("name", WHOLE)
def test_whole_layer_mxfp8_forward_sampled(name):
    from tests.test_gpu_forward import check_forward_sampled
    check_forward_sampled(gen.get_config(name + "_mx"), 128)


@pytest.mark.parametrize("name", WHOLE)
def test_whole_layer_bf16_backward_sampled(name):
    from tests.test_gpu_backward import check_backward_sampled
    check_backward_sampled(gen.get_config(name), ntok=48)


@pytest.mark.parametrize("name", ["glm52"])
def test_whole_layer_mxfp8_backward_sampled(name):
    from tests.test_gpu_mxfp8_backward import check_backward_sampled
    check_backward_sampled(gen.get_config(name + "_mx"), ntok=48)


@pytest.mark.parametrize("name", list(SHAPES))
def test_ep64_share_mxfp8_backward_sampled(name):
    from tests.test_gpu_mxfp8_backward import check_backward_sampled
    check_backward_sampled(gen.get_config("ep64_" + name))
