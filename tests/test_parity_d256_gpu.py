"""GPU parity at head dim 256 (the plain forward: dense, causal, jagged;
bf16, fp16, fp32) against the fp64 oracle, with the tolerances of each
dtype.  The 256-wide kernels use 32-key tiles and one wave per SIMD."""

import pytest

from test_parity_gpu import dense_case, jagged_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_dense(gpu_lib, dtype, causal):
    dense_case(2, 2, 300, 300, 256, dtype, causal, seed=120)
    dense_case(1, 2, 1, 1, 256, dtype, causal, seed=121)
    dense_case(1, 1, 129, 129, 256, dtype, causal, seed=122)


def test_d256_cross_attention(gpu_lib):
    dense_case(2, 2, 77, 333, 256, "bf16", False, seed=123)


@pytest.mark.parametrize("causal", [False, True])
def test_d256_jagged(gpu_lib, causal):
    jagged_case([5, 0, 300, 64, 129], 2, 256, "bf16", 256, causal, seed=124)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_bias_and_mask(gpu_lib, dtype, causal):
    """Head dim 256 on the biased forward: additive bias and boolean mask,
    full-shape and broadcast operands, ragged 32-key tiles."""
    from test_parity_bias_gpu import bias_case
    bias_case(2, 2, 300, 300, 256, dtype, causal, "add", seed=123)
    bias_case(2, 2, 200, 200, 256, dtype, causal, "mask", seed=124)
    bias_case(2, 2, 130, 130, 256, dtype, causal, "add", bshape=(1, 2, 130, 130), seed=125)

