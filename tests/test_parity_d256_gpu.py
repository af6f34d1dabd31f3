"""GPU parity at head dim 256 against the fp64 oracle, with the tolerances
of each dtype: the forward (dense, causal, jagged, biased; bf16, fp16,
fp32), the JVP (bf16, fp16; launches over 64-wide slices of the value
columns) and the backward (dense, jagged, biased; bf16, fp16).  The
256-wide kernels run one wave per SIMD; the plain forward streams 64-key
tiles through the split K-side / V-side LDS layout, the JVP and the biased
instances 32-key tiles."""

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



@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_backward(gpu_lib, dtype, causal):
    """dQ, dK, dV at head dim 256 (dK and dV from two passes of the dK/dV
    kernel): ragged 128-row tiles, one row, cross-attention, and the jagged
    layout with empty, short and truncated sequences."""
    from test_parity_bwd_gpu import bwd_case
    from test_parity_jagged_bwd_gpu import jagged_bwd_case
    bwd_case(2, 2, 300, 300, 256, causal, seed=241, dtype=dtype)
    bwd_case(1, 2, 1, 1, 256, causal, seed=242, dtype=dtype)
    if not causal:
        bwd_case(1, 2, 77, 333, 256, False, seed=243, dtype=dtype)
    jagged_bwd_case([5, 0, 300, 64, 129, 1], 2, 256, dtype, 256, causal, seed=244)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_bias_backward(gpu_lib, dtype, causal):
    """The backward with an additive bias (and its gradient) or a boolean
    mask at head dim 256, full-shape and broadcast operands."""
    from test_parity_bias_bwd_gpu import bias_bwd_case
    bias_bwd_case(2, 2, 300, 300, 256, dtype, causal, "add", seed=245)
    bias_bwd_case(2, 2, 300, 300, 256, dtype, causal, "mask", seed=246)
    bias_bwd_case(2, 2, 200, 200, 256, dtype, causal, "add", bshape=(1, 2, 200, 200), seed=247)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_jvp(gpu_lib, dtype, causal):
    """O, tO, LSE at head dim 256: ragged tiles, one row and (non-causal)
    cross-attention; each value half comes from its own launch, both write
    the same LSE."""
    from test_parity_gpu import jvp_case
    jvp_case(2, 2, 300, 300, 256, dtype, causal, seed=251)
    jvp_case(1, 2, 1, 1, 256, dtype, causal, seed=252)
    if not causal:
        jvp_case(1, 2, 77, 333, 256, dtype, False, seed=253)
