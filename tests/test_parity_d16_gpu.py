"""GPU parity at head dim 16 against the fp64 oracle: equal dims 16 on the
dense, causal, JVP and jagged forward (bf16, fp16, fp32), a value dim of 16
under wider query/key dims, and the backward (dense, jagged, biased; bf16,
fp16).  A 16-wide value tile is laid out 32 wide in LDS with a zero upper
half, so the PV product keeps whole MFMA blocks; the backward's gradient
kernels run the whole 16-wide head that way."""

import pytest

from test_parity_gpu import dense_case, jvp_case, jagged_case
from test_parity_dv_gpu import dv_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d16_dense_and_jvp(gpu_lib, dtype, causal):
    dense_case(2, 3, 300, 300, 16, dtype, causal, seed=130)
    dense_case(1, 2, 1, 1, 16, dtype, causal, seed=131)
    jvp_case(2, 2, 300, 300, 16, dtype, causal, seed=132)


@pytest.mark.parametrize("causal", [False, True])
def test_d16_jagged(gpu_lib, causal):
    jagged_case([5, 0, 300, 64, 129], 2, 16, "bf16", 256, causal, seed=133)


@pytest.mark.parametrize("Dqk", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_value_dim_16(gpu_lib, Dqk, dtype):
    dv_case(2, 2, 300, 300, Dqk, 16, dtype, False, False, seed=134)
    dv_case(1, 2, 200, 200, Dqk, 16, dtype, True, False, seed=135)
    dv_case(1, 2, 200, 200, Dqk, 16, dtype, True, True, seed=136)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d16_bias_and_mask(gpu_lib, dtype, causal):
    """Head dim 16 on the biased forward: additive bias and boolean mask,
    full-shape and broadcast operands, ragged tiles."""
    from test_parity_bias_gpu import bias_case
    bias_case(2, 3, 300, 300, 16, dtype, causal, "add", seed=137)
    bias_case(2, 3, 300, 300, 16, dtype, causal, "mask", seed=138)
    bias_case(2, 2, 200, 200, 16, dtype, causal, "add", bshape=(1, 2, 200, 200), seed=139)
    if not causal:
        bias_case(1, 2, 77, 333, 16, dtype, False, "mask", seed=140, keep=0.3)



@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d16_backward(gpu_lib, dtype, causal):
    """dQ, dK, dV at head dim 16: several 128-row tiles with ragged tails,
    one row, cross-attention, and the jagged layout with empty, short and
    truncated sequences."""
    from test_parity_bwd_gpu import bwd_case
    from test_parity_jagged_bwd_gpu import jagged_bwd_case
    bwd_case(2, 3, 300, 300, 16, causal, seed=141, dtype=dtype)
    bwd_case(1, 2, 1, 1, 16, causal, seed=142, dtype=dtype)
    if not causal:
        bwd_case(1, 2, 77, 333, 16, False, seed=143, dtype=dtype)
    jagged_bwd_case([5, 0, 300, 64, 129, 1, 128, 700], 2, 16, dtype, 256, causal, seed=144)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d16_bias_backward(gpu_lib, dtype, causal):
    """The backward with an additive bias (and its gradient) or a boolean
    mask at head dim 16, full-shape and broadcast operands."""
    from test_parity_bias_bwd_gpu import bias_bwd_case
    bias_bwd_case(2, 3, 300, 300, 16, dtype, causal, "add", seed=145)
    bias_bwd_case(2, 3, 300, 300, 16, dtype, causal, "mask", seed=146)
    bias_bwd_case(2, 2, 200, 200, 16, dtype, causal, "add", bshape=(1, 2, 200, 200), seed=147)
