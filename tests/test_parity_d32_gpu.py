"""GPU parity at head dim 32 (the 32-wide instances of every path) against
the fp64 oracle: dense and causal forward in bf16, fp16 and fp32, the fused
JVP, the jagged forward, bias and mask, and the dense and jagged backward.
Tolerances are those of each dtype (tests/parity.py and the backward
files)."""

import pytest

from test_parity_gpu import dense_case, jvp_case, jagged_case
from test_parity_bias_gpu import bias_case
from test_parity_bwd_gpu import bwd_case
from test_parity_jagged_bwd_gpu import jagged_bwd_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d32_dense(gpu_lib, dtype, causal):
    dense_case(2, 3, 300, 300, 32, dtype, causal, seed=90)
    dense_case(1, 2, 1, 1, 32, dtype, causal, seed=91)
    dense_case(2, 2, 640, 640, 32, dtype, causal, seed=92)  # small causal grid: paired key-split instances


def test_d32_cross_attention(gpu_lib):
    dense_case(2, 2, 77, 333, 32, "bf16", False, seed=93)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_d32_jvp(gpu_lib, dtype, causal):
    jvp_case(2, 3, 400, 400, 32, dtype, causal, seed=94)


@pytest.mark.parametrize("causal", [False, True])
def test_d32_jagged(gpu_lib, causal):
    jagged_case([5, 0, 300, 64, 129], 3, 32, "bf16", 256, causal, seed=95)


@pytest.mark.parametrize("kind", ["add", "mask"])
def test_d32_bias(gpu_lib, kind):
    for dtype in ("bf16", "fp16", "fp32"):
        bias_case(2, 3, 300, 300, 32, dtype, True, kind, seed=96)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d32_bwd(gpu_lib, dtype, causal):
    bwd_case(2, 3, 300, 300, 32, causal, seed=97, dtype=dtype)
    jagged_bwd_case([5, 0, 300, 64, 129, 1], 2, 32, dtype, 256, causal, seed=98)
