"""The Python binding rejects host tensors before anything reaches the C ABI (no GPU needed)."""

import pytest
import torch

from blockwise_fp8_linear_quant_amd import binding as B


def test_host_tensors_are_rejected():
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        B.fp8_quant_1x128(x)
    with pytest.raises(TypeError):
        B.fp8_quant_1x128_dual(x)
    with pytest.raises(TypeError):
        B.fp8_quant_128x128(x)
    q = torch.zeros((4, 128), dtype=torch.uint8)
    s = torch.zeros((1, 4), dtype=torch.float32)
    w = torch.zeros((128, 128), dtype=torch.uint8)
    sw = torch.zeros((1, 1), dtype=torch.float32)
    with pytest.raises(TypeError):
        B.fp8_block_gemm_fwd(q, s, w, sw)
    with pytest.raises(TypeError):
        B.bf16_gemm_nt(x, x)
    with pytest.raises(TypeError):
        B.fp8_e4m3_encode(torch.zeros(8))


def test_linear_input_width_is_checked():
    # A [4, 256] input to a 128-wide linear must not be read as [8, 128].
    from blockwise_fp8_linear_quant_amd.linear import _rows
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _rows(x, 128)
    assert _rows(x, 256).shape == (4, 256)
    assert _rows(torch.zeros((2, 3, 128), dtype=torch.bfloat16), 128).shape == (6, 128)
