"""The binding refuses tensors the kernels would overrun, before any launch.

The C ABI sees only pointers and leading dimensions; outputs smaller than the
region a kernel writes, scale tensors shorter than the blocks it reads and
block scales that are not dense would become out-of-bounds device accesses.
Each case here must raise ValueError in the binding.
"""

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd import binding
    return torch, binding


def test_undersized_outputs_are_refused(env):
    torch, B = env
    x = torch.zeros((300, 256), dtype=torch.bfloat16, device="cuda")
    small = torch.zeros((299, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        B.fp8_quant_1x128(x, q=small)
    with pytest.raises(ValueError):                       # token layout needs 384 padded columns
        B.fp8_quant_1x128(x, transpose_out=True, q=torch.zeros((256, 300), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        B.fp8_quant_1x128_dual(x, scales=torch.zeros((2, 200), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        B.fp8_quant_128x128(x, scales=torch.zeros((3, 1), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        B.fp8_swiglu_quant_1x128_dual(x, x, h_out=torch.zeros((300, 128), dtype=torch.bfloat16, device="cuda"))


def test_gemm_operands_are_checked(env):
    torch, B = env
    M, N, K = 256, 256, 512
    xq = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    wq = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sx = torch.zeros((K // 128, M), dtype=torch.float32, device="cuda")
    sw = torch.zeros((N // 128, K // 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):                       # row scales for 3 of 4 blocks
        B.fp8_block_gemm_fwd(xq, sx[:3], wq, sw)
    with pytest.raises(ValueError):                       # block scales not dense
        B.fp8_block_gemm_fwd(xq, sx, wq, torch.zeros((N // 128, 8), dtype=torch.float32, device="cuda")[:, :4])
    with pytest.raises(ValueError):                       # output too small
        B.fp8_block_gemm_fwd(xq, sx, wq, sw, y=torch.zeros((M, N - 1), dtype=torch.float32, device="cuda"))
    dyqT = torch.zeros((N, 256), dtype=torch.uint8, device="cuda")
    xqT = torch.zeros((K, 256), dtype=torch.uint8, device="cuda")
    sdyT = torch.zeros((2, N), dtype=torch.float32, device="cuda")
    sxT = torch.zeros((2, K), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):                       # M = 300 needs 384 padded tokens
        B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=300)
    with pytest.raises(ValueError):                       # dW must be float32 [N, K]
        B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=256, dw=torch.zeros((N, K - 128), dtype=torch.float32,
                                                                         device="cuda"))
