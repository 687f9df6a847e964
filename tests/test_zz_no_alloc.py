"""The allocation-free split GEMM (fp8_block_gemm_split2_noalloc) against the
split GEMM with a caller workspace (fp8_block_gemm with FP8BLK_GEMM_SPLIT2).

Both run the same kernels with the same split, so their outputs must be equal
bit for bit; they are also held to the acceptance rule against the oracle.  Two
calls in a row share the library's static scratch: a weight gradient of 2048 x
2048 (128 output tiles, the most the scratch holds), then a smaller forward
GEMM with a ragged token count; the first call's leftovers must not leak into
the second.  Everything goes through the C ABI.
"""

import numpy as np
import pytest

from blockwise_fp8_linear_quant_amd import workloads as W
from oracle import compare, gemm, quant
from tests.gpu_util import dev_bf16, host, sample_index, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd import binding
    return binding


def test_noalloc_split_matches_workspace_split(B):
    import torch
    # Call 1: weight gradient dW [2048, 2048] over 4096 tokens (128 tiles of 256 x 128).
    M, N, K = 4096, 2048, 2048
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(94, 0, "o", "x"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(94, 0, "o", "dy"))
    dyqT, sdyT = B.fp8_quant_1x128(dev_bf16(dyb), transpose_out=True)
    xqT, sxT = B.fp8_quant_1x128(dev_bf16(xb), transpose_out=True)
    say("noalloc split wgrad", (M, N, K))
    got = torch.full((N, K), float("nan"), device="cuda")
    B.fp8_block_gemm_split2_noalloc(B.OP_WGRAD, dyqT, sdyT, xqT, sxT, M, N, K, got)
    ref = torch.empty((N, K), dtype=torch.float32, device="cuda")
    B.fp8_block_gemm(B.OP_WGRAD, dyqT, sdyT, xqT, sxT, M, N, K, ref, split2=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    odyqT, osdyT = quant.quant_1x128_tokens(dyb)
    oxqT, osxT = quant.quant_1x128_tokens(xb)
    rng = np.random.default_rng(94)
    g = host(got)
    rows = sample_index(N, 24, rng, must=(0, N - 1, 255, 256))
    cols = sample_index(K, 24, rng, must=(0, K - 1, 127, 128))
    for r, c in ((rows, None), (None, cols)):
        y, bnd = gemm.wgrad(odyqT, osdyT, oxqT, osxT, r, c)
        ok, rep = compare.check_fp32(g[r] if r is not None else g[:, c], y, bnd)
        assert ok, ("noalloc wgrad", rep)

    # Call 2: a smaller forward GEMM, Y [300, 256] over K = 384, FP32 and BF16.
    M2, N2, K2 = 300, 256, 384
    xb2 = W.normal_bf16((M2, K2), 1.0, W.seed_for(94, 1, "o", "x"))
    wb2 = W.normal_bf16((N2, K2), 0.02, W.seed_for(94, 1, "o", "w"))
    xq, sx = B.fp8_quant_1x128(dev_bf16(xb2))
    wq, sw, _, _ = B.fp8_quant_128x128(dev_bf16(wb2))
    yr, bnd = gemm.fwd(*quant.quant_1x128_rows(xb2), *quant.quant_128x128(wb2))
    for od in (torch.float32, torch.bfloat16):
        say("noalloc split fwd", od, (M2, N2, K2))
        y1 = torch.empty((M2, N2), dtype=od, device="cuda")
        y2 = torch.empty((M2, N2), dtype=od, device="cuda")
        B.fp8_block_gemm_split2_noalloc(B.OP_FWD, xq, sx, wq, sw, M2, N2, K2, y1)
        B.fp8_block_gemm(B.OP_FWD, xq, sx, wq, sw, M2, N2, K2, y2, split2=True)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16 if od == torch.bfloat16 else torch.int32),
                           y2.view(torch.int16 if od == torch.bfloat16 else torch.int32))
        g2 = host(y1)
        ok, rep = compare.check_fp32(g2, yr, bnd) if od == torch.float32 else compare.check_bf16(g2, yr, bnd)
        assert ok, ("noalloc fwd", od, rep)

    # Beyond the scratch: refused with a clear status before anything runs.
    big = torch.empty((2048, 6144), dtype=torch.float32, device="cuda")
    xqT6 = torch.zeros((6144, M), dtype=torch.uint8, device="cuda")
    sxT6 = torch.zeros((M // 128, 6144), dtype=torch.float32, device="cuda")
    with pytest.raises(B._lib.Fp8BlkError, match="workspace too small"):
        B.fp8_block_gemm_split2_noalloc(B.OP_WGRAD, dyqT, sdyT, xqT6, sxT6, M, N, 6144, big)
