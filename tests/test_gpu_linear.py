"""GPU parity of the Fp8Linear module against the oracle.

One linear of the M=4096 layer shape family at a smaller token count: the
forward output, the data gradient and the FP32 weight gradient accumulated
over two micro-batches are checked element by element against the float64
oracle (same acceptance rule as the GEMM tests; with the FP8 matrix
instructions, the derived bound (2^-10 + 1e-5) * sum |a*b|), and the FP8
weight cache is checked to rebuild exactly when the weight changes.
"""

import numpy as np
import pytest

from blockwise_fp8_linear_quant_amd import workloads as W
from oracle import compare, gemm, quant
from tests.gpu_util import dev_bf16, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def _oracle_step(xb, wb, dyb):
    xq, sx = quant.quant_1x128_rows(xb)
    xqT, sxT = quant.quant_1x128_tokens(xb)
    wq, sw = quant.quant_128x128(wb)
    wqT, swT = quant.quant_128x128(np.ascontiguousarray(wb.T))
    dyq, sdy = quant.quant_1x128_rows(dyb)
    dyqT, sdyT = quant.quant_1x128_tokens(dyb)
    return (gemm.fwd(xq, sx, wq, sw), gemm.dgrad(dyq, sdy, wqT, swT), gemm.wgrad(dyqT, sdyT, xqT, sxT))


@pytest.mark.parametrize("mc,rtol", [(False, compare.FP32_RTOL), (True, 2.0 ** -10 + 1e-5)])
def test_fp8_linear_forward_backward_two_microbatches(torch_mod, mc, rtol):
    torch = torch_mod
    from blockwise_fp8_linear_quant_amd.linear import Fp8Linear
    M, K, N = 300, 256, 384          # ragged token count, several tiles
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(2, 1, "qkv", "w"))
    lin = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous(), fp8_matrix_core=mc)
    dw_sum = None
    bnd_sum = None
    for mb in range(2):
        xb = W.normal_bf16((M, K), 1.0, W.seed_for(2, 10 + mb, "qkv", "x"))
        dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(2, 10 + mb, "qkv", "dy"))
        x = dev_bf16(xb).contiguous().requires_grad_(True)
        say("Fp8Linear micro-batch", mb, M, K, N, "matrix core" if mc else "exact")
        y = lin(x)
        y.backward(dev_bf16(dyb).contiguous())
        torch.cuda.synchronize()
        (yy, yb), (dxx, dxb), (dww, dwb) = _oracle_step(xb, wb, dyb)
        ok, rep = compare.check_bf16(host(y.detach()), yy, yb, rtol=rtol)
        assert ok, ("forward", mb, rep)
        ok, rep = compare.check_bf16(host(x.grad), dxx, dxb, rtol=rtol)
        assert ok, ("dgrad", mb, rep)
        dw_sum = dww if dw_sum is None else dw_sum + dww
        bnd_sum = dwb if bnd_sum is None else bnd_sum + dwb
    ok, rep = compare.check_fp32(host(lin.weight.main_grad), dw_sum, bnd_sum, rtol=rtol)
    assert ok, ("wgrad accumulated", rep)
    assert lin.weight.grad is None
    assert lin.weight_quantisations == 1      # one FP8 weight for both micro-batches


def test_fp8_linear_weight_cache_follows_updates(torch_mod):
    torch = torch_mod
    from blockwise_fp8_linear_quant_amd.linear import Fp8Linear
    M, K, N = 128, 128, 256
    wb = W.normal_bf16((N, K), 0.02, 5)
    lin = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous())
    xb = W.normal_bf16((M, K), 1.0, 6)
    x = dev_bf16(xb).contiguous()
    say("Fp8Linear cache")
    with torch.no_grad():
        y0 = lin(x)
        y1 = lin(x)
        assert lin.weight_quantisations == 1
        lin.weight.mul_(2.0)                   # exact in BF16: codes unchanged, scales doubled
        y2 = lin(x)
    torch.cuda.synchronize()
    assert lin.weight_quantisations == 2
    assert torch.equal(y0, y1)
    assert torch.equal(y2.float(), (2.0 * y0.float()).to(torch.bfloat16).float())


def test_fp8_linear_weight_written_through_data(torch_mod):
    """A write through weight.data bypasses the version counter; after
    invalidate_weight_cache() the next forward uses the new weight, bit-equal to
    a fresh module built on it, and a backward reads the new transposed copy."""
    torch = torch_mod
    from blockwise_fp8_linear_quant_amd.linear import Fp8Linear
    M, K, N = 256, 256, 384
    wa, wb_ = W.normal_bf16((N, K), 0.02, 15), W.normal_bf16((N, K), 0.02, 16)
    xb = W.normal_bf16((M, K), 1.0, 17)
    dyb = W.normal_bf16((M, N), 1e-3, 18)
    x, dy = dev_bf16(xb).contiguous(), dev_bf16(dyb).contiguous()
    lin = Fp8Linear(K, N, weight=dev_bf16(wa).contiguous())
    fresh = Fp8Linear(K, N, weight=dev_bf16(wb_).contiguous())
    say("Fp8Linear weight.data write")
    with torch.no_grad():
        lin(x)
        lin.weight.data.copy_(dev_bf16(wb_))      # the version counter does not move
        lin.invalidate_weight_cache()
    xa = x.clone().requires_grad_(True)
    xf = x.clone().requires_grad_(True)
    ya, yf = lin(xa), fresh(xf)
    ya.backward(dy)
    yf.backward(dy)
    torch.cuda.synchronize()
    assert lin.weight_quantisations == 2
    assert torch.equal(ya, yf)
    assert torch.equal(xa.grad, xf.grad)
    assert torch.equal(lin.weight.main_grad, fresh.weight.main_grad)


def _rel(a, b):
    a, b = a.double(), b.double()
    return float((a - b).norm() / b.norm())


def test_fused_rmsnorm_linear(torch_mod):
    """forward_rmsnorm: forward bit-for-bit the oracle's fused RMSNorm value
    through the FP8 GEMM (acceptance rule as above); backward against the
    unfused composition F.rms_norm -> Fp8Linear (same FP8 data gradient, the
    RMSNorm backward by PyTorch autograd)."""
    torch = torch_mod
    import torch.nn.functional as F
    from blockwise_fp8_linear_quant_amd.linear import Fp8Linear
    from oracle import fused
    M, K, N = 300, 256, 384
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(2, 20, "qkv", "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(2, 20, "qkv", "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(2, 20, "qkv", "dy"))
    gam = (np.random.default_rng(5).standard_normal(K) * 0.1 + 1.0).astype(np.float32)
    gb = W.f32_to_bf16_bits(gam)
    gamma = torch.from_numpy(gb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    dy = dev_bf16(dyb).contiguous()
    say("fused rmsnorm linear", M, K, N)
    lin_f = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous())
    x1, g1 = dev_bf16(xb).contiguous().requires_grad_(True), gamma.clone().requires_grad_(True)
    y1 = lin_f.forward_rmsnorm(x1, g1, 1e-6)
    y1.backward(dy)
    lin_u = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous())
    x2, g2 = dev_bf16(xb).contiguous().requires_grad_(True), gamma.clone().requires_grad_(True)
    y2 = lin_u(F.rms_norm(x2, (K,), g2, 1e-6))
    y2.backward(dy)
    torch.cuda.synchronize()
    hb, _ = fused.rmsnorm_bf16(xb, gb, 1e-6)
    hq, sh = quant.quant_1x128_rows(hb)
    wq, sw = quant.quant_128x128(wb)
    yy, bnd = gemm.fwd(hq, sh, wq, sw)
    ok, rep = compare.check_bf16(host(y1.detach()), yy, bnd)
    assert ok, ("fused rmsnorm forward", rep)
    assert _rel(x1.grad, x2.grad) < 2e-2, _rel(x1.grad, x2.grad)
    assert _rel(g1.grad, g2.grad) < 2e-2, _rel(g1.grad, g2.grad)
    assert _rel(lin_f.weight.main_grad, lin_u.weight.main_grad) < 2e-2


def test_fused_swiglu_linear(torch_mod):
    """forward_swiglu: forward against the oracle's fused SwiGLU value through
    the FP8 GEMM; backward against F.silu(gate) * up -> Fp8Linear."""
    torch = torch_mod
    import torch.nn.functional as F
    from blockwise_fp8_linear_quant_amd.linear import Fp8Linear
    from oracle import fused
    M, K, N = 300, 256, 384
    gb_ = W.normal_bf16((M, K), 1.0, W.seed_for(2, 21, "down", "x"))
    ub_ = W.normal_bf16((M, K), 1.0, W.seed_for(2, 21, "down", "dy"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(2, 21, "down", "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(2, 22, "down", "dy"))
    gub = np.concatenate([gb_, ub_], axis=1)
    dy = dev_bf16(dyb).contiguous()
    say("fused swiglu linear", M, K, N)
    lin_f = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous())
    gu1 = dev_bf16(gub).contiguous().requires_grad_(True)
    y1 = lin_f.forward_swiglu(gu1)
    y1.backward(dy)
    lin_u = Fp8Linear(K, N, weight=dev_bf16(wb).contiguous())
    gu2 = dev_bf16(gub).contiguous().requires_grad_(True)
    g, u = gu2.split([K, K], dim=1)
    y2 = lin_u(F.silu(g) * u)
    y2.backward(dy)
    torch.cuda.synchronize()
    hb = fused.swiglu_bf16(gb_, ub_)
    hq, sh = quant.quant_1x128_rows(hb)
    wq, sw = quant.quant_128x128(wb)
    yy, bnd = gemm.fwd(hq, sh, wq, sw)
    ok, rep = compare.check_bf16(host(y1.detach()), yy, bnd)
    assert ok, ("fused swiglu forward", rep)
    assert _rel(gu1.grad, gu2.grad) < 2e-2, _rel(gu1.grad, gu2.grad)
    assert _rel(lin_f.weight.main_grad, lin_u.weight.main_grad) < 2e-2
