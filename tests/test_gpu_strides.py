"""GPU parity with every operand a view into a wider buffer.

Each input and output of the C ABI's quantisers and GEMMs is placed 16 bytes
into a buffer whose rows are longer than the view (leading dimension above
the width, padded to the alignment the header asks for).  The results must
match the oracle as for dense operands -- codes and scales bit-exact, GEMM
outputs within the FP32 tolerance or one BF16 ulp -- and nothing outside the
views may change: every buffer starts filled with a sentinel (0x7F codes,
NaN scales and outputs) that must survive around the view.  M = 300 gives a
ragged token tail; K = 384 and N = 256 span several 128-wide blocks and tiles.
The fused SwiGLU and RMSNorm producers get the same treatment for their
inputs, their BF16 value output and their four quantised outputs.
"""

import numpy as np
import pytest

from blockwise_fp8_linear_quant_amd import workloads as W
from oracle import compare, fused, gemm, quant
from tests.gpu_util import host, say

pytestmark = pytest.mark.gpu

M, K, N = 300, 384, 256
MP = 384                       # M padded to whole 128-token groups


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd import binding
    return binding


class Wide:
    """A [rows, cols] view 16 bytes into a [rows, ld] device buffer filled with `fill`."""

    def __init__(self, rows, cols, dtype, fill, extra=40):
        import torch
        esz = torch.empty((), dtype=dtype).element_size()
        per16 = 16 // esz
        self.off = per16
        self.ld = -(-(cols + self.off + extra) // per16) * per16
        self.cols = cols
        self.buf = torch.full((rows, self.ld), fill, dtype=dtype, device="cuda")
        self.view = self.buf[:, self.off:self.off + cols]
        self.fill = fill

    def upload(self, a):
        import torch
        self.view.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(self.buf.dtype))
        return self.view

    def outside_untouched(self):
        b = host(self.buf).astype(np.float64)
        outside = np.ones(b.shape, dtype=bool)
        outside[:, self.off:self.off + self.cols] = False
        v = b[outside]
        return bool(np.all(np.isnan(v))) if np.isnan(self.fill) else bool(np.all(v == self.fill))


def wide_bf16(bits):
    import torch
    w = Wide(bits.shape[0], bits.shape[1], torch.int16, 0)
    w.upload(bits.view(np.int16))
    return w.view.view(torch.bfloat16)


def codes(rows, cols):
    import torch
    return Wide(rows, cols, torch.uint8, 0x7F)


def f32(rows, cols):
    import torch
    return Wide(rows, cols, torch.float32, float("nan"))


def exact(got, ref, what):
    ok, n = compare.check_exact(np.ascontiguousarray(got), np.ascontiguousarray(ref))
    assert ok, (what, n)


def test_quantisers_on_strided_views(B):
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(95, M, K, "x"))
    oq, os_ = quant.quant_1x128_rows(xb)
    oqT, osT = quant.quant_1x128_tokens(xb)
    obq, obs = quant.quant_128x128(xb)
    obqT, _ = quant.quant_128x128(np.ascontiguousarray(xb.T))
    G, GT = K // 128, MP // 128

    say("strided row-wise quantiser", M, K)
    q, s = codes(M, K), f32(G, M)
    B.fp8_quant_1x128(wide_bf16(xb), q=q.view, scales=s.view)
    exact(host(q.view), oq, "rows q")
    exact(host(s.view), os_.T, "rows s")
    assert q.outside_untouched() and s.outside_untouched()

    say("strided token quantiser", M, K)
    qT, sT = codes(K, MP), f32(GT, K)
    B.fp8_quant_1x128(wide_bf16(xb), transpose_out=True, q=qT.view, scales=sT.view)
    got = host(qT.view)
    exact(got[:, :M], oqT, "tokens q")
    assert np.all(got[:, M:] == 0), "token pads"
    exact(host(sT.view), osT.T, "tokens s")
    assert qT.outside_untouched() and sT.outside_untouched()

    say("strided dual quantiser", M, K)
    q, s, qT, sT = codes(M, K), f32(G, M), codes(K, MP), f32(GT, K)
    B.fp8_quant_1x128_dual(wide_bf16(xb), q=q.view, scales=s.view, qT=qT.view, scalesT=sT.view)
    exact(host(q.view), oq, "dual q")
    exact(host(s.view), os_.T, "dual s")
    got = host(qT.view)
    exact(got[:, :M], oqT, "dual qT")
    assert np.all(got[:, M:] == 0), "dual pads"
    exact(host(sT.view), osT.T, "dual sT")
    for w in (q, s, qT, sT):
        assert w.outside_untouched()

    say("strided 128x128 quantiser", M, K)
    q, qT = codes(M, K), codes(K, M)
    _, bs, _, bsT = B.fp8_quant_128x128(wide_bf16(xb), with_transpose=True, q=q.view, qT=qT.view)
    exact(host(q.view), obq, "blocks q")
    exact(host(qT.view), obqT, "blocks qT")
    exact(host(bs), obs, "blocks s")
    exact(host(bsT), obs.T, "blocks sT")
    assert q.outside_untouched() and qT.outside_untouched()


@pytest.fixture(scope="module")
def operands():
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(96, M, K, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(96, N, K, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(96, M, N, "dy"))
    o = {}
    o["xq"], o["sx"] = quant.quant_1x128_rows(xb)
    o["wq"], o["sw"] = quant.quant_128x128(wb)
    o["wqT"], o["swT"] = quant.quant_128x128(np.ascontiguousarray(wb.T))
    o["dyq"], o["sdy"] = quant.quant_1x128_rows(dyb)
    o["xqT"], o["sxT"] = quant.quant_1x128_tokens(xb)
    o["dyqT"], o["sdyT"] = quant.quant_1x128_tokens(dyb)
    return o


def _padded_tokens(cT):
    out = np.zeros((cT.shape[0], MP), dtype=np.uint8)
    out[:, :M] = cT
    return out


def test_fwd_and_dgrad_on_strided_views(B, operands):
    import torch
    o = operands
    xq = codes(M, K).upload(o["xq"])
    sx = f32(K // 128, M).upload(o["sx"].T)
    wq = codes(N, K).upload(o["wq"])
    sw = torch.from_numpy(o["sw"]).cuda()
    want, bnd = gemm.fwd(o["xq"], o["sx"], o["wq"], o["sw"])

    say("strided fwd FP32", M, N, K)
    y = f32(M, N)
    B.fp8_block_gemm_fwd(xq, sx, wq, sw, y=y.view)
    ok, rep = compare.check_fp32(host(y.view), want, bnd)
    assert ok, rep
    assert y.outside_untouched()

    say("strided fwd BF16", M, N, K)
    yb = Wide(M, N, torch.int16, 0x7FC1)              # a BF16 NaN pattern as the sentinel
    B.fp8_block_gemm_fwd(xq, sx, wq, sw, y=yb.view.view(torch.bfloat16))
    ok, rep = compare.check_bf16(host(yb.view).view(np.uint16), want, bnd)
    assert ok, rep
    assert yb.outside_untouched()

    say("strided dgrad FP32", M, N, K)
    dyq = codes(M, N).upload(o["dyq"])
    sdy = f32(N // 128, M).upload(o["sdy"].T)
    wqT = codes(K, N).upload(o["wqT"])
    swT = torch.from_numpy(o["swT"]).cuda()
    dx = f32(M, K)
    B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, dx=dx.view)
    want, bnd = gemm.dgrad(o["dyq"], o["sdy"], o["wqT"], o["swT"])
    ok, rep = compare.check_fp32(host(dx.view), want, bnd)
    assert ok, rep
    assert dx.outside_untouched()


def test_wgrad_on_strided_views(B, operands):
    o = operands
    GT = MP // 128
    dyqT = codes(N, MP).upload(_padded_tokens(o["dyqT"]))
    sdyT = f32(GT, N).upload(o["sdyT"].T)
    xqT = codes(K, MP).upload(_padded_tokens(o["xqT"]))
    sxT = f32(GT, K).upload(o["sxT"].T)
    want, bnd = gemm.wgrad(o["dyqT"], o["sdyT"], o["xqT"], o["sxT"])

    say("strided wgrad FP32", M, N, K)
    dw = f32(N, K)
    B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=dw.view)
    ok, rep = compare.check_fp32(host(dw.view), want, bnd)
    assert ok, rep
    assert dw.outside_untouched()

    say("strided wgrad accumulate", M, N, K)
    dw.view.copy_(dw.view * 0.5)                       # dW0 = Y / 2, exact
    dw0 = host(dw.view).astype(np.float64)
    B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=dw.view, accumulate=True)
    got = host(dw.view)
    ok, rep = compare.check_fp32(got, want + dw0, bnd + np.abs(dw0) * 2.0 ** -14)
    assert ok, rep
    assert dw.outside_untouched()


def _ulp_diff(a_bits, b_bits):
    """|a - b| in BF16 ulps (order-preserving integer map of the bit patterns)."""
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))


def _check_dual_of(h_bits, q, s, qT, sT, label):
    """The four wide outputs hold the oracle's two 1x128 quantisations of h_bits."""
    oq, os_ = quant.quant_1x128_rows(h_bits)
    oqT, osT = quant.quant_1x128_tokens(h_bits)
    exact(host(q.view), oq, label + " q")
    exact(host(s.view), os_.T, label + " s")
    got = host(qT.view)
    exact(got[:, :M], oqT, label + " qT")
    assert np.all(got[:, M:] == 0), label + " pads"
    exact(host(sT.view), osT.T, label + " sT")
    for w in (q, s, qT, sT):
        assert w.outside_untouched(), label


def _dual_outputs(C):
    return codes(M, C), f32(C // 128, M), codes(C, MP), f32(MP // 128, C)


def test_fused_producers_on_strided_views(B):
    import torch
    C = K
    g = W.normal_bf16((M, C), 1.0, W.seed_for(97, M, C, "x"))
    u = W.normal_bf16((M, C), 1.0, W.seed_for(97, M, C, "dy"))
    say("strided swiglu producer", M, C)
    hw = Wide(M, C, torch.int16, 0x7FC1)
    q, s, qT, sT = _dual_outputs(C)
    B.fp8_swiglu_quant_1x128_dual(wide_bf16(g), wide_bf16(u), h_out=hw.view.view(torch.bfloat16),
                                  q=q.view, scales=s.view, qT=qT.view, scalesT=sT.view)
    h = host(hw.view).view(np.uint16)
    assert _ulp_diff(h, fused.swiglu_bf16(g, u)).max() <= 1
    assert hw.outside_untouched()
    _check_dual_of(h, q, s, qT, sT, "swiglu")

    x = W.normal_bf16((M, C), 1.0, W.seed_for(97, M, C, "w"))
    gam = W.f32_to_bf16_bits((np.random.default_rng(97).standard_normal(C) * 0.1 + 1.0).astype(np.float32))
    gdev = torch.from_numpy(gam.view(np.int16)).cuda().view(torch.bfloat16)
    say("strided rmsnorm producer", M, C)
    yw = Wide(M, C, torch.int16, 0x7FC1)
    q, s, qT, sT = _dual_outputs(C)
    B.fp8_rmsnorm_quant_1x128_dual(wide_bf16(x), gdev, 1e-6, y_out=yw.view.view(torch.bfloat16),
                                   q=q.view, scales=s.view, qT=qT.view, scalesT=sT.view)
    y = host(yw.view).view(np.uint16)
    want, _ = fused.rmsnorm_bf16(x, gam, 1e-6)
    assert _ulp_diff(y, want).max() <= 1
    assert yw.outside_untouched()
    _check_dual_of(y, q, s, qT, sT, "rmsnorm")
