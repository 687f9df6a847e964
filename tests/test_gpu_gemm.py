"""GPU parity of the block-scaled FP8 GEMMs (forward, dgrad, wgrad).

FP32 outputs: |gpu - Y| <= 1e-5 * sum|a*b| + 1e-6 elementwise (Y, budget from
the float64 oracle).  BF16 outputs: within one BF16 ulp of the rounded oracle
value, or inside the FP32 budget where cancellation makes |Y| tiny.
Lossless inputs must agree bit-for-bit.  Small shapes (several tiles, ragged
tails) are checked on every element; the workload sizes are checked on
sampled rows and columns, which the oracle computes one by one.
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


def _torch():
    import torch
    return torch


class Layer:
    """One linear layer's BF16 tensors, their GPU quantisations and the oracle's."""

    def __init__(self, B, xb, wb, dyb):
        self.B, self.xb, self.wb, self.dyb = B, xb, wb, dyb
        self.M, self.K = xb.shape
        self.N = wb.shape[0]
        self.x, self.w = dev_bf16(xb), dev_bf16(wb)
        self.dy = dev_bf16(dyb) if dyb is not None else None

    def fwd(self, out_dtype):
        B = self.B
        xq, sx = B.fp8_quant_1x128(self.x)
        wq, sw, _, _ = B.fp8_quant_128x128(self.w)
        y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=out_dtype)
        oxq, osx = quant.quant_1x128_rows(self.xb)
        owq, osw = quant.quant_128x128(self.wb)
        return host(y), (lambda rows=None, cols=None: gemm.fwd(oxq, osx, owq, osw, rows, cols))

    def dgrad(self, out_dtype):
        B = self.B
        dyq, sdy = B.fp8_quant_1x128(self.dy)
        _, _, wqT, swT = B.fp8_quant_128x128(self.w, with_transpose=True)
        dx = B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=out_dtype)
        odyq, osdy = quant.quant_1x128_rows(self.dyb)
        owqT, oswT = quant.quant_128x128(np.ascontiguousarray(self.wb.T))
        return host(dx), (lambda rows=None, cols=None: gemm.dgrad(odyq, osdy, owqT, oswT, rows, cols))

    def wgrad(self, accumulate=False, dw0=None):
        B = self.B
        torch = _torch()
        dyqT, sdyT = B.fp8_quant_1x128(self.dy, transpose_out=True)
        xqT, sxT = B.fp8_quant_1x128(self.x, transpose_out=True)
        dw = None
        if accumulate:
            dw = torch.from_numpy(dw0).cuda()
        dw = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=self.M, dw=dw, accumulate=accumulate)
        odyqT, osdyT = quant.quant_1x128_tokens(self.dyb)
        oxqT, osxT = quant.quant_1x128_tokens(self.xb)
        return host(dw), (lambda rows=None, cols=None: gemm.wgrad(odyqT, osdyT, oxqT, osxT, rows, cols))


def check_full(got, ref_fn, out, label, base=None):
    y, bnd = ref_fn()
    if base is not None:
        y = y + base
    if out == "bf16":
        ok, rep = compare.check_bf16(got, y, bnd)
    else:
        ok, rep = compare.check_fp32(got, y, bnd)
    assert ok, f"{label}: {rep}"
    return rep


def check_sampled(got, ref_fn, out, label, rng, k=40):
    I, J = got.shape
    rows = sample_index(I, k, rng, must=(0, I - 1, I // 2, (I // 128) * 128 - 1))
    cols = sample_index(J, k, rng, must=(0, J - 1, 127, 128))
    for sel_r, sel_c in ((rows, None), (None, cols)):
        y, bnd = ref_fn(sel_r, sel_c)
        g = got[sel_r] if sel_r is not None else got[:, sel_c]
        if out == "bf16":
            ok, rep = compare.check_bf16(g, y, bnd)
        else:
            ok, rep = compare.check_fp32(g, y, bnd)
        assert ok, f"{label}: {rep}"


# ---------------------------------------------------------------------------


def _lossless(rng, shape, exps):
    R, L = shape
    k = rng.integers(0, 4, size=shape)
    v = rng.choice([-1.0, 1.0], size=shape) * 448.0 * np.ldexp(1.0, -k)
    v[:, ::128] = 448.0
    v = v * np.ldexp(1.0, np.repeat(exps, 128, axis=1)[:, :L])
    return W.f32_to_bf16_bits(v.astype(np.float32))


def test_lossless_family_bit_exact(B):
    """Lossless quantisation and an FP32-representable result: bit-exact for any summation order.

    Every group holds values from {+-448 * 2^-k, k = 0..3} times 2^j with one
    448 * 2^j, so s = 2^j exactly and codes are exact.  Exponents vary per row
    and block within a 2-binade window, so every partial and every running sum
    of the GPU's accumulation fits in 24 bits.
    """
    rng = np.random.default_rng(1)
    M, N, K = 160, 256, 384
    xb = _lossless(rng, (M, K), rng.integers(-1, 1, size=(M, 3)))
    wv = rng.choice([-1.0, 1.0], size=(N, K)) * 448.0 * np.ldexp(1.0, -rng.integers(0, 4, size=(N, K)))
    for bn in range(N // 128):
        for bk in range(K // 128):
            j = int(rng.integers(-8, -6))
            wv[bn * 128, bk * 128] = 448.0
            wv[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128] *= 2.0 ** j
    wb = W.f32_to_bf16_bits(wv.astype(np.float32))
    L = Layer(B, xb, wb, None)
    say("gemm lossless fwd f32", (M, N, K))
    got, ref = L.fwd(_torch().float32)
    y, _ = ref()
    assert np.array_equal(y.astype(np.float32).astype(np.float64), y), "test data must give FP32-exact sums"
    assert np.array_equal(got.astype(np.float64), y), "lossless family must be bit-exact"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 256, 128), (128, 128, 384), (300, 384, 256),
                                   (257, 512, 640), (1000, 256, 1024)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fwd_dgrad_small(B, M, N, K, out):
    torch = _torch()
    od = torch.float32 if out == "f32" else torch.bfloat16
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(91, M, 0, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(91, M, 0, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(91, M, 0, "dy"))
    L = Layer(B, xb, wb, dyb)
    say("gemm fwd", out, (M, N, K))
    got, ref = L.fwd(od)
    check_full(got, ref, out, f"fwd {M}x{N}x{K}")
    say("gemm dgrad", out, (M, N, K))
    got, ref = L.dgrad(od)
    check_full(got, ref, out, f"dgrad {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (100, 256, 128), (128, 128, 384), (300, 384, 256),
                                   (1000, 256, 512)])
def test_wgrad_small(B, M, N, K):
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(92, M, 0, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(92, M, 0, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(92, M, 0, "dy"))
    L = Layer(B, xb, wb, dyb)
    say("gemm wgrad", (M, N, K))
    got, ref = L.wgrad()
    check_full(got, ref, "f32", f"wgrad {M}x{N}x{K}")
    dw0 = np.random.default_rng(M).standard_normal((N, K)).astype(np.float32) * 1e-3
    say("gemm wgrad accumulate", (M, N, K))
    got, ref = L.wgrad(accumulate=True, dw0=dw0)
    y, bnd = ref()
    # The FP32 add of the old value rounds once: half an ulp of the sum, within 2^-23 |dW0| + the budget.
    ok, rep = compare.check_fp32(got, y + dw0.astype(np.float64), bnd + np.abs(dw0) * (2.0 ** -23 / compare.FP32_RTOL))
    assert ok, rep


def test_config1_full(B):
    """Configuration 1: X [256, 2048] ~ N(0,1), W [2048, 2048] ~ N(0, 0.02), Y FP32, every element."""
    torch = _torch()
    xb = W.normal_bf16((256, 2048), 1.0, W.seed_for(1, 0, "o", "x"))
    wb = W.normal_bf16((2048, 2048), 0.02, W.seed_for(1, 0, "o", "w"))
    L = Layer(B, xb, wb, None)
    say("gemm cfg1 fwd f32 full")
    got, ref = L.fwd(torch.float32)
    rep = check_full(got, ref, "f32", "cfg1")
    assert rep["worst"] < 0.5


@pytest.mark.parametrize("lin", [n for n, _, _ in W.LINEARS])
def test_layer_M4096(B, lin):
    """Configurations 2 and 3: fwd (BF16 out), dgrad (BF16), wgrad (FP32) at 4096 tokens."""
    torch = _torch()
    _, k, n = [l for l in W.LINEARS if l[0] == lin][0]
    xb = W.normal_bf16((4096, k), 1.0, W.seed_for(2, 0, lin, "x"))
    wb = W.normal_bf16((n, k), 0.02, W.seed_for(2, 0, lin, "w"))
    dyb = W.normal_bf16((4096, n), 1e-3, W.seed_for(2, 0, lin, "dy"))
    L = Layer(B, xb, wb, dyb)
    rng = np.random.default_rng(hash(lin) % 2 ** 32)
    say("gemm layer fwd", lin)
    got, ref = L.fwd(torch.bfloat16)
    check_sampled(got, ref, "bf16", f"{lin} fwd", rng)
    say("gemm layer dgrad", lin)
    got, ref = L.dgrad(torch.bfloat16)
    check_sampled(got, ref, "bf16", f"{lin} dgrad", rng)
    say("gemm layer wgrad", lin)
    got, ref = L.wgrad()
    check_sampled(got, ref, "f32", f"{lin} wgrad", rng)


@pytest.mark.parametrize("layer", [0, 27])
@pytest.mark.parametrize("lin", [n for n, _, _ in W.LINEARS])
def test_outliers_M8192(B, layer, lin):
    """Configuration 4: the first and last layers' four linears at 8192 tokens, 1% of
    input channels x32 -- fwd (BF16), dgrad (BF16) and wgrad (FP32) on sampled rows
    and columns."""
    torch = _torch()
    xb, wb, dyb = W.layer_tensors(4, layer, lin, 8192, outliers=True)
    L = Layer(B, xb, wb, dyb)
    rng = np.random.default_rng(4000 + layer)
    say("gemm cfg4 fwd", layer, lin)
    got, ref = L.fwd(torch.bfloat16)
    check_sampled(got, ref, "bf16", f"cfg4 L{layer} {lin} fwd", rng, k=24)
    say("gemm cfg4 dgrad", layer, lin)
    got, ref = L.dgrad(torch.bfloat16)
    check_sampled(got, ref, "bf16", f"cfg4 L{layer} {lin} dgrad", rng, k=24)
    say("gemm cfg4 wgrad", layer, lin)
    got, ref = L.wgrad()
    check_sampled(got, ref, "f32", f"cfg4 L{layer} {lin} wgrad", rng, k=24)


def test_stress_ragged_M3000(B):
    """Configuration 5: down-projection, 3000 tokens, fwd (BF16) + wgrad (FP32, 56-token tail group)."""
    torch = _torch()
    xb = W.student_t_stress((3000, 6144), W.seed_for(5, 0, "down", "x"))
    wb = W.normal_bf16((2048, 6144), 0.02, W.seed_for(5, 0, "down", "w"))
    dyb = W.normal_bf16((3000, 2048), 1e-3, W.seed_for(5, 0, "down", "dy"))
    L = Layer(B, xb, wb, dyb)
    rng = np.random.default_rng(5)
    say("gemm cfg5 fwd")
    got, ref = L.fwd(torch.bfloat16)
    check_sampled(got, ref, "bf16", "cfg5 fwd", rng, k=64)
    say("gemm cfg5 wgrad")
    got, ref = L.wgrad()
    check_sampled(got, ref, "f32", "cfg5 wgrad", rng, k=64)


def test_empty_contraction_and_empty_outputs(B):
    torch = _torch()
    dev = "cuda:0"
    # M = 0 tokens: wgrad overwrite writes zeros, accumulate leaves dW unchanged.
    dyqT = torch.zeros((256, 0), dtype=torch.uint8, device=dev)
    xqT = torch.zeros((128, 0), dtype=torch.uint8, device=dev)
    s1 = torch.zeros((0, 256), dtype=torch.float32, device=dev)
    s2 = torch.zeros((0, 128), dtype=torch.float32, device=dev)
    dw = torch.full((256, 128), 3.0, device=dev)
    B.fp8_block_gemm_wgrad(dyqT, s1, xqT, s2, M=0, dw=dw, accumulate=True)
    assert torch.all(dw == 3.0)
    B.fp8_block_gemm_wgrad(dyqT, s1, xqT, s2, M=0, dw=dw, accumulate=False)
    assert torch.all(dw == 0.0)
    # M = 0 rows in the forward: nothing to do, no error.
    xq = torch.zeros((0, 128), dtype=torch.uint8, device=dev)
    sx = torch.zeros((1, 0), dtype=torch.float32, device=dev)
    wq = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    sw = torch.zeros((1, 1), dtype=torch.float32, device=dev)
    y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.float32)
    assert y.shape == (0, 128)


@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (1000, 1024, 256)])
def test_two_k_groups_unsplit(B, M, N, K):
    """Without a workspace, a grid of at most one 128 x 128 tile per CU whose
    contraction has an even number of 128-blocks runs as two K groups of four
    waves, each over half the blocks, summed before the epilogue.  (1000, 1024,
    256) takes that kernel in all three GEMMs; (300, 384, 512) in the forward
    only (odd block counts elsewhere take the 4-wave tiles).  Every element of
    the BF16 forward, the FP32 dgrad and the wgrad (overwrite and accumulate)."""
    torch = _torch()
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(97, M, 0, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(97, M, 0, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(97, M, 0, "dy"))
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    xq, sx = B.fp8_quant_1x128(x)
    wq, sw, wqT, swT = B.fp8_quant_128x128(w, with_transpose=True)
    dyq, sdy = B.fp8_quant_1x128(dy)
    dyqT, sdyT = B.fp8_quant_1x128(dy, transpose_out=True)
    xqT, sxT = B.fp8_quant_1x128(x, transpose_out=True)
    oxq, osx = quant.quant_1x128_rows(xb)
    owq, osw = quant.quant_128x128(wb)
    owqT, oswT = quant.quant_128x128(np.ascontiguousarray(wb.T))
    odyq, osdy = quant.quant_1x128_rows(dyb)
    odyqT, osdyT = quant.quant_1x128_tokens(dyb)
    oxqT, osxT = quant.quant_1x128_tokens(xb)
    say("gemm two K groups fwd", (M, N, K))
    y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16, workspace=False)
    check_full(host(y), lambda: gemm.fwd(oxq, osx, owq, osw), "bf16", f"fwd {M}x{N}x{K}")
    say("gemm two K groups dgrad", (M, N, K))
    dx = B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=torch.float32, workspace=False)
    check_full(host(dx), lambda: gemm.dgrad(odyq, osdy, owqT, oswT), "f32", f"dgrad {M}x{N}x{K}")
    say("gemm two K groups wgrad", (M, N, K))
    ref = lambda: gemm.wgrad(odyqT, osdyT, oxqT, osxT)
    dw = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, workspace=False)
    check_full(host(dw), ref, "f32", f"wgrad {M}x{N}x{K}")
    dw0 = np.random.default_rng(M + 7).standard_normal((N, K)).astype(np.float32) * 1e-3
    dwa = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=torch.from_numpy(dw0).cuda(), accumulate=True,
                                 workspace=False)
    yv, bnd = ref()
    ok, rep = compare.check_fp32(host(dwa), yv + dw0.astype(np.float64),
                                 bnd + np.abs(dw0) * (2.0 ** -23 / compare.FP32_RTOL))
    assert ok, f"wgrad accumulate {M}x{N}x{K}: {rep}"


@pytest.mark.parametrize("nblk", [1, 2, 3])
def test_big_tiles_short_contractions(B, nblk):
    """256 x 128 tiles (one full round of 16 x 16 tiles) with contractions of 1,
    2 and 3 scale blocks, where the software pipeline's prologue and its
    last-block guards decide what is read and converted: the forward GEMM
    (K = 128 nblk) in BF16 and the data gradient (N = 128 nblk) in FP32 over
    4000 ragged rows, and the weight gradient of a 4096 x 2048 weight over
    128 nblk - 28 tokens (a ragged last token group), every element against the
    oracle."""
    torch = _torch()
    M, D = 4000, 2048
    for lin, (name, N, K) in enumerate((("fwd", D, 128 * nblk), ("dgrad", 128 * nblk, D))):
        xb = W.normal_bf16((M, K), 1.0, W.seed_for(98, nblk, lin, "x"))
        wb = W.normal_bf16((N, K), 0.02, W.seed_for(98, nblk, lin, "w"))
        dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(98, nblk, lin, "dy"))
        L = Layer(B, xb, wb, dyb)
        say("gemm big tiles", name, (M, N, K))
        if name == "fwd":
            got, ref = L.fwd(torch.bfloat16)
            check_full(got, ref, "bf16", f"fwd {M}x{N}x{K}")
        else:
            got, ref = L.dgrad(torch.float32)
            check_full(got, ref, "f32", f"dgrad {M}x{N}x{K}")
    T, N, K = 128 * nblk - 28, 4096, D
    xb = W.normal_bf16((T, K), 1.0, W.seed_for(98, nblk, 2, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(98, nblk, 2, "w"))
    dyb = W.normal_bf16((T, N), 1e-3, W.seed_for(98, nblk, 2, "dy"))
    say("gemm big tiles wgrad", (T, N, K))
    got, ref = Layer(B, xb, wb, dyb).wgrad()
    check_full(got, ref, "f32", f"wgrad {N}x{K} over {T}")


def test_determinism(B):
    torch = _torch()
    xb = W.normal_bf16((512, 1024), 1.0, 8)
    wb = W.normal_bf16((768, 1024), 0.02, 9)
    L = Layer(B, xb, wb, None)
    a, _ = L.fwd(torch.float32)
    b, _ = L.fwd(torch.float32)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_every_code_through_both_operands(B):
    """All 254 finite E4M3 codes pass exactly through the A and the B operand.

    Codes are placed by hand (no quantiser): Y[r, n] = D(code_r) * D(code_n)
    with unit scales, exact in FP32.
    """
    torch = _torch()
    from oracle import e4m3
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    R = 256
    xq = np.zeros((R, 128), dtype=np.uint8)
    xq[:len(codes), 0] = codes
    xq[:len(codes), 77] = 0x38                 # + D(code_r) * D(code_n') at a second position
    wq = np.zeros((256, 128), dtype=np.uint8)
    wq[:len(codes), 0] = codes
    wq[:, 77] = 0x30                           # 0.5
    sx = np.ones((1, R), dtype=np.float32)
    sw = np.ones((2, 1), dtype=np.float32)
    d = lambda a: torch.from_numpy(a).cuda()
    say("gemm every code")
    y = host(B.fp8_block_gemm_fwd(d(xq), d(sx), d(wq), d(sw), out_dtype=torch.float32))
    dx = e4m3.decode(xq).astype(np.float64)
    dw = e4m3.decode(wq).astype(np.float64)
    ref = dx @ dw.T
    assert np.array_equal(y.astype(np.float64), ref)


# --- the FP8 matrix-core path (fp8_block_gemm with FP8BLK_GEMM_FP8_MATRIX_CORE) ---
# Its block products carry the hardware's in-group truncation: at most 7 of 8
# products of a group lose bits below 2^-13 of the group's largest product, so
# per block |err| <= 7 * 2^-13 * sum|p| and overall |err| <= 2^-10 * sum|a*b|
# plus the FP32 accumulation term.  On Gaussian operands it also meets the
# exact-block tolerance, which is checked where it holds.
FP8_PATH_RTOL = 2.0 ** -10 + 1e-5


class FastLayer(Layer):
    def fwd(self, out_dtype):
        B = self.B
        xq, sx = B.fp8_quant_1x128(self.x)
        wq, sw, _, _ = B.fp8_quant_128x128(self.w)
        y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=out_dtype, fp8_matrix_core=True)
        oxq, osx = quant.quant_1x128_rows(self.xb)
        owq, osw = quant.quant_128x128(self.wb)
        return host(y), (lambda rows=None, cols=None: gemm.fwd(oxq, osx, owq, osw, rows, cols))

    def dgrad(self, out_dtype):
        B = self.B
        dyq, sdy = B.fp8_quant_1x128(self.dy)
        _, _, wqT, swT = B.fp8_quant_128x128(self.w, with_transpose=True)
        dx = B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=out_dtype, fp8_matrix_core=True)
        odyq, osdy = quant.quant_1x128_rows(self.dyb)
        owqT, oswT = quant.quant_128x128(np.ascontiguousarray(self.wb.T))
        return host(dx), (lambda rows=None, cols=None: gemm.dgrad(odyq, osdy, owqT, oswT, rows, cols))

    def wgrad(self, accumulate=False, dw0=None):
        B = self.B
        torch = _torch()
        dyqT, sdyT = B.fp8_quant_1x128(self.dy, transpose_out=True)
        xqT, sxT = B.fp8_quant_1x128(self.x, transpose_out=True)
        dw = torch.from_numpy(dw0).cuda() if accumulate else None
        dw = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=self.M, dw=dw, accumulate=accumulate,
                                    fp8_matrix_core=True)
        odyqT, osdyT = quant.quant_1x128_tokens(self.dyb)
        oxqT, osxT = quant.quant_1x128_tokens(self.xb)
        return host(dw), (lambda rows=None, cols=None: gemm.wgrad(odyqT, osdyT, oxqT, osxT, rows, cols))


def _check_fp32_rtol(got, ref_fn, rtol, label, rng=None, k=40):
    if rng is None:
        y, bnd = ref_fn()
        ok, rep = compare.check_fp32(got, y, bnd, rtol=rtol)
        assert ok, f"{label}: {rep}"
        return
    I, J = got.shape
    rows = sample_index(I, k, rng, must=(0, I - 1))
    y, bnd = ref_fn(rows, None)
    ok, rep = compare.check_fp32(got[rows], y, bnd, rtol=rtol)
    assert ok, f"{label}: {rep}"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (300, 384, 256), (1000, 256, 1024)])
def test_fp8_matrix_core_small_gaussian(B, M, N, K):
    torch = _torch()
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(93, M, 0, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(93, M, 0, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(93, M, 0, "dy"))
    L = FastLayer(B, xb, wb, dyb)
    say("fp8 path fwd/dgrad/wgrad", (M, N, K))
    got, ref = L.fwd(torch.float32)
    _check_fp32_rtol(got, ref, FP8_PATH_RTOL, "fp8 fwd")
    got, ref = L.dgrad(torch.float32)
    _check_fp32_rtol(got, ref, FP8_PATH_RTOL, "fp8 dgrad")
    got, ref = L.wgrad()
    _check_fp32_rtol(got, ref, FP8_PATH_RTOL, "fp8 wgrad")
    # BF16 outputs and the accumulating weight gradient (the other epilogue branches)
    for name, fn in (("fp8 fwd bf16", L.fwd), ("fp8 dgrad bf16", L.dgrad)):
        got, ref = fn(torch.bfloat16)
        y, bnd = ref()
        ok, rep = compare.check_bf16(got, y, bnd, rtol=FP8_PATH_RTOL)
        assert ok, f"{name}: {rep}"
    dw0 = np.random.default_rng(5).standard_normal((N, K)).astype(np.float32)
    got, ref = L.wgrad(accumulate=True, dw0=dw0)
    y, bnd = ref()
    # the final FP32 add dW + Y rounds once: 2^-24 |dW| = FP8_PATH_RTOL-scaled 2^-14 |dW| at most
    ok, rep = compare.check_fp32(got, y + dw0, bnd + np.abs(dw0) * 2.0 ** -14, rtol=FP8_PATH_RTOL)
    assert ok, f"fp8 wgrad accumulate: {rep}"


@pytest.mark.parametrize("nblk", [1, 3])
def test_fp8_matrix_core_big_tiles_short_contractions(B, nblk):
    """The FP8 matrix path on 256 x 128 tiles with contractions of 1 and 3 scale
    blocks (forward and data gradient over 4000 ragged rows, weight gradient over
    128 nblk - 28 tokens), every element against the derived bound."""
    torch = _torch()
    M, D = 4000, 2048
    for lin, (name, N, K) in enumerate((("fwd", D, 128 * nblk), ("dgrad", 128 * nblk, D))):
        xb = W.normal_bf16((M, K), 1.0, W.seed_for(99, nblk, lin, "x"))
        wb = W.normal_bf16((N, K), 0.02, W.seed_for(99, nblk, lin, "w"))
        dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(99, nblk, lin, "dy"))
        L = FastLayer(B, xb, wb, dyb)
        say("fp8 path big tiles", name, (M, N, K))
        got, ref = (L.fwd if name == "fwd" else L.dgrad)(torch.float32)
        _check_fp32_rtol(got, ref, FP8_PATH_RTOL, f"fp8 {name} {M}x{N}x{K}")
    T, N, K = 128 * nblk - 28, 4096, D
    xb = W.normal_bf16((T, K), 1.0, W.seed_for(99, nblk, 2, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(99, nblk, 2, "w"))
    dyb = W.normal_bf16((T, N), 1e-3, W.seed_for(99, nblk, 2, "dy"))
    say("fp8 path big tiles wgrad", (T, N, K))
    got, ref = FastLayer(B, xb, wb, dyb).wgrad()
    _check_fp32_rtol(got, ref, FP8_PATH_RTOL, f"fp8 wgrad {N}x{K} over {T}")


def test_fp8_matrix_core_config1_exact_tolerance(B):
    """On configuration 1 (Gaussian) the FP8 path also meets the exact-block tolerance."""
    torch = _torch()
    xb = W.normal_bf16((256, 2048), 1.0, W.seed_for(1, 0, "o", "x"))
    wb = W.normal_bf16((2048, 2048), 0.02, W.seed_for(1, 0, "o", "w"))
    L = FastLayer(B, xb, wb, None)
    say("fp8 path cfg1")
    got, ref = L.fwd(torch.float32)
    check_full(got, ref, "f32", "fp8 path cfg1")


def test_fp8_matrix_core_stress_M3000(B):
    """Configuration 5 on the FP8 path: within the derived in-group truncation bound."""
    xb = W.student_t_stress((3000, 6144), W.seed_for(5, 0, "down", "x"))
    wb = W.normal_bf16((2048, 6144), 0.02, W.seed_for(5, 0, "down", "w"))
    dyb = W.normal_bf16((3000, 2048), 1e-3, W.seed_for(5, 0, "down", "dy"))
    L = FastLayer(B, xb, wb, dyb)
    rng = np.random.default_rng(55)
    say("fp8 path cfg5 wgrad")
    got, ref = L.wgrad()
    _check_fp32_rtol(got, ref, FP8_PATH_RTOL, "fp8 cfg5 wgrad", rng)


# ---------------------------------------------------------------------------
# Split-K: the contraction split in two, each half's FP32 partial tile stored in
# the workspace and added by the half that finishes second, in split order.


def _split_layer(B, M, N, K, seed):
    xb = W.normal_bf16((M, K), 1.0, W.seed_for(93, seed, 0, "x"))
    wb = W.normal_bf16((N, K), 0.02, W.seed_for(93, seed, 0, "w"))
    dyb = W.normal_bf16((M, N), 1e-3, W.seed_for(93, seed, 0, "dy"))
    return Layer(B, xb, wb, dyb)


@pytest.mark.parametrize("M,N,K", [(300, 256, 384), (1000, 384, 2048), (129, 128, 256)])
@pytest.mark.parametrize("mc", [False, True])
def test_split_k_forced_small(B, M, N, K, mc):
    """Forced split (FP8BLK_GEMM_SPLIT2) on shapes the oracle checks in full: forward
    (FP32 and BF16), data gradient and weight gradient (overwrite and accumulate)."""
    torch = _torch()
    L = _split_layer(B, M, N, K, M)
    rtol = 2.0 ** -10 + 1e-5 if mc else compare.FP32_RTOL
    xq, sx = B.fp8_quant_1x128(L.x)
    wq, sw, wqT, swT = B.fp8_quant_128x128(L.w, with_transpose=True)
    dyq, sdy, dyqT, sdyT = B.fp8_quant_1x128_dual(L.dy)
    xqT, sxT = B.fp8_quant_1x128(L.x, transpose_out=True)
    oxq, osx = quant.quant_1x128_rows(L.xb)
    owq, osw = quant.quant_128x128(L.wb)
    odyq, osdy = quant.quant_1x128_rows(L.dyb)
    owqT, oswT = quant.quant_128x128(np.ascontiguousarray(L.wb.T))
    odyqT, osdyT = quant.quant_1x128_tokens(L.dyb)
    oxqT, osxT = quant.quant_1x128_tokens(L.xb)
    for od, out in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        say("split-k forced fwd", out, mc, (M, N, K))
        y = host(B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=od, fp8_matrix_core=mc, split2=True))
        yr, bnd = gemm.fwd(oxq, osx, owq, osw)
        ok, rep = (compare.check_fp32(y, yr, bnd, rtol=rtol) if out == "f32"
                   else compare.check_bf16(y, yr, bnd, rtol=rtol))
        assert ok, ("fwd", out, rep)
    say("split-k forced dgrad", mc, (M, N, K))
    dx = host(B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=torch.bfloat16, fp8_matrix_core=mc, split2=True))
    yr, bnd = gemm.dgrad(odyq, osdy, owqT, oswT)
    ok, rep = compare.check_bf16(dx, yr, bnd, rtol=rtol)
    assert ok, ("dgrad", rep)
    say("split-k forced wgrad", mc, (M, N, K))
    yr, bnd = gemm.wgrad(odyqT, osdyT, oxqT, osxT)
    dw = host(B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, fp8_matrix_core=mc, split2=True))
    ok, rep = compare.check_fp32(dw, yr, bnd, rtol=rtol)
    assert ok, ("wgrad", rep)
    dw0 = np.random.default_rng(M + 1).standard_normal((N, K)).astype(np.float32) * 1e-3
    dw = torch.from_numpy(dw0).cuda()
    B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=dw, accumulate=True, fp8_matrix_core=mc, split2=True)
    ok, rep = compare.check_fp32(host(dw), yr + dw0.astype(np.float64),
                                 bnd + np.abs(dw0) * (2.0 ** -23 / compare.FP32_RTOL), rtol=rtol)
    assert ok, ("wgrad accumulate", rep)


def test_split_k_deterministic_and_counters_left_zero(B):
    """Two runs of a split GEMM give identical bits, and the caller-owned workspace's
    counters are zero again after each call."""
    torch = _torch()
    M, N, K = 4096, 2048, 2048              # the o projection's weight gradient
    L = _split_layer(B, M, N, K, 7)
    dyqT, sdyT = B.fp8_quant_1x128(L.dy, transpose_out=True)
    xqT, sxT = B.fp8_quant_1x128(L.x, transpose_out=True)
    need = B.fp8_block_gemm_split2_workspace_size(B.OP_WGRAD, M, N, K)
    assert need > 0 and B.fp8_block_gemm_workspace_size(B.OP_WGRAD, M, N, K) == 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    tiles = 65536 // 4                      # the fixed counter region
    say("split-k determinism", (M, N, K))
    a = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, workspace=ws, split2=True)
    torch.cuda.synchronize()
    assert int(ws[:4 * tiles].view(torch.int32).abs().sum()) == 0
    ws[4 * tiles:].fill_(0x7F)               # stale partials from earlier calls must not matter
    # A call of another shape in between (the down projection's weight gradient,
    # 384 tiles) shares the workspace: its partials must not reach any counter.
    L2 = _split_layer(B, M, 2048, 6144, 8)
    d_qT, d_sT = B.fp8_quant_1x128(L2.dy, transpose_out=True)
    x_qT, x_sT = B.fp8_quant_1x128(L2.x, transpose_out=True)
    ws2 = torch.zeros(B.fp8_block_gemm_split2_workspace_size(B.OP_WGRAD, M, 2048, 6144), dtype=torch.uint8,
                      device="cuda")
    ws2[:ws.numel()].copy_(ws)
    d = B.fp8_block_gemm_wgrad(d_qT, d_sT, x_qT, x_sT, M=M, workspace=ws2, split2=True)
    a2 = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, workspace=ws2, split2=True)
    torch.cuda.synchronize()
    assert int(ws2[:4 * tiles].view(torch.int32).abs().sum()) == 0
    assert torch.equal(a.view(torch.int32), a2.view(torch.int32))
    od_qT, od_sT = quant.quant_1x128_tokens(L2.dyb)
    ox_qT, ox_sT = quant.quant_1x128_tokens(L2.xb)
    check_sampled(host(d), lambda r=None, cc=None: gemm.wgrad(od_qT, od_sT, ox_qT, ox_sT, r, cc), "f32",
                  "split wgrad down (shared workspace)", np.random.default_rng(78), k=24)
    b = B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, workspace=ws, split2=True)
    torch.cuda.synchronize()
    assert int(ws[:4 * tiles].view(torch.int32).abs().sum()) == 0
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # Unsplit (the default): a different summation order, the same rule.
    c = host(B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, workspace=False))
    odyqT, osdyT = quant.quant_1x128_tokens(L.dyb)
    oxqT, osxT = quant.quant_1x128_tokens(L.xb)
    rng = np.random.default_rng(77)
    check_sampled(host(a), lambda r=None, cc=None: gemm.wgrad(odyqT, osdyT, oxqT, osxT, r, cc), "f32",
                  "split wgrad o", rng, k=32)
    check_sampled(c, lambda r=None, cc=None: gemm.wgrad(odyqT, osdyT, oxqT, osxT, r, cc), "f32",
                  "unsplit wgrad o", rng, k=32)


# (M, N, K) and the default split of the forward, data-gradient and weight-gradient
# GEMMs (1: unsplit).  The launch rule: an output of at most 64 tiles of 128 x 128
# is split along the contraction into the largest S of 8, 4 and 2 with S * tiles <= 256
# and at least two scale blocks per split, when the workspace holds S FP32 partial planes
# of the output (summed in split order by a second kernel).
SMALL_GRIDS = [((256, 2048, 2048), (8, 8, 1)),      # configuration 1's shape
               ((256, 2048, 2304), (8, 4, 1)),      # 18 blocks over 8 splits: 2 or 3 each
               ((300, 1024, 1024), (4, 4, 1)),
               ((1000, 128, 640), (2, 1, 4)),       # 5 blocks over 2 splits; 1000 tokens pad to 8 blocks
               ((2048, 256, 1024), (4, 1, 8))]


def _small_split_bytes(op, M, N, K, s):
    """The 64 KiB counter region (left alone) and S FP32 partial planes of the I x J
    output (0 when not split)."""
    I, J = {0: (M, N), 1: (M, K), 2: (N, K)}[op]
    return 0 if s == 1 else 65536 + s * I * J * 4


@pytest.mark.parametrize("shape,splits", SMALL_GRIDS)
@pytest.mark.parametrize("mc", [False, True])
def test_small_grid_split(B, shape, splits, mc):
    """Small grids split along the contraction by default (binding workspace): every
    element of the forward (FP32 and BF16), data gradient and weight gradient (overwrite
    and accumulate) against the oracle, on both matrix paths."""
    torch = _torch()
    M, N, K = shape
    for op, s in zip((B.OP_FWD, B.OP_DGRAD, B.OP_WGRAD), splits):
        assert B.fp8_block_gemm_workspace_size(op, M, N, K) == _small_split_bytes(op, M, N, K, s), (op, s)
    L = _split_layer(B, M, N, K, 11 * M + N)
    rtol = 2.0 ** -10 + 1e-5 if mc else compare.FP32_RTOL
    xq, sx, xqT, sxT = B.fp8_quant_1x128_dual(L.x)
    wq, sw, wqT, swT = B.fp8_quant_128x128(L.w, with_transpose=True)
    dyq, sdy, dyqT, sdyT = B.fp8_quant_1x128_dual(L.dy)
    oxq, osx = quant.quant_1x128_rows(L.xb)
    owq, osw = quant.quant_128x128(L.wb)
    for od, out in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        say("small-grid split fwd", out, mc, shape, splits[0])
        y = host(B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=od, fp8_matrix_core=mc))
        yr, bnd = gemm.fwd(oxq, osx, owq, osw)
        ok, rep = (compare.check_fp32(y, yr, bnd, rtol=rtol) if out == "f32"
                   else compare.check_bf16(y, yr, bnd, rtol=rtol))
        assert ok, ("fwd", out, rep)
    say("small-grid split dgrad", mc, shape, splits[1])
    odyq, osdy = quant.quant_1x128_rows(L.dyb)
    owqT, oswT = quant.quant_128x128(np.ascontiguousarray(L.wb.T))
    dx = host(B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=torch.bfloat16, fp8_matrix_core=mc))
    yr, bnd = gemm.dgrad(odyq, osdy, owqT, oswT)
    ok, rep = compare.check_bf16(dx, yr, bnd, rtol=rtol)
    assert ok, ("dgrad", rep)
    say("small-grid split wgrad", mc, shape, splits[2])
    odyqT, osdyT = quant.quant_1x128_tokens(L.dyb)
    oxqT, osxT = quant.quant_1x128_tokens(L.xb)
    yr, bnd = gemm.wgrad(odyqT, osdyT, oxqT, osxT)
    dw = host(B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, fp8_matrix_core=mc))
    ok, rep = compare.check_fp32(dw, yr, bnd, rtol=rtol)
    assert ok, ("wgrad", rep)
    dw0 = np.random.default_rng(M + 3).standard_normal((N, K)).astype(np.float32) * 1e-3
    dwt = torch.from_numpy(dw0).cuda()
    B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=dwt, accumulate=True, fp8_matrix_core=mc)
    ok, rep = compare.check_fp32(host(dwt), yr + dw0.astype(np.float64),
                                 bnd + np.abs(dw0) * (2.0 ** -23 / compare.FP32_RTOL), rtol=rtol)
    assert ok, ("wgrad accumulate", rep)


@pytest.mark.parametrize("mc", [False, True])
def test_small_grid_split_deterministic_and_counters_left_zero(B, mc):
    """Configuration 1's forward GEMM split 8 ways with a caller-owned workspace: two
    calls give identical bits, the counter region of the split in two stays zero,
    stale partial planes do not matter, a workspace one byte short runs unsplit, and
    the unsplit result meets the same rule."""
    torch = _torch()
    M, N, K = 256, 2048, 2048
    L = _split_layer(B, M, N, K, 5)
    xq, sx = B.fp8_quant_1x128(L.x)
    wq, sw, _, _ = B.fp8_quant_128x128(L.w)
    need = B.fp8_block_gemm_workspace_size(B.OP_FWD, M, N, K)
    assert need == _small_split_bytes(0, M, N, K, 8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say("small-grid split determinism", mc)
    a = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.float32, fp8_matrix_core=mc, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0     # the counter region is left alone
    ws[65536:].fill_(0x7F)
    b = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.float32, fp8_matrix_core=mc, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # One byte short of the planes: the call runs unsplit.
    short = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    d = B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.float32, fp8_matrix_core=mc, workspace=short)
    c = host(B.fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.float32, fp8_matrix_core=mc, workspace=False))
    yr, bnd = gemm.fwd(*quant.quant_1x128_rows(L.xb), *quant.quant_128x128(L.wb))
    rtol = 2.0 ** -10 + 1e-5 if mc else compare.FP32_RTOL
    assert torch.equal(torch.from_numpy(c).view(torch.int32), d.cpu().view(torch.int32))
    for got, what in ((host(a), "split"), (c, "unsplit")):
        ok, rep = compare.check_fp32(got, yr, bnd, rtol=rtol)
        assert ok, (what, rep)
    # The same workspace then serves the split in two (FP8BLK_GEMM_SPLIT2), whose
    # arrival counters the plane split must have left at zero.
    L2 = _split_layer(B, 300, 256, 384, 6)
    x2q, s2x = B.fp8_quant_1x128(L2.x)
    w2q, s2w, _, _ = B.fp8_quant_128x128(L2.w)
    assert B.fp8_block_gemm_split2_workspace_size(B.OP_FWD, 300, 256, 384) <= need
    y2 = B.fp8_block_gemm_fwd(x2q, s2x, w2q, s2w, out_dtype=torch.float32, fp8_matrix_core=mc, workspace=ws,
                              split2=True)
    torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    yr2, bnd2 = gemm.fwd(*quant.quant_1x128_rows(L2.xb), *quant.quant_128x128(L2.wb))
    ok, rep = compare.check_fp32(host(y2), yr2, bnd2, rtol=rtol)
    assert ok, ("split in two after the plane split", rep)
