"""The block-scaled FP8 GEMMs (forward, data gradient, weight gradient).  TEST INFRASTRUCTURE.

Pages: paperlayer.ai summary of arXiv 2608.27370v1, appendix C
"生産学習の詳細", item "FP8実装pipeline" -- the linear-layer GEMMs run on
blockwise E4M3 operands for the forward pass, the data gradient and the weight
gradient; gradients are kept in FP32 and the hidden flow in BF16.  arxiv-wiki
summary, section "접근 방법" item (4) -- activation scales per 1x128 group,
weight scales per 128x128 block.

Definition (the plain reading of "blockwise scaled GEMM"): with codes QA [I, L],
QB [J, L] and scales SA(i, l//128), SB(j, l//128),

    Y[i, j] = sum_lb SA(i, lb) * SB(j, lb) * sum_{l in lb} D(QA[i, l]) * D(QB[j, l])

which, by distributivity, is the ordinary product of the dequantised matrices:
Y = deq(A) @ deq(B)^T.  That is what is computed here, in float64 with numpy's
matmul as the only library step.  Every dequantised element D(q) * s is exact in
float64 (4 significant bits times 24); products and the sum carry float64
rounding only, about 1e-16 relative to the budget below.

The per-element error budget used by the acceptance test is
    Bnd[i, j] = sum_l |deq(A)[i, l]| * |deq(B)[j, l]|.

Operand mapping (row-major shapes, X [M, K], W [N, K], dY [M, N]):
    forward   Y  [M, N] = Xq . Wq^T      QA = Xq   (1x128 along K), QB = Wq   (128x128)
    dgrad     dX [M, K] = dYq . (WqT)^T  QA = dYq  (1x128 along N), QB = WqT  (128x128 of W^T)
    wgrad     dW [N, K] = dYqT . XqT^T   QA = dYqT (1x128 along M), QB = XqT  (1x128 along M)
"""

import numpy as np

from . import e4m3
from .quant import GROUP, bf16_bits_to_f32, expand_block_scales


def _deq(codes, row_scales):
    """D(codes[r, l]) * row_scales[r, l // 128] as float64."""
    L = codes.shape[1]
    s = np.repeat(np.asarray(row_scales, dtype=np.float64), GROUP, axis=1)[:, :L]
    return e4m3.decode(codes) * s


def block_gemm(qa, sa, qb, sb, rows=None, cols=None, budget=True):
    """Y = deq(A) @ deq(B)^T in float64, optionally only for selected rows/cols.

    qa [I, L], sa [I, ceil(L/128)], qb [J, L], sb [J, ceil(L/128)].
    rows / cols: optional index arrays selecting the outputs to compute (used to
    check large problems on a sample of outputs).  Returns (Y, Bnd) where Bnd is
    the error budget sum |a*b| (None when budget=False).
    """
    if rows is not None:
        qa, sa = qa[rows], sa[rows]
    if cols is not None:
        qb, sb = qb[cols], sb[cols]
    a = _deq(qa, sa)
    b = _deq(qb, sb)
    y = a @ b.T
    bnd = (np.abs(a) @ np.abs(b).T) if budget else None
    return y, bnd


def fwd(xq, sx, wq, sw, rows=None, cols=None, budget=True):
    """Forward Y[M, N] = Xq . Wq^T; sx [M, K/128] per-row groups, sw [N/128, K/128] blocks."""
    return block_gemm(xq, sx, wq, expand_block_scales(sw, wq.shape[0]), rows, cols, budget)


def dgrad(dyq, sdy, wqt, swt, rows=None, cols=None, budget=True):
    """Data gradient dX[M, K] = dY . W using WqT [K, N] and its block scales swt [K/128, N/128]."""
    return block_gemm(dyq, sdy, wqt, expand_block_scales(swt, wqt.shape[0]), rows, cols, budget)


def wgrad(dyqt, sdyt, xqt, sxt, rows=None, cols=None, budget=True):
    """Weight gradient dW[N, K] = dY^T . X from token-dimension groups.

    dyqt [N, M], sdyt [N, ceil(M/128)], xqt [K, M], sxt [K, ceil(M/128)].
    """
    return block_gemm(dyqt, sdyt, xqt, sxt, rows, cols, budget)


def bf16_gemm(a_bits, b_bits, rows=None, cols=None, budget=True):
    """Plain BF16 GEMM C = A . B^T in float64 (the baseline the FP8 GEMMs are compared with).

    Pages: paperlayer.ai summary, appendix D "MuonH Scaling-Ladder Analysis"
    (FP8 throughput relative to BF16 at 1.7B) -- the BF16 GEMM of the same
    shapes is the reference point.  a_bits [I, L], b_bits [J, L] are BF16 bit
    patterns; every BF16 value is exact in float64.  Returns (C, Bnd) with
    Bnd = |A| @ |B|^T (None when budget=False).
    """
    a = bf16_bits_to_f32(a_bits if rows is None else a_bits[rows]).astype(np.float64)
    b = bf16_bits_to_f32(b_bits if cols is None else b_bits[cols]).astype(np.float64)
    c = a @ b.T
    bnd = (np.abs(a) @ np.abs(b).T) if budget else None
    return c, bnd


def round_to_bf16(y):
    """float64 -> nearest BF16 (ties to even), returned as float64 values.

    Two steps would double-round, so the rounding is done directly on the
    float64 value: BF16 has 8 significant bits, so within the binade of |y| the
    BF16 spacing is 2**(floor(log2|y|) - 7), and subnormal BF16 values are
    spaced 2**-133.  Magnitudes that round beyond the largest BF16 become inf.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)
    binade = np.maximum(ex - 1, -126)
    spacing = np.ldexp(1.0, binade - 7)
    r = np.rint(a / spacing) * spacing
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > bf16_max, np.inf, r)
    return np.copysign(r, y)
