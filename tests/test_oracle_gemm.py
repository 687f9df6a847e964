"""Pins for the oracle's block-scaled GEMMs (CPU only).

* brute force: the per-block definition evaluated with exact rational
  arithmetic in pure-Python loops on tiny shapes;
* lossless family: inputs whose quantisation is exact, so the result must equal
  the exact product of the original BF16 matrices;
* index pins: one-hot K-blocks (which scale goes with which block) and scaled
  identity weights (weight-block scale indexing and the transposed operand);
* the BF16 rounding of results, against an exact nearest search.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import compare, e4m3, gemm, quant


def bits_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_bf16_trunc(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _exact_block_gemm(qa, sa, qb, sb):
    """sum_lb SA*SB*sum_l D(a)D(b) with Fractions (pure Python; tiny shapes only)."""
    I, L = qa.shape
    J = qb.shape[0]
    da = e4m3.decode(qa)
    db = e4m3.decode(qb)
    out = [[Fraction(0)] * J for _ in range(I)]
    bnd = [[Fraction(0)] * J for _ in range(I)]
    for i in range(I):
        for j in range(J):
            for lb in range(-(-L // 128)):
                part = Fraction(0)
                apart = Fraction(0)
                for l in range(lb * 128, min(L, lb * 128 + 128)):
                    p = Fraction(float(da[i, l])) * Fraction(float(db[j, l]))
                    part += p
                    apart += abs(p)
                scl = Fraction(float(sa[i, lb])) * Fraction(float(sb[j, lb]))
                out[i][j] += scl * part
                bnd[i][j] += abs(scl) * apart
    return out, bnd


@pytest.mark.parametrize("shape", [(5, 7, 128), (9, 3, 256), (4, 6, 300)])
def test_block_gemm_matches_exact_rational_definition(shape):
    I, J, L = shape
    rng = np.random.default_rng(sum(shape))
    a = to_bf16_trunc(rng.standard_normal((I, L)) * np.exp(rng.standard_normal((I, 1)) * 3))
    b = to_bf16_trunc(rng.standard_normal((J, L)) * 0.02)
    qa, sa = quant.quant_1x128_rows(a)
    qb, sb = quant.quant_1x128_rows(b)
    y, bnd = gemm.block_gemm(qa, sa, qb, sb)
    ey, eb = _exact_block_gemm(qa, sa, qb, sb)
    for i in range(I):
        for j in range(J):
            assert abs(Fraction(float(y[i, j])) - ey[i][j]) <= eb[i][j] * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 300)
            assert abs(Fraction(float(bnd[i, j])) - eb[i][j]) <= eb[i][j] * Fraction(1, 10 ** 12)


def test_forward_against_exact_definition_with_weight_blocks():
    rng = np.random.default_rng(21)
    M, N, K = 6, 130, 256
    x = to_bf16_trunc(rng.standard_normal((M, K)))
    w = to_bf16_trunc(rng.standard_normal((N, K)) * 0.02)
    xq, sx = quant.quant_1x128_rows(x)
    wq, sw = quant.quant_128x128(w)
    cols = np.array([0, 1, 127, 128, 129])
    y, bnd = gemm.fwd(xq, sx, wq, sw, cols=cols)
    # Exact: weight scale for output column n and K-block kb is sw[n // 128, kb].
    sb = np.stack([sw[n // 128] for n in cols])
    ey, eb = _exact_block_gemm(xq, sx, wq[cols], sb)
    for i in range(M):
        for j in range(len(cols)):
            assert abs(Fraction(float(y[i, j])) - ey[i][j]) <= eb[i][j] * Fraction(1, 10 ** 12)


def _lossless_group_values(rng, shape, exps):
    """Values from {+-448 * 2^-k, k=0..3} * 2^j with one +-448*2^j per 128-group (s = 2^j exactly)."""
    R, L = shape
    k = rng.integers(0, 4, size=shape)
    sgn = rng.choice([-1.0, 1.0], size=shape)
    v = sgn * 448.0 * np.ldexp(1.0, -k)
    v[:, ::128] = 448.0
    v = v * np.ldexp(1.0, np.repeat(exps, 128, axis=1)[:, :L])
    return v.astype(np.float32)


def test_lossless_family_is_exact():
    """If every group quantises losslessly, Y equals the exact product of the inputs."""
    rng = np.random.default_rng(33)
    M, N, L = 16, 12, 384
    ea = rng.integers(-8, 8, size=(M, 3))
    eb = rng.integers(-8, 8, size=(N, 3))
    a = _lossless_group_values(rng, (M, L), ea)
    b = _lossless_group_values(rng, (N, L), eb)
    qa, sa = quant.quant_1x128_rows(to_bf16_trunc(a))
    qb, sb = quant.quant_1x128_rows(to_bf16_trunc(b))
    assert np.all(sa == np.ldexp(np.float32(1.0), ea))
    y, _ = gemm.block_gemm(qa, sa, qb, sb)
    exact = a.astype(np.float64) @ b.astype(np.float64).T     # exact: few bits, small L
    assert np.array_equal(y, exact)


def test_one_hot_k_blocks_pin_scale_index():
    """Only K-block kb is non-zero: Y must use the scales of block kb and no other."""
    rng = np.random.default_rng(44)
    M, N, K = 4, 256, 512
    for kb in range(K // 128):
        x = np.zeros((M, K), dtype=np.float32)
        w = np.zeros((N, K), dtype=np.float32)
        x[:, kb * 128:(kb + 1) * 128] = rng.standard_normal((M, 128))
        w[:, kb * 128:(kb + 1) * 128] = rng.standard_normal((N, 128)) * 0.02
        # Give the other blocks of w distinct, non-zero content so a wrong block index shows.
        other = [b for b in range(K // 128) if b != kb]
        for b in other:
            w[:, b * 128:(b + 1) * 128] = (b + 1) * 0.5
        xq, sx = quant.quant_1x128_rows(to_bf16_trunc(x))
        wq, sw = quant.quant_128x128(to_bf16_trunc(w))
        y, _ = gemm.fwd(xq, sx, wq, sw)
        dx = e4m3.decode(xq)[:, kb * 128:(kb + 1) * 128] * sx[:, kb:kb + 1].astype(np.float64)
        dw = e4m3.decode(wq)[:, kb * 128:(kb + 1) * 128] * np.repeat(sw[:, kb], 128)[:, None].astype(np.float64)
        ref = dx @ dw.T
        assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_scaled_identity_weights_pin_block_scales_and_transpose():
    """W = blockdiag(c_b * I): Y = X W^T picks X's columns times the block constants.

    dgrad with WqT = Q(W^T) must give dY . W, i.e. the same block constants by
    the transposed index.
    """
    rng = np.random.default_rng(55)
    M, n = 8, 384
    consts = np.array([0.5, 3.0, 0.015625], dtype=np.float32)
    w = np.zeros((n, n), dtype=np.float32)
    for b in range(3):
        w[b * 128:(b + 1) * 128, b * 128:(b + 1) * 128] = np.eye(128) * consts[b]
    w[0:128, 256:384] = 0.25            # an off-diagonal block makes W non-symmetric
    x = (rng.integers(-7, 8, size=(M, n)) * 0.25).astype(np.float32)
    x[:, ::128] = 1.75                  # lossless groups: amax 1.75 -> s = 2^-8 exactly
    wb = to_bf16_trunc(w)
    xq, sx = quant.quant_1x128_rows(to_bf16_trunc(x))
    wq, sw = quant.quant_128x128(wb)
    y, _ = gemm.fwd(xq, sx, wq, sw)
    deq_x = e4m3.decode(xq) * np.repeat(sx, 128, axis=1)
    assert np.array_equal(deq_x, x.astype(np.float64))
    deq_w = e4m3.decode(wq) * np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)
    assert np.allclose(y, x.astype(np.float64) @ deq_w.T, rtol=1e-14, atol=0)
    # dgrad: dX = dY . W uses Q(W^T) with transposed block scales.
    dy = x
    wqt, swt = quant.quant_128x128(np.ascontiguousarray(wb.T))
    dxq, sdx = xq, sx
    dx, _ = gemm.dgrad(dxq, sdx, wqt, swt)
    assert np.allclose(dx, dy.astype(np.float64) @ deq_w, rtol=1e-14, atol=0)


def test_wgrad_token_groups_and_padding():
    """wgrad over a ragged token count equals the exact definition on token groups."""
    rng = np.random.default_rng(66)
    M, N, K = 200, 5, 6
    x = to_bf16_trunc(rng.standard_normal((M, K)))
    dy = to_bf16_trunc(rng.standard_normal((M, N)) * 1e-3)
    xqt, sxt = quant.quant_1x128_tokens(x)
    dyqt, sdyt = quant.quant_1x128_tokens(dy)
    assert xqt.shape == (K, M) and sxt.shape == (K, 2)
    y, _ = gemm.wgrad(dyqt, sdyt, xqt, sxt)
    ey, eb = _exact_block_gemm(dyqt, sdyt, xqt, sxt)
    for i in range(N):
        for j in range(K):
            assert abs(Fraction(float(y[i, j])) - ey[i][j]) <= eb[i][j] * Fraction(1, 10 ** 12)
    # Budget sanity: the result is within its own budget of the unquantised product.
    ref = bits_f32(dy).astype(np.float64).T @ bits_f32(x).astype(np.float64)
    _, bnd = gemm.wgrad(dyqt, sdyt, xqt, sxt)
    assert np.all(np.abs(y - ref) <= 0.15 * bnd + 1e-30)


def _nearest_bf16_exact(v):
    """Nearest BF16 to float64 v by exact search over neighbouring bit patterns; ties -> even."""
    f = np.float32(v)
    base = int(f.view(np.uint32)) >> 16
    best = None
    for b in range(max(base - 2, 0), base + 3):
        if (b & 0x7F80) == 0x7F80:
            continue
        cand = Fraction(float(bits_f32(np.uint16(b | (0x8000 if v < 0 else 0)))))
        d = abs(cand - Fraction(v))
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return float(best[1])


def test_round_to_bf16_against_exact_search():
    rng = np.random.default_rng(77)
    v = rng.standard_normal(3000) * np.exp(rng.uniform(-60, 60, 3000))
    # add exact ties: midpoints between consecutive BF16 values
    b = rng.integers(0x0100, 0x7F00, 300).astype(np.uint16)
    lo = bits_f32(b).astype(np.float64)
    hi = bits_f32(b + 1).astype(np.float64)
    # subnormal-range values (BF16 spacing 2^-133 below 2^-126)
    sub = rng.uniform(-1, 1, 500) * 2.0 ** -124
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2, sub])
    r = gemm.round_to_bf16(v)
    for vi, ri in zip(v, r):
        assert ri == _nearest_bf16_exact(vi), vi


def test_acceptance_checks_reject_planted_errors():
    rng = np.random.default_rng(88)
    y = rng.standard_normal(1000)
    bnd = np.abs(y) + 1.0
    ok, _ = compare.check_fp32(y.astype(np.float32), y, bnd)
    assert ok
    bad = y.astype(np.float32).copy()
    bad[17] += 1e-3
    ok, rep = compare.check_fp32(bad, y, bnd)
    assert not ok and rep["bad"] == 1
    r = gemm.round_to_bf16(y)
    gb = to_bf16_trunc(r.astype(np.float32))
    ok, _ = compare.check_bf16(gb, y, bnd)
    assert ok
    gb2 = gb.copy()
    gb2[3] += 2                       # two BF16 ulps away
    ok, rep = compare.check_bf16(gb2, y, bnd * 1e-9)
    assert not ok and rep["bad"] == 1


def _exact_bf16_gemm(a_bits, b_bits):
    """sum_l A[i, l] * B[j, l] over the BF16 values with Fractions (tiny shapes only)."""
    fa = bits_f32(a_bits)
    fb = bits_f32(b_bits)
    I, L = fa.shape
    J = fb.shape[0]
    out = [[sum((Fraction(float(fa[i, l])) * Fraction(float(fb[j, l])) for l in range(L)), Fraction(0))
            for j in range(J)] for i in range(I)]
    return out


@pytest.mark.parametrize("shape", [(3, 5, 64), (6, 2, 130)])
def test_bf16_gemm_matches_exact_rational_sum(shape):
    I, J, L = shape
    rng = np.random.default_rng(7 + sum(shape))
    a = to_bf16_trunc(rng.standard_normal((I, L)) * np.exp(rng.standard_normal((I, 1)) * 4))
    b = to_bf16_trunc(rng.standard_normal((J, L)))
    y, bnd = gemm.bf16_gemm(a, b)
    ey = _exact_bf16_gemm(a, b)
    for i in range(I):
        for j in range(J):
            assert abs(Fraction(float(y[i, j])) - ey[i][j]) <= Fraction(float(bnd[i, j])) * Fraction(1, 10 ** 12)


def test_bf16_gemm_operand_orientation():
    """C = A . B^T: a row of ones against a one-hot row of B picks one column of A."""
    I, J, L = 4, 3, 8
    a = to_bf16_trunc(np.arange(I * L, dtype=np.float32).reshape(I, L))
    b = np.zeros((J, L), dtype=np.uint16)
    for j in range(J):
        b[j, 2 * j + 1] = 0x3F80          # BF16 1.0
    y, _ = gemm.bf16_gemm(a, b)
    want = np.arange(I * L, dtype=np.float64).reshape(I, L)[:, [1, 3, 5]]
    assert np.array_equal(y, want)
    ysel, _ = gemm.bf16_gemm(a, b, rows=np.array([2]), cols=np.array([1, 2]))
    assert np.array_equal(ysel, want[[2]][:, [1, 2]])
