"""Pins for the oracle's fused producers (SwiGLU, RMSNorm), CPU only.

Expected values come from an independent evaluation: Python's decimal module at
60 digits for exp and sqrt, and an exact nearest-BF16 search with ties to even.
Closed forms (a 3-4 row, constant rows, eps inside the square root) and
invariants (power-of-two scaling, permutation) catch the plausible slips: a
subtracted mean, eps outside the root, a swapped sign in the sigmoid.
"""

from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import fused

getcontext().prec = 60


def bf16_bits(x):
    return (np.asarray([x], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]


def bits_value(b):
    return Decimal(float(np.uint32(int(b) << 16).view(np.float32)))


def nearest_bf16(d):
    """Exact nearest BF16 (ties to even) to a Decimal d of moderate magnitude."""
    if d == 0:
        return 0x8000 if d.is_signed() else 0
    b0 = int(bf16_bits(float(d)))
    cands = [b0 - 1, b0, b0 + 1]
    best = min(cands, key=lambda b: (abs(bits_value(b) - d), b & 1))
    return best


def dexp(x):
    return Decimal(x).exp()


@pytest.mark.parametrize("g", [-20.0, -3.5, -1.0, -0.5, 0.0, 2.0 ** -20, 0.5, 1.0, 3.75, 20.0, 88.0])
@pytest.mark.parametrize("u", [1.0, -2.5, 0.015625, 300.0])
def test_swiglu_matches_high_precision(g, u):
    gb = np.array([[bf16_bits(g)]], dtype=np.uint16)
    ub = np.array([[bf16_bits(u)]], dtype=np.uint16)
    got = int(fused.swiglu_bf16(gb, ub)[0, 0])
    gd, ud = bits_value(gb[0, 0]), bits_value(ub[0, 0])
    want = nearest_bf16(gd * ud / (1 + dexp(-gd)))
    assert got == want, (g, u, hex(got), hex(want))


def test_swiglu_closed_forms():
    g = np.array([[bf16_bits(0.0), bf16_bits(1.0), bf16_bits(-100.0), bf16_bits(1000.0)]], dtype=np.uint16)
    one = np.full_like(g, bf16_bits(1.0))
    h = fused.swiglu_bf16(g, one)[0]
    assert h[0] == 0                      # silu(0) = 0
    assert h[1] == 0x3F3B                 # silu(1) = 0.7310585... -> 0.73046875
    assert h[2] in (0x8000, 0x0000) or bits_value(h[2]).copy_abs() < Decimal("1e-40")
    assert h[3] == bf16_bits(1000.0)      # silu(x) = x for large x


def test_rmsnorm_three_four_row():
    x = np.array([[bf16_bits(3.0), bf16_bits(4.0)]], dtype=np.uint16)
    gamma = np.array([bf16_bits(1.0), bf16_bits(1.0)], dtype=np.uint16)
    y, rstd = fused.rmsnorm_bf16(x, gamma, 0.0)
    r = 1 / Decimal("12.5").sqrt()
    assert abs(Decimal(float(rstd[0])) - r) < r * Decimal("1e-15")
    assert int(y[0, 0]) == nearest_bf16(3 * r) and int(y[0, 1]) == nearest_bf16(4 * r)


def test_rmsnorm_eps_inside_the_root():
    x = np.array([[bf16_bits(0.5), bf16_bits(0.5)]], dtype=np.uint16)
    gamma = np.array([bf16_bits(1.0)] * 2, dtype=np.uint16)
    y, rstd = fused.rmsnorm_bf16(x, gamma, 0.25)
    r = 1 / Decimal("0.5").sqrt()               # mean 0.25 + eps 0.25
    assert abs(Decimal(float(rstd[0])) - r) < r * Decimal("1e-15")
    assert int(y[0, 0]) == nearest_bf16(Decimal("0.5") * r)


def test_rmsnorm_constant_rows_and_gamma():
    rng = np.random.default_rng(3)
    gam = (rng.standard_normal(64) * 0.5 + 1).astype(np.float32)
    gamma = (gam.view(np.uint32) >> 16).astype(np.uint16)
    x = np.zeros((3, 64), dtype=np.uint16)
    x[0, :] = bf16_bits(7.5)
    x[1, :] = bf16_bits(-0.001)
    x[2, :] = bf16_bits(2.0 ** -100)
    y, _ = fused.rmsnorm_bf16(x, gamma, 0.0)
    assert np.array_equal(y[0], gamma)                       # c / |c| * gamma
    assert np.array_equal(y[1], gamma ^ np.uint16(0x8000))   # sign flips only
    assert np.array_equal(y[2], gamma)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(9)
    xf = rng.standard_normal((4, 256)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    gamma = (np.abs(rng.standard_normal(256)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, _ = fused.rmsnorm_bf16(x, gamma, 0.0)
    x_scaled = (x.astype(np.uint32) + (5 << 7)).astype(np.uint16)   # x * 2^5 (normal BF16 exponents)
    ys, _ = fused.rmsnorm_bf16(x_scaled, gamma, 0.0)
    assert np.array_equal(y, ys)
    perm = rng.permutation(256)
    yp, _ = fused.rmsnorm_bf16(x[:, perm], gamma[perm], 0.0)
    assert np.array_equal(yp, y[:, perm])
