"""Pins for the oracle's quantisers (CPU only): closed forms, invariants and
hand-derived cases, none of which re-run the oracle's own arithmetic."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_to_bf16_bits(x):
    """Exact conversion of BF16-representable float32 values to BF16 bits."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value is not BF16-representable"
    return (b >> 16).astype(np.uint16)


def bits_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any BF16 is fine here


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()[:2]
                out[k] = int(v, 16)
    return out


def test_pow2_tie_discriminates_division_from_reciprocal():
    g = _read_golden("quant_pow2_tie.txt")
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0] = g["x_bits_0"]
    x[0, 1] = g["x_bits_1"]
    q, s = quant.quant_1x128_rows(x)
    assert s.view(np.uint32)[0, 0] == g["scale_bits"]
    assert q[0, 0] == g["code_0"]
    assert q[0, 1] == g["code_1"]
    assert np.all(q[0, 2:] == g["code_rest"])


def test_amax_element_encodes_to_448_for_every_bf16_magnitude():
    """For every positive finite BF16 a, a group with amax a puts code 0x7E on a.

    Also pins that the quotient a / fl32(a/448) stays within 448 * (1 +- 2^-20)
    for normal scales and 448 * (1 +- 1/128) for denormal ones, so saturation
    is never what puts 448 on the amax element -- checked with exact rational
    arithmetic on the binary32 scale.
    """
    bits = np.arange(1, 0x7F80, dtype=np.uint16)          # all positive finite BF16
    x = np.zeros((bits.size, 128), dtype=np.uint16)
    x[:, 5] = bits
    x[:, 6] = bits | 0x8000                               # -amax too
    q, s = quant.quant_1x128_rows(x)
    assert np.all(q[:, 5] == 0x7E)
    assert np.all(q[:, 6] == 0xFE)
    assert np.all(q[:, :5] == 0) and np.all(q[:, 7:] == 0)
    # Exact: |a/s - 448| <= 448 * 2^-23 * (1 + tiny) for normal s.
    sel = np.concatenate([np.arange(0, 300), np.arange(300, bits.size, 97)])
    for i in sel:
        a = Fraction(float(bits_f32(bits[i])))
        sv = Fraction(float(s[i, 0]))
        assert sv > 0
        ratio = a / sv
        if float(s[i, 0]) >= np.finfo(np.float32).tiny:
            assert abs(ratio - 448) <= Fraction(448, 1 << 20), (hex(bits[i]), float(ratio))
        else:
            # Denormal scale: a/448 >= 2^-133/448 keeps >= 146 denormal steps, so the
            # ratio stays within 448 * (1 +- 1/128) -- still far from the 464 midpoint.
            assert abs(ratio - 448) <= Fraction(448, 128), (hex(bits[i]), float(ratio))


def test_scale_is_amax_over_448_closed_form():
    """s equals amax/448 rounded to binary32, checked with exact rationals."""
    rng = np.random.default_rng(7)
    x = rand_bf16(rng, (64, 384))
    q, s = quant.quant_1x128_rows(x)
    xf = bits_f32(x)
    for r in range(0, 64, 9):
        for g in range(3):
            amax = Fraction(float(np.max(np.abs(xf[r, g * 128:(g + 1) * 128]))))
            exact = amax / 448
            sv = Fraction(float(s[r, g]))
            ulp = Fraction(2) ** (int(np.floor(np.log2(float(sv)))) - 23)
            assert abs(sv - exact) <= ulp / 2


def test_roundtrip_error_bound():
    """|D(q)*s - x| <= 2^-4 |x| for |x/s| >= 2^-6, else <= 2^-10 s (exact arithmetic in float64)."""
    rng = np.random.default_rng(11)
    x = rand_bf16(rng, (256, 1024), scale=3.0)
    q, s = quant.quant_1x128_rows(x)
    xf = bits_f32(x).astype(np.float64)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    back = e4m3.decode(q) * sf
    err = np.abs(back - xf)
    normal = np.abs(xf) >= (2.0 ** -6) * sf
    tol = 1 + 2.0 ** -20
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf[normal]) * tol)
    assert np.all(err[~normal] <= 2.0 ** -10 * sf[~normal] * tol)


def test_block_constant_groups():
    for c in [1.0, -3.5, 0.02001953125, 448.0, 1e-30, -7.0e20]:
        cb = f32_to_bf16_bits(np.float32(c)) if np.float32(c).view(np.uint32) & 0xFFFF == 0 else \
            (np.float32(c).view(np.uint32) >> 16).astype(np.uint16)
        x = np.full((3, 256), cb, dtype=np.uint16)
        q, s = quant.quant_1x128_rows(x)
        assert np.all(q == (0x7E if c > 0 else 0xFE))
        w = np.full((130, 260), cb, dtype=np.uint16)
        qw, sw = quant.quant_128x128(w)
        assert np.all(qw == (0x7E if c > 0 else 0xFE))
        assert sw.shape == (2, 3)
        assert np.all(sw == sw[0, 0])


def test_zero_groups_and_partial_groups():
    rng = np.random.default_rng(3)
    x = rand_bf16(rng, (8, 300))
    x[2, 128:256] = 0
    x[5, :] = 0x8000                                     # all -0
    q, s = quant.quant_1x128_rows(x)
    assert s.shape == (8, 3)
    assert s[2, 1] == 0 and np.all(q[2, 128:256] == 0)
    assert np.all(s[5] == 0) and np.all(q[5] == 0)
    # A partial group (44 valid columns) is quantised as if padded with zeros.
    xp = np.zeros((8, 384), dtype=np.uint16)
    xp[:, :300] = x
    qp, sp = quant.quant_1x128_rows(xp)
    assert np.array_equal(sp, s)
    assert np.array_equal(qp[:, :300], q)
    assert np.all(qp[:, 300:] == 0)


def test_scale_equivariance_negation_permutation():
    rng = np.random.default_rng(5)
    x = rand_bf16(rng, (16, 256))
    q, s = quant.quant_1x128_rows(x)
    # x * 2^t: same codes, scales * 2^t (BF16 exponent shift, no over/underflow here).
    for t in (-20, -3, 5, 40):
        xs = f32_to_bf16_bits(bits_f32(x) * np.float32(2.0 ** t))
        q2, s2 = quant.quant_1x128_rows(xs)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** t))
    # Negation flips sign bits only (zeros become negative zeros 0x80).
    qn, sn = quant.quant_1x128_rows(x ^ 0x8000)
    assert np.array_equal(sn, s)
    assert np.array_equal(qn, q ^ 0x80)
    # A permutation inside each group permutes the codes.
    perm = np.concatenate([rng.permutation(128), 128 + rng.permutation(128)])
    qp, sp = quant.quant_1x128_rows(x[:, perm])
    assert np.array_equal(sp, s) and np.array_equal(qp, q[:, perm])


def test_group_membership_from_planted_maxima():
    """Plant a distinct maximum in each (row, group); the scale must be that maximum/448."""
    R, C = 5, 640
    x = np.full((R, C), f32_to_bf16_bits(np.float32(0.5)), dtype=np.uint16)
    planted = {}
    for r in range(R):
        for g in range(C // 128):
            val = np.float32(2.0 ** (r + 2 * g + 1))
            col = g * 128 + (37 * r + 11 * g) % 128
            x[r, col] = f32_to_bf16_bits(val)
            planted[(r, g)] = (col, val)
    q, s = quant.quant_1x128_rows(x)
    for (r, g), (col, val) in planted.items():
        assert s[r, g] == np.float32(val / np.float32(448.0))
        assert q[r, col] == 0x7E
    # The token-dimension quantiser groups along rows of its input.
    xt = np.ascontiguousarray(x.T)                       # [C, R] tokens x features
    qt, st = quant.quant_1x128_tokens(xt)
    assert np.array_equal(qt, q) and np.array_equal(st, s)


def test_128x128_blocks_and_transpose_identity():
    rng = np.random.default_rng(9)
    w = rand_bf16(rng, (300, 520), scale=0.02)
    q, s = quant.quant_128x128(w)
    assert s.shape == (3, 5)
    wf = bits_f32(w)
    for br in range(3):
        for bc in range(5):
            blk = wf[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
            amax = np.max(np.abs(blk))
            assert s[br, bc] == np.float32(amax / np.float32(448.0))
            i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert q[br * 128 + i, bc * 128 + j] in (0x7E, 0xFE)
    qt, st = quant.quant_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_denormal_scales_kept():
    """A group whose amax is tiny gets a binary32-denormal scale, not zero."""
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0] = 0x0001          # smallest BF16 subnormal, 2^-133
    x[0, 1] = 0x8001
    q, s = quant.quant_1x128_rows(x)
    assert s[0, 0] > 0 and s[0, 0] < np.finfo(np.float32).tiny
    assert q[0, 0] == 0x7E and q[0, 1] == 0xFE
