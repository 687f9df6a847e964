"""Pins for the oracle's E4M3 codec (CPU only).

The encoder is checked against a brute-force nearest-value search over the
decoded code table (a different algorithm: table search instead of exponent
arithmetic), exhaustively over every binary32 magnitude in the range where
rounding decisions happen, and against hand-derived landmark codes.
"""

import os

import numpy as np
import pytest

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _landmarks():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), float(value)))
    return rows


def test_landmark_codes_decode():
    rows = _landmarks()
    assert len(rows) >= 15
    for code, value in rows:
        got = e4m3.decode(np.array([code], dtype=np.uint8))[0]
        if np.isnan(value):
            assert np.isnan(got), hex(code)
        else:
            assert got == value, (hex(code), got, value)
            assert np.signbit(got) == np.signbit(value), hex(code)


def test_landmark_codes_encode():
    for code, value in _landmarks():
        if np.isnan(value):
            continue
        got = e4m3.encode(np.array([value], dtype=np.float32))[0]
        assert got == code, (hex(code), hex(got))


def test_table_structure():
    # 126 finite positive values, strictly increasing with the code, mirrored by sign.
    d = e4m3.decode(np.arange(256, dtype=np.uint8))
    pos = d[1:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos.max() == 448.0
    neg = d[0x81:0xFF]
    assert np.array_equal(neg, -pos)
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(~np.isnan(d)) == 254


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


# ---- brute force: nearest value in the code table, ties to the even code ----

_POS_VALUES = e4m3.decode(np.arange(0, 0x7F, dtype=np.uint8))  # codes 0x00..0x7E, increasing


def _brute_encode(v32):
    """Nearest finite E4M3 magnitude by table search; ties -> even code; >448 -> 448."""
    v32 = np.asarray(v32, dtype=np.float32)
    a = np.abs(v32).astype(np.float64)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first table value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= _POS_VALUES[-1], 0x7E, code)        # saturation
    code = np.where(a <= _POS_VALUES[0], 0, code)
    sign = np.signbit(v32).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def test_bruteforce_exhaustive_decision_range():
    """Every positive binary32 in [2^-12, 2^10): 22 binades x 2^23 values.

    Below 2^-12 everything rounds to zero; at or above 2^10 everything
    saturates -- both covered by the next test.
    """
    lo_bits = np.float32(2.0 ** -12).view(np.uint32)
    hi_bits = np.float32(2.0 ** 10).view(np.uint32)
    chunk = 1 << 23
    for start in range(int(lo_bits), int(hi_bits), chunk):
        bits = np.arange(start, min(start + chunk, int(hi_bits)), dtype=np.uint32)
        v = bits.view(np.float32)
        a = e4m3.encode(v)
        b = _brute_encode(v)
        if not np.array_equal(a, b):
            i = np.nonzero(a != b)[0][0]
            pytest.fail(f"mismatch at {v[i]!r} bits {bits[i]:#x}: oracle {a[i]:#x} brute {b[i]:#x}")


def test_bruteforce_outside_range_and_signs():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(e4m3.encode(v), _brute_encode(v))
    # Negative inputs differ from positive ones only in the sign bit.
    pos = np.abs(v)
    assert np.array_equal(e4m3.encode(-pos), e4m3.encode(pos) | 0x80)
    # Signed zeros and tiny values keep their sign.
    tiny = np.array([0.0, -0.0, 1e-45, -1e-45, 2.0 ** -10, -(2.0 ** -10)], dtype=np.float32)
    assert list(e4m3.encode(tiny)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def test_ties_and_saturation_closed_forms():
    # Midpoints between consecutive codes round to the even code.
    vals = _POS_VALUES
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2)   # exact in binary32
    got = e4m3.encode(mids).astype(np.int64)
    lo_codes = np.arange(0, 0x7E)
    expect = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1)
    assert np.array_equal(got, expect)
    # Saturation: everything above 448 (finite or infinite) -> 448.
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e5, 3e38, np.inf], dtype=np.float32)
    assert np.all(e4m3.encode(big) == 0x7E)
    assert np.all(e4m3.encode(-big) == 0xFE)
    assert np.all(e4m3.encode(np.array([np.nan], dtype=np.float32)) & 0x7F == 0x7F)


def test_decision_rule_matches_the_encoder():
    """The boundary rule used for the all-binary32 GPU scan reproduces encode()."""
    import torch
    from tests.encode_rule import decision_midpoints, expected_codes_torch
    rng = np.random.default_rng(77)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    dense = np.arange(int(np.float32(2.0 ** -11).view(np.uint32)), int(np.float32(500.0).view(np.uint32)), 97,
                      dtype=np.uint32)
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 1, 0x80000001],
                        dtype=np.uint32)
    bits = np.concatenate([bits, dense, dense | np.uint32(0x80000000), specials])
    mids = torch.from_numpy(decision_midpoints())
    got = expected_codes_torch(torch, torch.from_numpy(bits.view(np.int32)), mids)
    assert np.array_equal(got.numpy().astype(np.uint8), e4m3.encode(bits.view(np.float32)))
