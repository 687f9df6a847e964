"""Pins for the oracle's bit-exact acceptance test (CPU only).

Every quantiser parity test ends in ``compare.check_exact``, so a loose
comparison there would let wrong codes or scales through unnoticed.  The cases
below are planted differences whose expected verdict follows from what
"bit-exact" means, not from the function's code: a single changed byte, the
sign of a zero scale, a denormal against zero, NaN payloads, and shape or
dtype mismatches.  A value-based float comparison would pass -0 against +0
and fail identical NaNs; both are caught here.
"""

import numpy as np

from oracle import compare


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def test_identical_codes_match():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 256, size=(37, 300), dtype=np.uint8)
    assert compare.check_exact(q, q.copy()) == (True, 0)


def test_one_changed_byte_is_counted():
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=(64, 129), dtype=np.uint8)
    for pos, delta in (((0, 0), 1), ((63, 128), 0x80), ((17, 64), 0x7F)):
        r = q.copy()
        r[pos] ^= np.uint8(delta)
        assert compare.check_exact(q, r) == (False, 1), pos
    r = q.copy()
    r[3, :5] ^= np.uint8(1)
    assert compare.check_exact(r, q) == (False, 5)


def test_signed_zero_scales_differ():
    pos, neg = _f32([0x00000000]), _f32([0x80000000])
    assert pos[0] == neg[0]                     # equal as values ...
    assert compare.check_exact(pos, neg) == (False, 1)   # ... but not bit-exact
    assert compare.check_exact(neg, neg.copy()) == (True, 0)


def test_denormal_scale_is_not_zero():
    den = _f32([0x00000001, 0x3F800000])
    zero = _f32([0x00000000, 0x3F800000])
    assert compare.check_exact(den, zero) == (False, 1)


def test_nan_payloads():
    a = _f32([0x7FC00000, 0x7FC00001, 0xFFC00000])
    assert compare.check_exact(a, a.copy()) == (True, 0)      # identical NaNs match
    b = _f32([0x7FC00000, 0x7FC00002, 0x7FC00000])
    assert compare.check_exact(a, b) == (False, 2)            # payload and sign differ


def test_one_ulp_scale_difference():
    s = np.array([1.0, 448.0, 2.0 ** -126], dtype=np.float32)
    t = s.copy()
    t[1] = np.nextafter(t[1], np.float32(np.inf))
    assert compare.check_exact(s, t) == (False, 1)


def test_shape_and_dtype_mismatch_fail():
    q = np.zeros((4, 128), dtype=np.uint8)
    assert compare.check_exact(q, np.zeros((4, 129), dtype=np.uint8)) == (False, -1)
    assert compare.check_exact(q, np.zeros((128, 4), dtype=np.uint8)) == (False, -1)
    assert compare.check_exact(q, q.astype(np.int8)) == (False, -1)
    s = np.ones(8, dtype=np.float32)
    assert compare.check_exact(s, s.astype(np.float64)) == (False, -1)


def test_strided_views_compare_elementwise():
    buf = np.arange(2 * 300, dtype=np.uint32).reshape(2, 300).astype(np.uint8)
    view = buf[:, 10:266]
    assert compare.check_exact(view, np.ascontiguousarray(view)) == (True, 0)
    s = np.arange(40, dtype=np.float32).reshape(8, 5)
    assert compare.check_exact(s.T, np.ascontiguousarray(s.T)) == (True, 0)
