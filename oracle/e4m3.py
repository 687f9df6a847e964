"""OCP E4M3 -- the FP8 operand format of the linear GEMMs.  TEST INFRASTRUCTURE.

The pages name the format only as "E4M3" (arxiv-wiki summary, section
"접근 방법" item (4); paperlayer.ai summary, appendix C "生産学習の詳細",
item "FP8実装pipeline").  Reading taken here: the OCP 8-bit floating point
E4M3 encoding (the one with a largest finite value of 448, not the "FNUZ"
variant with 240):

* bit 7 = sign, bits 6..3 = exponent field E (bias 7), bits 2..0 = mantissa f;
* E in 1..15: value (8 + f) * 2**(E - 10)  (i.e. 1.f * 2**(E-7));
* E == 0: subnormal value f * 2**-9;
* S.1111.111 (0x7F / 0xFF) is NaN; there are no infinities, so the largest
  finite magnitude is 0x7E = 1.75 * 2**8 = 448;
* 0x80 is negative zero.

Conversion from binary32 rounds to the nearest E4M3 value with ties going to
the even mantissa, keeps the sign (also for results that round to zero), and
saturates magnitudes above 448 to 448.  NaN maps to NaN (0x7F with the sign).

Nothing here is vectorised cleverly: the encoder works in float64 on the
exact value of each binary32 input, so every step is an exact operation except
the single rounding ``np.rint`` (round half to even) that the format asks for.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6      # smallest normal magnitude (code 0x08)
_SUB_QUANTUM = 2.0 ** -9     # spacing of subnormals (code 0x01)


def decode(codes):
    """E4M3 codes (uint8 array) -> float64 values (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    normal = (8 + f) * np.ldexp(1.0, (e - 10).astype(np.int32))
    sub = f * _SUB_QUANTUM
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def encode(values):
    """binary32 values -> E4M3 codes (uint8), RNE with saturation at 448.

    Steps (all exact in float64 except the rint):
      1. a = |v|; the spacing of E4M3 values around a is 2**(floor(log2 a)-3)
         for a >= 2**-6 and the subnormal spacing 2**-9 below that;
      2. n = rint(a / spacing) -- round half to even, which is "ties to even
         mantissa" because the mantissa's last bit is n's last bit;
      3. m = n * spacing, clamped to 448 (saturation);
      4. m is an E4M3 value; write its exponent/mantissa fields, add the sign.
    """
    v = np.asarray(values, dtype=np.float32)
    sign = np.signbit(v).astype(np.uint8) << 7
    with np.errstate(invalid="ignore"):      # signalling NaNs raise the invalid flag when widened
        a = np.abs(v).astype(np.float64)
    nan = np.isnan(a)
    inf = np.isinf(a)
    a = np.where(nan | inf, 0.0, a)

    # Step 1: binade exponent of a (frexp gives a = mant * 2**ex, mant in [0.5,1)).
    _, ex = np.frexp(a)
    binade = np.maximum(ex - 1, -6)          # below 2**-6 use the subnormal spacing
    spacing = np.ldexp(1.0, binade - 3)
    # Step 2: round to a whole number of spacings, ties to even.
    n = np.rint(a / spacing)
    # Step 3: the rounded magnitude, saturated.
    m = np.minimum(n * spacing, E4M3_MAX)
    m = np.where(inf, E4M3_MAX, m)

    # Step 4: fields of the E4M3 value m.
    _, mex = np.frexp(m)
    e_unb = mex - 1                           # m = 1.f * 2**e_unb for normals
    is_sub = m < _MIN_NORMAL
    f_norm = np.rint(m / np.ldexp(1.0, e_unb - 3)) - 8
    code_norm = ((e_unb + 7) << 3).astype(np.int64) + f_norm.astype(np.int64)
    code_sub = np.rint(m / _SUB_QUANTUM).astype(np.int64)
    code = np.where(is_sub, code_sub, code_norm).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)
