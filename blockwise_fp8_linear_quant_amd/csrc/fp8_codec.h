// E4M3 codec and exact group quotient for the gfx950 quantisers.
//
// Format: OCP E4M3 (bias 7, largest finite 448, subnormals f*2^-9, S.1111.111
// is NaN), which is what the Puro-2B summaries call the "E4M3" operand format
// of the blockwise FP8 linear GEMMs (arxiv-wiki summary, section "접근 방법",
// item (4)).  Conversion rounds to nearest with ties to even mantissa, keeps
// the sign, and saturates magnitudes above 448.
//
// Quantisation of one group with maximum magnitude amax:
//     s    = fl32(amax / 448)                  (IEEE binary32 division)
//     code = E4M3(fl32(x / s))                  (IEEE binary32 division, then RNE)
// The per-element division is replaced by an exact equivalent that costs one
// ldexp, one multiply and two FMAs:
//   * both x and s are multiplied by 2^k so that s' = s * 2^k lies in [1, 2);
//     the quotient is unchanged and no step can overflow or underflow for any
//     quotient large enough to reach a non-zero E4M3 code;
//   * r = fl32(1 / s') is formed once per group by an IEEE division;
//   * q0 = fl32(x' * r); e = x' - q0 * s' (exact by FMA); q = fl32(q0 + e * r).
// Markstein's theorem (correctly rounded reciprocal, faithful first quotient,
// exact residual, round-to-nearest) makes q the correctly rounded x'/s'.  The
// host build of this header is checked exhaustively on the CPU against IEEE
// division for every pair of BF16 inputs (x, amax) with |x| <= amax.
//
// This header is compiled both for the device (hipcc) and for the host test
// driver (g++), so it uses only plain C++ plus two host/device math calls.
// Floating-point contraction must be off: every rounding is written out.

#pragma once
#include <stdint.h>
#include <string.h>
#include <math.h>

#ifndef FP8BLK_HD
#if defined(__HIPCC__)
#define FP8BLK_HD __host__ __device__ __forceinline__
#else
#define FP8BLK_HD static inline
#endif
#endif

namespace fp8blk {

FP8BLK_HD uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
FP8BLK_HD float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

// Per-group constants of the exact quotient.
struct GroupQ {
  float s;        // stored scale fl32(amax / 448)
  float s_n;      // s * 2^k in [1, 2)
  float r_n;      // fl32(1 / s_n)
  int k;          // power-of-two normalisation
};

FP8BLK_HD GroupQ group_setup(float amax) {
  GroupQ g;
  g.s = amax / 448.0f;
  if (g.s == 0.0f) {           // all-zero group: codes 0x00, scale 0
    g.s_n = 1.0f; g.r_n = 1.0f; g.k = 0;
    return g;
  }
  int e;
  (void)frexpf(g.s, &e);        // s = m * 2^e, m in [0.5, 1)
  g.k = 1 - e;
  g.s_n = ldexpf(g.s, g.k);
  g.r_n = 1.0f / g.s_n;
  return g;
}

// The same constants from a 128-entry table, for group maxima that are BF16
// values (low 16 bits zero).  For a normal BF16 amax = (128 + m) * 2^(e - 134)
// (e the biased exponent, m the 7 stored mantissa bits),
//     amax / 448 = ((128 + m) / 7) * 2^(e - 140),
// and scaling by a power of two commutes with rounding while the result stays
// normal, so fl32(amax / 448) = T(m) * 2^(e - 140) with T(m) = fl32((128+m)/7)
// in [18.28, 36.43].  The table holds T(m) normalised to [1, 2) (by 2^-4, or
// 2^-5 from m = 96 on, where (128 + m) / 7 reaches 32 exactly) and its
// correctly rounded reciprocal; the stored scale is rebuilt with one ldexp.
// Maxima with e < 10 (scales at or below the binary32 normal range), zero,
// and non-finite values take group_setup itself.  Equal to group_setup on
// every BF16 amax (checked exhaustively on the host).
struct SetupEntry {
  float s_n;
  float r_n;
};

FP8BLK_HD SetupEntry setup_entry(int m) {
  const float t = (float)(128 + m) / 7.0f;
  SetupEntry e;
  e.s_n = ldexpf(t, m >= 96 ? -5 : -4);
  e.r_n = 1.0f / e.s_n;
  return e;
}

// The same 128 entries evaluated at compile time (binary32, round to nearest
// even; dividing by 16 or 32 is exact, like the ldexpf of setup_entry), so a
// kernel can copy its table instead of dividing.
struct SetupTable {
  SetupEntry e[128];
};

constexpr SetupTable make_setup_table() {
  SetupTable tb{};
  for (int m = 0; m < 128; ++m) {
    const float t = (float)(128 + m) / 7.0f;
    tb.e[m].s_n = m >= 96 ? t / 32.0f : t / 16.0f;
    tb.e[m].r_n = 1.0f / tb.e[m].s_n;
  }
  return tb;
}

FP8BLK_HD GroupQ group_setup_bf16(float amax, const SetupEntry* tab) {
  const uint32_t b = f32_bits(amax);
  const int e = (int)(b >> 23);
  if (e < 10 || e > 254) return group_setup(amax);
  const int m = (int)((b >> 16) & 0x7fu);
  const SetupEntry t = tab[m];
  GroupQ g;
  g.k = 140 - e - (m >= 96 ? 5 : 4);
  g.s_n = t.s_n;
  g.r_n = t.r_n;
  g.s = ldexpf(t.s_n, -g.k);
  return g;
}

// fl32(x / s) for every x whose quotient can reach a non-zero code; tiny
// quotients (< 2^-12) come out tiny with the right sign, which encodes the same.
FP8BLK_HD float group_quotient(float x, const GroupQ& g) {
  float xn = ldexpf(x, g.k);
  float q0 = xn * g.r_n;
  // en = q0 * s_n - xn, the negated residual (exact).  Written with this sign
  // so that an exact zero residual is +0 and -en = -0 leaves a -0 quotient -0.
  float en = fmaf(q0, g.s_n, -xn);
  return fmaf(-en, g.r_n, q0);
}

// Two-operation form of the same quotient, for groups whose reciprocal is a
// finite binary32 (every BF16 group maximum from about 1.3e-36 up).  With the
// reciprocal split into a double word,
//     rhi = 1 / s rounded down,   rlo = fl32((1 - s * rhi) * rhi) >= 0
// (the residual 1 - s * rhi is exact by FMA, and non-negative because rhi is
// rounded down), the quotient is
//     q = fl32(x * rhi + fl32(x * rlo))          (one multiply, one FMA),
// which carries an error of a few 2^-48 relative before its single rounding;
// rlo >= 0 keeps the sign of a zero x.  It yields the same E4M3 code as
// E4M3(fl32(x / s)) for every pair of BF16 values with |x| <= amax, both
// signs (checked exhaustively on the host, with the constants formed exactly
// as here from the table-driven setup); the binary32 quotient itself may
// differ in its last place where the code cannot.  Zero groups get
// rhi = -0 and rlo = +0: their elements are +-0, and x * (-0) + x * (+0) is
// +0 for both signs of zero, so their codes come out 0x00 with no mask.
struct GroupQ2 {
  float rhi;
  float rlo;
};

// The two-operation constants of group g; false if 1 / s overflows binary32,
// in which case the caller must use group_quotient.
FP8BLK_HD bool group_setup2(const GroupQ& g, GroupQ2& o) {
  o.rhi = -0.0f;
  o.rlo = 0.0f;
  if (g.s == 0.0f) return true;
  // fl32(1 / s) = 2^k * fl32(1 / s_n) exactly: the scaling is by a power of
  // two and the result is a normal binary32 (or overflows to infinity).
  float rhi = ldexpf(g.r_n, g.k);
  if (!(rhi <= 3.4028234663852886e38f)) return false;
  // Round down: if fl32(1 / s) rounded up (negative residual), step to the
  // binary32 below it (rhi is a positive normal, so its bit pattern minus one).
  if (fmaf(-g.s, rhi, 1.0f) < 0.0f) rhi = bits_f32(f32_bits(rhi) - 1u);
  o.rhi = rhi;
  o.rlo = fmaf(-g.s, rhi, 1.0f) * rhi;
  return true;
}

FP8BLK_HD float group_quotient2(float x, const GroupQ2& g) { return fmaf(x, g.rhi, x * g.rlo); }

// binary32 -> OCP E4M3 code (low 8 bits), RNE, saturating, sign kept.
FP8BLK_HD uint32_t e4m3_encode(float q) {
  uint32_t u = f32_bits(q);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  // Normal results (|q| >= 2^-6): round the binary32 mantissa to 3 bits, ties
  // to even, then move the exponent bias from 127 to 7 (120 << 3 = 960).
  uint32_t rn = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  uint32_t code_n = rn - 960u;
  // Subnormal results (|q| < 2^-6): round |q| * 2^9 to an integer, ties to
  // even, by adding 1.5 * 2^23 (the sum's unit in the last place is 1).
  float t = bits_f32(a) * 512.0f;
  t = t + 12582912.0f;
  uint32_t code_s = f32_bits(t) - 0x4b400000u;
  uint32_t code = (a < 0x3c800000u) ? code_s : code_n;
  code = code < 0x7eu ? code : 0x7eu;           // saturate at 448
  code = (a > 0x7f800000u) ? 0x7fu : code;      // NaN stays NaN
  return code | sign;
}

// BF16 bit pattern -> binary32 (exact).
FP8BLK_HD float bf16_to_f32(uint32_t b) { return bits_f32(b << 16); }

// binary32 -> BF16 bits, round to nearest even (finite inputs).
FP8BLK_HD uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace fp8blk
