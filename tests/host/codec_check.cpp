// Host build of the device codec (csrc/fp8_codec.h) for CPU checks.
//
// 1. main(): exhaustive proof that the kernels' exact-quotient shortcut gives
//    the same E4M3 code as IEEE division fl32(x / fl32(amax / 448)) for every
//    pair of BF16 values (x, amax) with |x| <= amax, and the same binary32
//    quotient whenever that quotient is >= 2^-12.
// 2. codec_encode(): the device encoder, exported for a ctypes comparison with
//    the oracle's encoder.
#include <cstdio>
#include <cstdint>
#include <cmath>
#include "fp8_codec.h"

extern "C" void codec_encode(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)fp8blk::e4m3_encode(in[i]);
}

extern "C" int codec_quotient_scan(uint32_t amax_lo, uint32_t amax_hi, uint64_t* n_checked) {
  long long bad = 0;
  unsigned long long checked = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : bad, checked)
  for (uint32_t ab = amax_lo; ab < amax_hi; ++ab) {
    float amax = fp8blk::bf16_to_f32(ab);
    fp8blk::GroupQ g = fp8blk::group_setup(amax);
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      for (uint32_t sgn = 0; sgn < 2; ++sgn) {
        float x = fp8blk::bf16_to_f32(xb | (sgn << 15));
        float qf = fp8blk::group_quotient(x, g);
        float qr = x / g.s;
        ++checked;
        uint32_t cf = fp8blk::e4m3_encode(qf), cr = fp8blk::e4m3_encode(qr);
        bool ok = (cf == cr);
        if (std::fabs(qr) >= 0x1p-12f) ok = ok && (fp8blk::f32_bits(qf) == fp8blk::f32_bits(qr));
        else ok = ok && std::fabs(qf) < 0x1p-11f && std::signbit(qf) == std::signbit(qr);
        if (!ok) {
          if (bad < 10)
            std::printf("MISMATCH amax=%#x x=%#x fast=%a ref=%a codes %#x %#x\n", ab, xb | (sgn << 15),
                        qf, qr, cf, cr);
          ++bad;
        }
      }
    }
  }
  if (n_checked) *n_checked = checked;
  return (int)(bad > 0x7fffffff ? 0x7fffffff : bad);
}

// The two-operation quotient (group_setup2 / group_quotient2, constants from
// the table-driven setup as in the kernels) against IEEE division, both signs,
// for every BF16 pair with |x| <= amax whose reciprocal is finite: returns the
// number of pairs whose E4M3 codes differ.  *n_checked counts the pairs,
// *n_q_diff those whose binary32 quotients differ (allowed), *n_skipped the
// maxima whose reciprocal overflows (they keep the normalised quotient).
extern "C" int codec_quotient2_scan(uint64_t* n_checked, uint64_t* n_q_diff, uint64_t* n_skipped) {
  static constexpr fp8blk::SetupTable kTab = fp8blk::make_setup_table();
  long long bad = 0;
  unsigned long long checked = 0, qdiff = 0, skipped = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : bad, checked, qdiff, skipped)
  for (uint32_t ab = 1; ab < 0x7f80; ++ab) {
    const float amax = fp8blk::bf16_to_f32(ab);
    const fp8blk::GroupQ g = fp8blk::group_setup_bf16(amax, kTab.e);
    fp8blk::GroupQ2 g2;
    if (!fp8blk::group_setup2(g, g2)) {
      ++skipped;
      continue;
    }
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      for (uint32_t sgn = 0; sgn < 2; ++sgn) {
        const float x = fp8blk::bf16_to_f32(xb | (sgn << 15));
        const float q2 = fp8blk::group_quotient2(x, g2);
        const float qr = x / g.s;
        ++checked;
        qdiff += fp8blk::f32_bits(q2) != fp8blk::f32_bits(qr);
        const uint32_t c2 = fp8blk::e4m3_encode(q2), cr = fp8blk::e4m3_encode(qr);
        if (c2 != cr) {
          if (bad < 10) std::printf("QUOTIENT2 MISMATCH amax=%#x x=%#x q2=%a ref=%a codes %#x %#x\n", ab,
                                    xb | (sgn << 15), q2, qr, c2, cr);
          ++bad;
        }
      }
    }
  }
  // A zero group (amax = 0): both signed zeros must give code 0x00 (no mask).
  {
    const fp8blk::GroupQ g = fp8blk::group_setup(0.0f);
    fp8blk::GroupQ2 g2;
    const bool ok2 = fp8blk::group_setup2(g, g2);
    const uint32_t zeros[2] = {0x0000u, 0x8000u};
    for (uint32_t xb : zeros) {
      const uint32_t code = fp8blk::e4m3_encode(fp8blk::group_quotient2(fp8blk::bf16_to_f32(xb), g2));
      if (!ok2 || code != 0u) {
        std::printf("ZERO GROUP x=%#x code %#x\n", xb, code);
        ++bad;
      }
    }
  }
  if (n_checked) *n_checked = checked;
  if (n_q_diff) *n_q_diff = qdiff;
  if (n_skipped) *n_skipped = skipped;
  return (int)(bad > 0x7fffffff ? 0x7fffffff : bad);
}

// Table-driven group setup against group_setup for every BF16 magnitude:
// returns the number of maxima whose four constants differ in any bit.  The
// table is the compile-time one the kernels copy; its entries must also equal
// setup_entry's, evaluated at run time.
extern "C" int codec_setup_table_scan(void) {
  static constexpr fp8blk::SetupTable kTab = fp8blk::make_setup_table();
  const fp8blk::SetupEntry* tab = kTab.e;
  int bad = 0;
  for (int m = 0; m < 128; ++m) {
    const fp8blk::SetupEntry r = fp8blk::setup_entry(m);
    if (fp8blk::f32_bits(r.s_n) != fp8blk::f32_bits(tab[m].s_n) || fp8blk::f32_bits(r.r_n) != fp8blk::f32_bits(tab[m].r_n)) {
      std::printf("TABLE MISMATCH m=%d\n", m);
      ++bad;
    }
  }
  for (uint32_t ab = 0; ab < 0x7f80; ++ab) {
    const float amax = fp8blk::bf16_to_f32(ab);
    const fp8blk::GroupQ a = fp8blk::group_setup(amax), b = fp8blk::group_setup_bf16(amax, tab);
    const bool same = fp8blk::f32_bits(a.s) == fp8blk::f32_bits(b.s) && a.k == b.k &&
                      (a.s == 0.0f || (fp8blk::f32_bits(a.s_n) == fp8blk::f32_bits(b.s_n) &&
                                       fp8blk::f32_bits(a.r_n) == fp8blk::f32_bits(b.r_n)));
    if (!same) {
      if (bad < 10) std::printf("SETUP MISMATCH amax=%#x s %a %a k %d %d\n", ab, a.s, b.s, a.k, b.k);
      ++bad;
    }
  }
  return bad;
}

int main() {
  uint64_t n = 0;
  int bad = codec_quotient_scan(1, 0x7f80, &n);
  std::printf("checked %llu pairs, %d mismatches\n", (unsigned long long)n, bad);
  return bad != 0;
}
