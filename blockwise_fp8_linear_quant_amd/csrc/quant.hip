// Blockwise E4M3 quantisers for gfx950 (HBM-streaming kernels).
//
// Pages: arxiv-wiki summary of Puro-2B, section "접근 방법" item (4) -- FP8
// E4M3 values with one scale per 1-D group of 128 activations and one per
// 128x128 weight block; paperlayer.ai summary, appendix C "生産学習の詳細",
// item "FP8実装pipeline" -- all three GEMMs of a linear layer (forward, data
// gradient, weight gradient) take such operands.
//
// Every kernel reads BF16 once with 16-byte loads, reduces the group maximum
// exactly (max of |x| in binary32), forms s = fl32(amax / 448) and writes
// E4M3(fl32(x / s)) with the exact quotient of fp8_codec.h and the hardware
// round-to-nearest-even conversion (see enc4).  Zero groups get s = 0 and
// codes 0x00.
#include "internal.h"
#include "fp8_codec.h"

namespace fp8blk {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_fmax(float v) {
  int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}
// DPP controls (gfx9): quad_perm [1,0,3,2] = xor 1, quad_perm [2,3,0,1] = xor 2,
// row_half_mirror reverses each 8-lane half, row_ror:8 = xor 8 inside a row of 16.
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kRor8 = 0x128;

// Max over the 8 lanes {8a .. 8a+7}.
__device__ __forceinline__ float max8(float v) {
  v = dpp_fmax<kXor1>(v);
  v = dpp_fmax<kXor2>(v);
  return dpp_fmax<kHalfMirror>(v);
}

// Eight BF16 values starting at column col of a row; columns >= C read as +0.
__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ row, int64_t col, int64_t C) {
  if (col + 8 <= C) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + col));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  uint32_t w[4] = {0, 0, 0, 0};
  for (int i = 0; i < 8; ++i)
    if (col + i < C) w[i >> 1] |= (uint32_t)row[col + i] << ((i & 1) * 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Eight BF16 values at p (the caller guarantees they are all in bounds).
__device__ __forceinline__ uint4 load8_full(const uint16_t* __restrict__ p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float elem(const uint4& v, int i) {
  const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
  return (i & 1) ? bits_f32(w & 0xffff0000u) : bits_f32(w << 16);
}

// Hardware E4M3 conversion.  v_cvt_pk_fp8_f32 rounds to nearest even with
// subnormals and signed zeros exactly like the format definition for every
// |v| < 464 (checked exhaustively against the software encoder on gfx950);
// at 464 and above it returns NaN instead of saturating.  Group quotients are
// at most ~449.5 in magnitude (|x| <= amax and s = fl32(amax / 448), even for
// denormal s), so the quantisers use it directly.
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0, 1
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);  // bytes 2, 3
}

// Codes of four values of one group, packed little-endian into a dword.
__device__ __forceinline__ uint32_t code4(float a, float b, float c, float d, const GroupQ& g) {
  return enc4(group_quotient(a, g), group_quotient(b, g), group_quotient(c, g), group_quotient(d, g));
}
// The same with the two-operation quotient (groups whose reciprocal is finite).
__device__ __forceinline__ uint32_t code4(float a, float b, float c, float d, const GroupQ2& g) {
  return enc4(group_quotient2(a, g), group_quotient2(b, g), group_quotient2(c, g), group_quotient2(d, g));
}

// True in every lane if every active lane's flag is true (a wave vote, so a
// branch on it is uniform).
__device__ __forceinline__ bool wave_all(bool v) { return __all(v ? 1 : 0) != 0; }

// Any binary32 -> E4M3 code: hardware below 464, saturation at and above it
// (infinities included), and S.1111.111 (0x7F with the sign) for NaN.
__device__ __forceinline__ uint32_t encode_any(float x) {
  const uint32_t u = f32_bits(x), a = u & 0x7fffffffu;
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xffu;
  if (a >= 0x43e80000u) c = (a > 0x7f800000u ? 0x7fu : 0x7eu) | ((u >> 24) & 0x80u);
  return c;
}

// 4x4 byte transpose: rows r[0..3] (byte j = column j) -> columns c[0..3]
// (byte i = row i).  v_perm_b32 picks bytes of (S0 << 32 | S1).
__device__ __forceinline__ void transpose4x4(const uint32_t (&r)[4], uint32_t (&c)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  const uint32_t t1 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  const uint32_t t2 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Store 8 code bytes at p[0..7], only columns col+i < C.
__device__ __forceinline__ void store8(uint8_t* __restrict__ p, int64_t col, int64_t C, uint32_t lo, uint32_t hi) {
  if (col + 8 <= C) {
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    return;
  }
  for (int i = 0; i < 8; ++i)
    if (col + i < C) p[i] = (uint8_t)(((i < 4) ? lo : hi) >> ((i & 3) * 8));
}

// LDS-only workgroup barrier: lgkmcnt(0), then s_barrier.  __syncthreads()
// would also make every wave wait for its outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x3 << 14));   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposed codes of a 128x128 tile.  Thread (rb, c) = (t / 16, t % 16)
// holds, in cw[j], the 8 codes of column 8c + j for tile rows 8rb .. 8rb + 7.
// Written straight to global memory those are 8-byte pieces 32 bytes apart;
// instead the tile goes through `stage` (16 KB of LDS) so that every column's
// 128 bytes leave as 8 consecutive lanes x 16 bytes.  Row `col` of the stage
// holds 16 slots of 8 bytes, slot s at s ^ 2((col / 8) % 8): 16-byte pairs stay
// together and a wave's writes spread over the banks.  dst points at column 0,
// row 0 of the tile (rows contiguous, ld bytes between columns); columns at or
// beyond ncols are not written.  All 256 threads must call it.
__device__ __forceinline__ void store_codes_transposed(const uint32_t (&cw)[8][2], uint4* stage, uint8_t* dst,
                                                       int64_t ld, int64_t ncols) {
  const int t = threadIdx.x, c = t & 15, rb = t >> 4;
  uint8_t* st = reinterpret_cast<uint8_t*>(stage);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = 8 * c + j;
    *reinterpret_cast<uint2*>(st + col * 128 + (rb ^ (2 * (c & 7))) * 8) = make_uint2(cw[j][0], cw[j][1]);
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int id = t + 256 * u, col = id >> 3, k = id & 7;
    const uint4 w = *reinterpret_cast<const uint4*>(st + col * 128 + ((2 * k) ^ (2 * ((col >> 3) & 7))) * 8);
    if (col < ncols) *reinterpret_cast<uint4*>(dst + col * ld + 16 * k) = w;
  }
}

// ---------------------------------------------------------------------------
// Row-wise 1x128: a wave quantises 8 rows x one 128-column group; lane (r, c)
// with r = lane/8, c = lane%8 holds columns [8c, 8c+8) and [64+8c, 64+8c+8)
// so each load instruction covers 128 contiguous bytes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 8 + (lane >> 3);
  const int64_t g = blockIdx.y;
  const int c = lane & 7;
  const int64_t col0 = g * 128 + c * 8;
  const int64_t col1 = col0 + 64;
  const bool row_ok = row < R;

  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
  if (row_ok) {
    const uint16_t* p = x + row * ldx;
    v0 = load8(p, col0, C);
    v1 = load8(p, col1, C);
  }
  float f[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = elem(v0, i);
    f[8 + i] = elem(v1, i);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = max8(amax);

  const GroupQ gq = group_setup(amax);
  GroupQ2 g2;
  const bool fast = wave_all(group_setup2(gq, g2));
  const uint32_t keep = (gq.s == 0.0f) ? 0u : 0xffffffffu;   // zero group -> codes 0x00
  uint32_t w[4];
  if (fast) {   // zero groups come out 0x00 by themselves (group_setup2)
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = code4(f[4 * d], f[4 * d + 1], f[4 * d + 2], f[4 * d + 3], g2);
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = keep & code4(f[4 * d], f[4 * d + 1], f[4 * d + 2], f[4 * d + 3], gq);
  }
  if (row_ok) {
    uint8_t* qr = q + row * ldq;
    if (col0 < C) store8(qr + col0, col0, C, w[0], w[1]);
    if (col1 < C) store8(qr + col1, col1, C, w[2], w[3]);
    if (c == 0) s[g * lds + row] = gq.s;
  }
}

// ---------------------------------------------------------------------------
// Token-dimension 1x128 with transposed output: a wave quantises 128 tokens x
// 64 features.  Lane (b, c), b = lane/8, c = lane%8, loads tokens
// [16b, 16b+16) x features [8c, 8c+8) (16-byte loads, 128 contiguous bytes
// per token row per instruction) and writes, for each of its 8 features, the
// 16 codes of its tokens as one 16-byte store -- the transpose happens in
// registers.  The per-feature maximum over 128 tokens is a reduction over the
// 8 lanes sharing c (lane distance 8, 16, 32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_tokens_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t C, int64_t ldx,
    uint8_t* __restrict__ qT, int64_t ldq, float* __restrict__ s, int64_t lds, uint32_t nfb) {
  const int lane = threadIdx.x & 63;
  // One-dimensional grid (token groups can exceed the 65535 limit of y):
  // workgroup (token group, feature block) in feature-fastest order.
  const int64_t tg = blockIdx.x / nfb, fb = blockIdx.x % nfb;
  const int64_t f0 = (fb * 4 + (threadIdx.x >> 6)) * 64 + (lane & 7) * 8;
  const int b = lane >> 3;
  const int64_t t0 = tg * 128 + b * 16;

  uint4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t tok = t0 + i;
    v[i] = (tok < M && f0 < C) ? load8(x + tok * ldx, f0, C) : make_uint4(0, 0, 0, 0);
  }
  float am[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(elem(v[i], j)));
    m = dpp_fmax<kRor8>(m);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    am[j] = m;
  }
  // Two-operation constants and scales of the 8 groups; the normalised
  // constants are formed again only if some group of the wave needs them.
  GroupQ2 g2[8];
  float sc[8];
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const GroupQ gq = group_setup(am[j]);
    ok = group_setup2(gq, g2[j]) && ok;
    sc[j] = gq.s;
  }
  const bool fast = wave_all(ok);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
    if (fast) {   // zero groups come out 0x00 by themselves (group_setup2)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        w[d] = code4(elem(v[4 * d], j), elem(v[4 * d + 1], j), elem(v[4 * d + 2], j), elem(v[4 * d + 3], j), g2[j]);
    } else {
      const uint32_t keep = (sc[j] == 0.0f) ? 0u : 0xffffffffu;
      const GroupQ gq = group_setup(am[j]);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        w[d] = keep & code4(elem(v[4 * d], j), elem(v[4 * d + 1], j), elem(v[4 * d + 2], j), elem(v[4 * d + 3], j),
                            gq);
    }
    if (f0 + j < C) {
      *reinterpret_cast<uint4*>(qT + (f0 + j) * ldq + t0) = make_uint4(w[0], w[1], w[2], w[3]);
      if (b == 0) s[tg * lds + f0 + j] = sc[j];
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks: a 256-thread workgroup quantises one block.  Thread (rb, c),
// rb = t/16, c = t%16, holds rows [8rb, 8rb+8) x columns [8c, 8c+8); the block
// maximum is reduced in the wave and across the 4 waves through LDS.  The
// optional transposed copy is written from the same registers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_blocks_kernel(
    const uint16_t* __restrict__ w, int64_t R, int64_t C, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ sT, uint32_t nbc) {
  __shared__ float red[4];
  __shared__ uint4 stage[1024];      // transposed code tile (store_codes_transposed)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;   // one-dimensional grid, column tiles fastest
  const int c = t & 15, rb = t >> 4;
  const int64_t r0 = br * 128 + rb * 8, c0 = bc * 128 + c * 8;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + i;
    v[i] = (r < R && c0 < C) ? load8(w + r * ldw, c0, C) : make_uint4(0, 0, 0, 0);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem(v[i], j)));
  m = max8(m);
  m = dpp_fmax<kRor8>(m);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const GroupQ gq = group_setup(m);
  GroupQ2 g2;
  const bool fast = group_setup2(gq, g2);   // one group per workgroup: uniform
  const uint32_t keep = (gq.s == 0.0f) ? 0u : 0xffffffffu;
  // Row-major codes: rw[i][0] = columns 0..3 of row i, rw[i][1] = columns 4..7.
  uint32_t rw[8][2];
  if (fast) {   // a zero block comes out 0x00 by itself (group_setup2)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        rw[i][hh] = code4(elem(v[i], 4 * hh), elem(v[i], 4 * hh + 1), elem(v[i], 4 * hh + 2), elem(v[i], 4 * hh + 3),
                          g2);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        rw[i][hh] = keep & code4(elem(v[i], 4 * hh), elem(v[i], 4 * hh + 1), elem(v[i], 4 * hh + 2),
                                 elem(v[i], 4 * hh + 3), gq);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (r0 + i < R && c0 < C) store8(q + (r0 + i) * ldq + c0, c0, C, rw[i][0], rw[i][1]);
  if (qT != nullptr) {
    // Transposed copy: column j of this thread's 8x8 block = rows 0..7 of it.
    uint32_t cw[8][2];
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t rr[4] = {rw[4 * rb2][hh], rw[4 * rb2 + 1][hh], rw[4 * rb2 + 2][hh], rw[4 * rb2 + 3][hh]};
        uint32_t cc[4];
        transpose4x4(rr, cc);
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[4 * hh + j][rb2] = cc[j];
      }
    if ((br + 1) * 128 <= R) {
      // Whole 128-row block: every column's 128 codes are in range.
      store_codes_transposed(cw, stage, qT + bc * 128 * ldqT + br * 128, ldqT, C - bc * 128);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < C && r0 < R) store8(qT + (c0 + j) * ldqT + r0, r0, R, cw[j][0], cw[j][1]);
    }
  }
  if (t == 0) {
    const int64_t nbr = (R + 127) / 128, nbc = (C + 127) / 128;
    s[br * nbc + bc] = gq.s;
    if (sT != nullptr) sT[bc * nbr + br] = gq.s;
  }
}

__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ x, uint8_t* __restrict__ q, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) q[i] = (uint8_t)encode_any(x[i]);
}

// ---------------------------------------------------------------------------
// Both 1x128 orientations from one read: a 256-thread workgroup takes a tile
// of 128 rows (tokens) x 128 columns (features), thread (rb, c), rb = t/16,
// c = t%16, holding rows [8rb, 8rb+8) x columns [8c, 8c+8) as in the block
// quantiser.  Row maxima (groups along the columns) are reduced over the 16
// lanes of a DPP row; column maxima (groups along the tokens) over lanes 16
// and 32 apart and then across the 4 waves through LDS.  Each element is
// encoded twice -- with its row's scale into q (row-wise layout) and with its
// column's scale into qT (transposed, tokens contiguous) -- so the outputs are
// those of the two separate quantisers, bit for bit, for 2 bytes read instead
// of 4.  Token rows past R (up to the 128-padded length) read as zero and
// come out as 0x00 pads in qT.
// ---------------------------------------------------------------------------
__device__ constexpr SetupTable kSetupTab = make_setup_table();

__device__ __forceinline__ uint32_t code4_each(float a, float b, float c, float d, const GroupQ (&g)[8], int j0) {
  // Four values of one row, columns j0..j0+3, each with its own column's
  // scale.  A zero column group has s_n = r_n = 1, k = 0 and only +-0
  // elements, so its quotients are +-0; the caller masks those bytes to 0x00.
  return enc4(group_quotient(a, g[j0 + 0]), group_quotient(b, g[j0 + 1]), group_quotient(c, g[j0 + 2]),
              group_quotient(d, g[j0 + 3]));
}
// The same with the two-operation quotient (zero column groups: rhi = rlo = 0).
__device__ __forceinline__ uint32_t code4_each(float a, float b, float c, float d, const GroupQ2 (&g)[8], int j0) {
  return enc4(group_quotient2(a, g[j0 + 0]), group_quotient2(b, g[j0 + 1]), group_quotient2(c, g[j0 + 2]),
              group_quotient2(d, g[j0 + 3]));
}

// Element sources of the dual quantiser: eight BF16 values (bit patterns) of
// row r starting at column c0, columns >= C as +0.
struct SrcPlain {   // a BF16 tensor
  const uint16_t* x;
  int64_t ldx;
  __device__ __forceinline__ uint4 load(int64_t r, int64_t c0, int64_t C) const { return load8(x + r * ldx, c0, C); }
  __device__ __forceinline__ uint4 load_full(int64_t r, int64_t c0) const { return load8_full(x + r * ldx + c0); }
};

// Two binary32 values -> packed BF16, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950).  It equals f32_to_bf16_rne on every binary32
// input except NaNs (checked exhaustively on gfx950), so the fused
// producers' BF16 values, and the codes formed from them, are unchanged.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// SwiGLU of the gate and up halves of the gate_up projection: silu(g) * u
// evaluated in binary32 (g * (1 / (1 + e^-g)) then times u), rounded once to
// BF16 -- the down projection's BF16 input, produced in registers.
struct SrcSwiGLU {
  const uint16_t* g;
  int64_t ldg;
  const uint16_t* u;
  int64_t ldu;
  __device__ __forceinline__ uint4 load(int64_t r, int64_t c0, int64_t C) const {
    return combine(load8(g + r * ldg, c0, C), load8(u + r * ldu, c0, C));
  }
  __device__ __forceinline__ uint4 load_full(int64_t r, int64_t c0) const {
    return combine(load8_full(g + r * ldg + c0), load8_full(u + r * ldu + c0));
  }
  __device__ __forceinline__ uint4 combine(const uint4 a, const uint4 b) const {
    float h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gj = elem(a, j);
      h[j] = (gj / (1.0f + expf(-gj))) * elem(b, j);
    }
    return make_uint4(pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]), pack_bf16(h[6], h[7]));
  }
};

// RMSNorm output x * rstd(row) * gamma(col) in binary32, rounded once to BF16,
// with rstd from rmsnorm_rstd_kernel.
struct SrcRMSNorm {
  const uint16_t* x;
  int64_t ldx;
  const float* rstd;
  const uint16_t* gamma;
  __device__ __forceinline__ uint4 load(int64_t r, int64_t c0, int64_t C) const {
    return combine(load8(x + r * ldx, c0, C), load8(gamma, c0, C), rstd[r]);
  }
  __device__ __forceinline__ uint4 load_full(int64_t r, int64_t c0) const {
    return combine(load8_full(x + r * ldx + c0), load8_full(gamma + c0), rstd[r]);
  }
  __device__ __forceinline__ uint4 combine(const uint4 a, const uint4 w, const float rs) const {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (elem(a, j) * rs) * elem(w, j);
    return make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7]));
  }
};

// Maxima, codes and stores of one 128x128 tile whose values thread (rb, c)
// holds in v[8] (rows 8rb..8rb+7, columns 8c..8c+7).  cred: this tile's
// column-maximum exchange buffer.
template <bool FULL>
__device__ __forceinline__ void dual_encode(
    const uint4 (&v)[8], int64_t br, int64_t bc, int64_t R, int64_t C,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ sT, int64_t ldsT,
    float (*cred)[128], const SetupEntry* stab, uint4* stage, float4* rowq, float4* colq,
    float2* rowq2, float2* colq2, int* tiny) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t & 15, rb = t >> 4;
  const int64_t r0 = br * 128 + rb * 8, c0 = bc * 128 + c * 8;
  // Column maxima of this thread's 8 columns over its 8 rows, then over the
  // 4 row blocks of the wave (lanes 16 and 32 apart); after the barrier
  // thread t < 128 combines the 4 waves' maxima of column t.
  float cm[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(elem(v[i], j)));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    cm[j] = m;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) cred[wave][c * 8 + j] = cm[j];
  }
  // Row maxima over the 16 lanes of a DPP row (the 128 columns of the tile).
  float rm[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem(v[i], j)));
    m = max8(m);
    rm[i] = dpp_fmax<kRor8>(m);
  }
  // LDS-only barrier, so that a fused producer's BF16 stores stay in flight.
  lds_barrier();
  const int tt = t & 127;
  const float cmx = fmaxf(fmaxf(cred[0][tt], cred[1][tt]), fmaxf(cred[2][tt], cred[3][tt]));

  // Group constants are set up once per group and shared through LDS (each
  // thread would otherwise set up all 16 of its groups): lane c < 8 of each
  // DPP row sets up row r0 + c (all 16 lanes hold the 8 row maxima) and
  // stores its scale, thread t < 128 does the same for column t.  The tables
  // are index-major (rowq[i][rb], colq[j][c]): the 16 lanes of a read either
  // share one row entry or take 16 consecutive column entries, free of bank
  // conflicts.  rowq2/colq2 hold the two-operation constants {rhi, rlo};
  // a group whose reciprocal overflows sets *tiny, and the whole tile then
  // takes the normalised quotient from rowq/colq {s_n, r_n, k, s}.
  {
    float m = rm[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = (c == i) ? rm[i] : m;
    if (c < 8) {
      const GroupQ g = group_setup_bf16(m, stab);
      GroupQ2 g2;
      if (!group_setup2(g, g2)) *tiny = 1;
      rowq[c * 16 + rb] = make_float4(g.s_n, g.r_n, __int_as_float(g.k), g.s);
      rowq2[c * 16 + rb] = make_float2(g2.rhi, g2.rlo);
      if (FULL || r0 + c < R) s[bc * lds + r0 + c] = g.s;
    }
  }
  if (t < 128) {
    const GroupQ g = group_setup_bf16(cmx, stab);
    GroupQ2 g2;
    if (!group_setup2(g, g2)) *tiny = 1;
    colq[(t & 7) * 16 + (t >> 3)] = make_float4(g.s_n, g.r_n, __int_as_float(g.k), g.s);
    colq2[(t & 7) * 16 + (t >> 3)] = make_float2(g2.rhi, g2.rlo);
    if (FULL || bc * 128 + t < C) sT[br * ldsT + bc * 128 + t] = g.s;
  }
  lds_barrier();
  uint32_t rw[8][2];
  if (*tiny == 0) {
    // Zero groups come out 0x00 by themselves here (group_setup2).
    GroupQ2 gc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 e = colq2[j * 16 + c];
      gc[j].rhi = e.x; gc[j].rlo = e.y;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 e = rowq2[i * 16 + rb];
      GroupQ2 g;
      g.rhi = e.x; g.rlo = e.y;
      const uint32_t lo = code4(elem(v[i], 0), elem(v[i], 1), elem(v[i], 2), elem(v[i], 3), g);
      const uint32_t hi = code4(elem(v[i], 4), elem(v[i], 5), elem(v[i], 6), elem(v[i], 7), g);
      rw[i][0] = code4_each(elem(v[i], 0), elem(v[i], 1), elem(v[i], 2), elem(v[i], 3), gc, 0);
      rw[i][1] = code4_each(elem(v[i], 4), elem(v[i], 5), elem(v[i], 6), elem(v[i], 7), gc, 4);
      const int64_t r = r0 + i;
      if (FULL) {
        *reinterpret_cast<uint2*>(q + r * ldq + c0) = make_uint2(lo, hi);
      } else if (r < R && c0 < C) {
        store8(q + r * ldq + c0, c0, C, lo, hi);
      }
    }
  } else {
    GroupQ gc[8];
    uint32_t cmask[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 e = colq[j * 16 + c];
      gc[j].s_n = e.x; gc[j].r_n = e.y; gc[j].k = __float_as_int(e.z); gc[j].s = e.w;
      if (e.w != 0.0f) cmask[j >> 2] |= 0xffu << (8 * (j & 3));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 e = rowq[i * 16 + rb];
      GroupQ g;
      g.s_n = e.x; g.r_n = e.y; g.k = __float_as_int(e.z); g.s = e.w;
      const uint32_t keep = (g.s == 0.0f) ? 0u : 0xffffffffu;
      const uint32_t lo = keep & code4(elem(v[i], 0), elem(v[i], 1), elem(v[i], 2), elem(v[i], 3), g);
      const uint32_t hi = keep & code4(elem(v[i], 4), elem(v[i], 5), elem(v[i], 6), elem(v[i], 7), g);
      rw[i][0] = cmask[0] & code4_each(elem(v[i], 0), elem(v[i], 1), elem(v[i], 2), elem(v[i], 3), gc, 0);
      rw[i][1] = cmask[1] & code4_each(elem(v[i], 4), elem(v[i], 5), elem(v[i], 6), elem(v[i], 7), gc, 4);
      const int64_t r = r0 + i;
      if (FULL) {
        *reinterpret_cast<uint2*>(q + r * ldq + c0) = make_uint2(lo, hi);
      } else if (r < R && c0 < C) {
        store8(q + r * ldq + c0, c0, C, lo, hi);
      }
    }
  }
  // Token-dimension codes: 4x4 byte transposes into words of 4 tokens each.
  uint32_t cw[8][2];
#pragma unroll
  for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t rr4[4] = {rw[4 * rb2][hh], rw[4 * rb2 + 1][hh], rw[4 * rb2 + 2][hh], rw[4 * rb2 + 3][hh]};
      uint32_t cc[4];
      transpose4x4(rr4, cc);
#pragma unroll
      for (int j = 0; j < 4; ++j) cw[4 * hh + j][rb2] = cc[j];
    }
  // Token rows past R hold 0x00 codes: the padded layout stores them as pads.
  store_codes_transposed(cw, stage, qT + bc * 128 * ldqT + br * 128, ldqT, FULL ? 128 : C - bc * 128);
}

// The dual quantiser over any element source, one 128x128 tile per workgroup
// (row tile blockIdx.x / nbc, column tile blockIdx.x % nbc); interior tiles
// take unguarded loads and stores.
// `hout` (optional, BF16 [R, ld_h]) receives the source values themselves --
// for a fused producer, the BF16 tensor it would otherwise have written.
template <class Src>
__global__ __launch_bounds__(256) void quant_dual_kernel(
    Src src, int64_t R, int64_t C,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ sT, int64_t ldsT,
    uint16_t* __restrict__ hout, int64_t ldh, uint32_t nbc) {
  __shared__ float cred[4][128];
  __shared__ SetupEntry stab[128];   // group constants by BF16 significand (see group_setup_bf16)
  __shared__ uint4 stage[1024];      // transposed code tile (store_codes_transposed)
  __shared__ float4 rowq[128], colq[128];   // per-group constants {s_n, r_n, k, s} of the tile
  __shared__ float2 rowq2[128], colq2[128]; // two-operation constants {rhi, rlo}
  __shared__ int tiny;                       // some group of the tile has no finite reciprocal
  const int t = threadIdx.x;
  if (t < 128) stab[t] = kSetupTab.e[t];
  if (t == 0) tiny = 0;
  const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;   // one-dimensional grid, column tiles fastest
  const bool full = (br + 1) * 128 <= R && (bc + 1) * 128 <= C;
  const int c = t & 15, rb = t >> 4;
  const int64_t r0 = br * 128 + rb * 8, c0 = bc * 128 + c * 8;
  uint4 v[8];
  if (full) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src.load_full(r0 + i, c0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + i;
      v[i] = (r < R && c0 < C) ? src.load(r, c0, C) : make_uint4(0, 0, 0, 0);
    }
  }
  if (hout != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + i;
      if (r < R && c0 < C) {
        uint16_t* p = hout + r * ldh + c0;
        if (c0 + 8 <= C) {
          *reinterpret_cast<uint4*>(p) = v[i];
        } else {
          const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          for (int j = 0; j < 8; ++j)
            if (c0 + j < C) p[j] = (uint16_t)(w[j >> 1] >> ((j & 1) * 16));
        }
      }
    }
  }
  if (full)
    dual_encode<true>(v, br, bc, R, C, q, ldq, s, lds, qT, ldqT, sT, ldsT, cred, stab, stage, rowq, colq, rowq2, colq2,
                      &tiny);
  else
    dual_encode<false>(v, br, bc, R, C, q, ldq, s, lds, qT, ldqT, sT, ldsT, cred, stab, stage, rowq, colq, rowq2,
                       colq2, &tiny);
}

// RMSNorm statistics: rstd[r] = 1 / sqrt(mean_c x[r, c]^2 + eps) in binary32,
// one wave per row (squares are exact in binary32; the sum is accumulated per
// lane over 8-element chunks and then across the wave).
__global__ __launch_bounds__(256) void rmsnorm_rstd_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           int64_t ldx, float eps, float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const uint16_t* row = x + r * ldx;
  float acc = 0.0f;
  for (int64_t c0 = (int64_t)lane * 8; c0 < C; c0 += 512) {
    const uint4 v = load8(row, c0, C);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = elem(v, j);
      acc = fmaf(e, e, acc);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) rstd[r] = 1.0f / sqrtf(acc / (float)C + eps);
}

}  // namespace

void launch_quant_rows(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  dim3 grid((unsigned)((R + 31) / 32), (unsigned)((C + 127) / 128));
  hipLaunchKernelGGL(quant_rows_kernel, grid, dim3(256), 0, st, x, R, C, ldx, q, ldq, s, lds);
}

void launch_quant_tokens(const uint16_t* x, int64_t M, int64_t C, int64_t ldx,
                         uint8_t* qT, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  const uint32_t nfb = (uint32_t)((C + 255) / 256);
  const dim3 grid((unsigned)(nfb * ((M + 127) / 128)));
  hipLaunchKernelGGL(quant_tokens_kernel, grid, dim3(256), 0, st, x, M, C, ldx, qT, ldq, s, lds, nfb);
}

void launch_quant_blocks(const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                         uint8_t* q, int64_t ldq, float* s,
                         uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st) {
  const uint32_t nbc = (uint32_t)((C + 127) / 128);
  const dim3 grid((unsigned)(nbc * ((R + 127) / 128)));
  hipLaunchKernelGGL(quant_blocks_kernel, grid, dim3(256), 0, st, w, R, C, ldw, q, ldq, s, qT, ldqT, sT, nbc);
}

void launch_quant_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds,
                       uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, hipStream_t st) {
  const uint32_t nbc = (uint32_t)((C + 127) / 128);
  const dim3 grid((unsigned)(nbc * ((R + 127) / 128)));
  hipLaunchKernelGGL(quant_dual_kernel<SrcPlain>, grid, dim3(256), 0, st, SrcPlain{x, ldx}, R, C, q, ldq, s, lds,
                     qT, ldqT, sT, ldsT, (uint16_t*)nullptr, (int64_t)0, nbc);
}

void launch_swiglu_quant_dual(const uint16_t* g, int64_t ldg, const uint16_t* u, int64_t ldu, int64_t R, int64_t C,
                              uint8_t* q, int64_t ldq, float* s, int64_t lds,
                              uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                              uint16_t* h, int64_t ldh, hipStream_t st) {
  const uint32_t nbc = (uint32_t)((C + 127) / 128);
  const dim3 grid((unsigned)(nbc * ((R + 127) / 128)));
  hipLaunchKernelGGL(quant_dual_kernel<SrcSwiGLU>, grid, dim3(256), 0, st, SrcSwiGLU{g, ldg, u, ldu}, R, C,
                     q, ldq, s, lds, qT, ldqT, sT, ldsT, h, ldh, nbc);
}

void launch_rmsnorm_quant_dual(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t R, int64_t C,
                               float* rstd, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                               uint16_t* y, int64_t ldy, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_rstd_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, x, R, C, ldx, eps, rstd);
  const uint32_t nbc = (uint32_t)((C + 127) / 128);
  const dim3 grid((unsigned)(nbc * ((R + 127) / 128)));
  hipLaunchKernelGGL(quant_dual_kernel<SrcRMSNorm>, grid, dim3(256), 0, st, SrcRMSNorm{x, ldx, rstd, gamma}, R, C,
                     q, ldq, s, lds, qT, ldqT, sT, ldsT, y, ldy, nbc);
}

void launch_encode(const float* x, uint8_t* q, int64_t n, hipStream_t st) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, q, n);
}

}  // namespace fp8blk
