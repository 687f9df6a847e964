// Block-scaled E4M3 GEMM for gfx950 (CDNA4 FP8 MFMA).
//
// Pages: paperlayer.ai summary of arXiv 2608.27370v1, appendix C
// "生産学習の詳細", item "FP8実装pipeline" -- the forward, data-gradient and
// weight-gradient GEMMs of each linear layer run on blockwise E4M3 operands;
// arxiv-wiki summary, section "접근 방법" item (4) -- one scale per 1x128
// activation group and per 128x128 weight block.
//
// One kernel family computes
//     C[i, j] = sum_lb SA(i, lb) * SB(j, lb) * P_lb[i, j],
//     P_lb[i, j] = sum_{l in block lb} A[i, l] * B[j, l]      (E4M3 codes)
// with both operands contraction-contiguous ("NT"), which is the natural
// layout of all three GEMMs:
//     forward  C = Y  [M, N]: A = Xq   [M, K],  B = Wq  [N, K]   (SB per 128x128 block)
//     dgrad    C = dX [M, K]: A = dYq  [M, N],  B = WqT [K, N]   (SB per 128x128 block)
//     wgrad    C = dW [N, K]: A = dYqT [N, M],  B = XqT [K, M]   (SB per row)
//
// gfx950 design:
//   * one 128-wide scale block is multiplied per step: either by four
//     v_mfma_f32_16x16x32_f16 on operands converted exactly from E4M3 to F16
//     in registers (PREC_F16, whose block partial is the exact sum up to FP32
//     rounding), or by one v_mfma_f32_16x16x128_f8f6f4 (PREC_FP8, faster, but
//     the matrix core truncates small products inside groups of 8 -- see Prec);
//   * each block partial of a 16x16 sub-tile starts from zero and is folded
//     into an FP32 register accumulator with one FMA per element and block:
//     acc = fma(P_lb, SA*SB, acc);
//   * operand tiles stay E4M3 in HBM and LDS (1 byte per element), staged in
//     128-byte rows (one K block) with an XOR swizzle of the 16-byte chunks so
//     that fragment reads are bank-conflict free; global loads for block lb+1
//     are in flight while block lb is multiplied (double-buffered LDS, one
//     barrier per block);
//   * workgroups are renumbered so that each of the 8 XCDs (own L2) works on
//     a contiguous range of output tiles, grouped 8 tile-rows at a time.
#include "internal.h"
#include "fp8_codec.h"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Four E4M3 codes (one dword) -> four F16 values, exact (every E4M3 value is an
// F16 normal or zero).
__device__ __forceinline__ void cvt4(uint32_t w, v8h& out, int half) {
  const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  out[4 * half + 0] = lo[0];
  out[4 * half + 1] = lo[1];
  out[4 * half + 2] = hi[0];
  out[4 * half + 3] = hi[1];
}

// 32 codes of a fragment (lane's K range of one 128-wide block) -> 4 F16
// operands of 8 values, chunk c holding codes 8c..8c+7.
__device__ __forceinline__ void cvt_frag(const uint4& lo, const uint4& hi, v8h (&f)[4]) {
  cvt4(lo.x, f[0], 0); cvt4(lo.y, f[0], 1);
  cvt4(lo.z, f[1], 0); cvt4(lo.w, f[1], 1);
  cvt4(hi.x, f[2], 0); cvt4(hi.y, f[2], 1);
  cvt4(hi.z, f[3], 0); cvt4(hi.w, f[3], 1);
}

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

__device__ __forceinline__ void map_tile(int pid, int nblocks, int tilesM, int tilesN, int& tm, int& tn) {
  // Workgroup pid runs on XCD pid % 8; give each XCD a contiguous logical range.
  const int q = nblocks / 8, r = nblocks % 8;
  const int xcd = pid % 8, local = pid / 8;
  const int logical = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  // Grouped order: kGroupM tile-rows at a time, walking down columns.
  const int per_group = kGroupM * tilesN;
  const int gid = logical / per_group;
  const int first_m = gid * kGroupM;
  const int gm = min(tilesM - first_m, kGroupM);
  const int in_group = logical - gid * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// PREC selects how the exact 128-term block product is formed:
//   PREC_F16: the E4M3 codes are converted exactly to F16 in registers and
//     multiplied with v_mfma_f32_16x16x32_f16 (4 per block); the matrix core
//     adds the products of one instruction without intermediate truncation, so
//     each block partial carries only FP32 rounding (a few 2^-24 relative);
//   PREC_FP8: one v_mfma_f32_16x16x128_f8f6f4 per block.  On gfx950 this
//     instruction sums products in groups of 8 after aligning them to the
//     largest product of the group and truncating below 2^-13 of it, so a block
//     partial can be off by up to about 7 * 2^-13 of the group's largest
//     product when values inside a group differ widely in magnitude.
enum Prec { PREC_F16 = 0, PREC_FP8 = 1 };

template <int SB_MODE, int OUT, int PREC>
__global__ __launch_bounds__(kThreads, 2) void block_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ SB, int64_t ldsb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * BK];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = wave >> 1, wn = wave & 1;          // 2 x 2 waves, 64 x 64 each
  const int nLB = (int)(L / BK);

  // Global -> LDS staging: thread t moves rows (t/8) + 32k, 16-byte chunk t%8.
  const int lrow = t >> 3, lchunk = t & 7;
  uint4 ra[4], rb[4];
  auto gload = [&](int lb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = i0 + lrow + 32 * k;
      ra[k] = (r < I) ? *reinterpret_cast<const uint4*>(A + r * lda + (int64_t)lb * BK + lchunk * 16)
                      : make_uint4(0, 0, 0, 0);
      rb[k] = *reinterpret_cast<const uint4*>(B + (j0 + lrow + 32 * k) * ldb + (int64_t)lb * BK + lchunk * 16);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int off = swz(lrow + 32 * k, lchunk);
      *reinterpret_cast<uint4*>(&lds_a[buf][off]) = ra[k];
      *reinterpret_cast<uint4*>(&lds_b[buf][off]) = rb[k];
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  // Rows of this lane's outputs in sub-tile mi: rbase + mi*16 + r, r = 0..3.
  const int64_t rbase = i0 + wm * 64 + (lane >> 4) * 4;
  const int64_t cbase = j0 + wn * 64 + (lane & 15);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int lb = 0; lb < nLB; ++lb) {
    const int buf = lb & 1;
    if (lb + 1 < nLB) gload(lb + 1);

    // Scales of this block.
    float sa[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int64_t row = rbase + mi * 16;
      const float* p = SA + (int64_t)lb * ldsa + row;
      if (row + 4 <= I) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        sa[mi][0] = v.x; sa[mi][1] = v.y; sa[mi][2] = v.z; sa[mi][3] = v.w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[mi][r] = (row + r < I) ? p[r] : 0.0f;
      }
    }
    float sb[4];
    if (SB_MODE == SB_BLOCK) {
      const float s = SB[(j0 / 128) * nLB + lb];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[mi][r] *= s;
    } else {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) sb[ni] = SB[(int64_t)lb * ldsb + cbase + ni * 16];
    }

    // Fragments: lane holds row (lane%16) of a 16-row sub-tile, 32 K-bytes
    // starting at 32*(lane/16); A and B use the same K arrangement, so the
    // order in which the MFMA pairs K elements does not matter.
    const int ch = (lane >> 4) * 2;
    if (PREC == PREC_FP8) {
      v8i fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 64 + mi * 16 + (lane & 15);
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds_a[buf][swz(row, ch)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds_a[buf][swz(row, ch + 1)]);
        fa[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 64 + ni * 16 + (lane & 15);
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds_b[buf][swz(row, ch)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds_b[buf][swz(row, ch + 1)]);
        fb[ni] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          // E4M3 x E4M3 (format selectors 0, 0), no block scaling in the MFMA.
          const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[mi], fb[ni], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = (SB_MODE == SB_BLOCK) ? sa[mi][r] : sa[mi][r] * sb[ni];
            acc[mi][ni][r] = fmaf(p[r], s, acc[mi][ni][r]);
          }
        }
      }
    } else {
      v8h fb[4][4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 64 + ni * 16 + (lane & 15);
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds_b[buf][swz(row, ch)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds_b[buf][swz(row, ch + 1)]);
        cvt_frag(lo, hi, fb[ni]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 64 + mi * 16 + (lane & 15);
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds_a[buf][swz(row, ch)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds_a[buf][swz(row, ch + 1)]);
        v8h fa[4];
        cvt_frag(lo, hi, fa);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          v4f p = zero;
#pragma unroll
          for (int c = 0; c < 4; ++c) p = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[c], fb[ni][c], p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = (SB_MODE == SB_BLOCK) ? sa[mi][r] : sa[mi][r] * sb[ni];
            acc[mi][ni][r] = fmaf(p[r], s, acc[mi][ni][r]);
          }
        }
      }
    }

    if (lb + 1 < nLB) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane owns rows rbase + mi*16 + r, column cbase + ni*16.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = rbase + mi * 16 + r;
      if (row >= I) continue;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t col = cbase + ni * 16;
        const float v = acc[mi][ni][r];
        if (OUT == OUT_F32) {
          static_cast<float*>(Cout)[row * ldc + col] = v;
        } else if (OUT == OUT_F32_ACC) {
          float* p = static_cast<float*>(Cout) + row * ldc + col;
          *p = *p + v;
        } else {
          static_cast<uint16_t*>(Cout)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(256) void fill_zero_kernel(void* __restrict__ C, int64_t rows, int64_t cols, int64_t ldc) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i - r * cols;
    if (OUT == OUT_BF16) static_cast<uint16_t*>(C)[r * ldc + c] = 0;
    else static_cast<float*>(C)[r * ldc + c] = 0.0f;
  }
}

template <int SB_MODE, int OUT>
void launch_t(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
              const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
              int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int prec, hipStream_t st) {
  const int tilesM = (int)((I + BM - 1) / BM), tilesN = (int)(J / BN);
  if (prec == PREC_FP8)
    hipLaunchKernelGGL((block_gemm_kernel<SB_MODE, OUT, PREC_FP8>), dim3(tilesM * tilesN), dim3(kThreads), 0, st,
                       A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN);
  else
    hipLaunchKernelGGL((block_gemm_kernel<SB_MODE, OUT, PREC_F16>), dim3(tilesM * tilesN), dim3(kThreads), 0, st,
                       A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN);
}

}  // namespace

void launch_block_gemm(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                       const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb, int sb_mode,
                       int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int out_mode,
                       int prec, hipStream_t st) {
  if (L == 0) {   // empty contraction: the product is zero
    if (out_mode == OUT_F32_ACC) return;
    const int64_t n = I * J;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (out_mode == OUT_BF16)
      hipLaunchKernelGGL(fill_zero_kernel<OUT_BF16>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    else
      hipLaunchKernelGGL(fill_zero_kernel<OUT_F32>, dim3(blocks), dim3(256), 0, st, C, I, J, ldc);
    return;
  }
#define FP8BLK_GEMM_CASE(SBM, OM)                                                    \
  if (sb_mode == SBM && out_mode == OM) {                                            \
    launch_t<SBM, OM>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, prec, st);      \
    return;                                                                          \
  }
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_F32)
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_BF16)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32_ACC)
#undef FP8BLK_GEMM_CASE
}

}  // namespace fp8blk
