// Block-scaled E4M3 GEMM for gfx950 (CDNA4 matrix cores).
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
//   * operands stay E4M3 in HBM and LDS (one byte per element); each
//     workgroup stages a BM x 128 tile of A and a BN x 128 tile of B per
//     scale block with global_load_lds_dwordx4 (no VGPR round trip), double
//     buffered so block lb+1 streams in while block lb is multiplied; rows
//     are 128 bytes with the 16-byte chunks XOR-swizzled by (row % 8) so the
//     ds_read_b128 fragment reads are bank-conflict free;
//   * the block product of a 16x16 sub-tile is formed in the matrix core from
//     a zero accumulator -- either four v_mfma_f32_16x16x32_f16 on operands
//     converted exactly from E4M3 to F16 in registers (PREC_F16: the block
//     partial is the exact sum up to FP32 rounding), or one
//     v_mfma_f32_16x16x128_f8f6f4 (PREC_FP8: twice the matrix rate, but the
//     hardware truncates small products inside groups of 8, see Prec) -- and
//     folded into FP32 accumulators with one FMA per element and block;
//   * the scales of block lb+1 (rows of A, and rows of B for the weight
//     gradient) are staged into LDS alongside the operand tiles;
//   * workgroups are renumbered so that each of the 8 XCDs (own L2) works on a
//     contiguous range of output tiles, grouped 8 tile-rows at a time.
#include "internal.h"
#include "fp8_codec.h"

namespace fp8blk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

// PREC selects how the 128-term block product is formed:
//   PREC_F16: the E4M3 codes are converted exactly to F16 in registers
//     (v_cvt_scalef32_pk_f16_fp8 with scale 1; every E4M3 value is an F16
//     normal or zero) and multiplied with v_mfma_f32_16x16x32_f16, four per
//     block.  The matrix core adds the products of one instruction without
//     intermediate truncation, so the block partial carries only FP32
//     rounding (a few 2^-24 relative).
//   PREC_FP8: one v_mfma_f32_16x16x128_f8f6f4 per block.  On gfx950 this
//     instruction sums products in groups of 8 after aligning them to the
//     largest product of the group and truncating 13 bits below it, so a block
//     partial can be off by up to about 7 * 2^-13 of the group's largest
//     product when values inside a group differ widely in magnitude.
enum Prec { PREC_F16 = 0, PREC_FP8 = 1 };

// Four E4M3 codes (one dword) -> four F16 values of an operand, exact.
__device__ __forceinline__ void cvt4(uint32_t w, v8h& out, int half) {
  const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  out[4 * half + 0] = lo[0];
  out[4 * half + 1] = lo[1];
  out[4 * half + 2] = hi[0];
  out[4 * half + 3] = hi[1];
}

// A lane's 32 codes of one block -> four F16 MFMA operands (chunk c = codes 8c..8c+7).
__device__ __forceinline__ void cvt_frag(const uint4& lo, const uint4& hi, v8h (&f)[4]) {
  cvt4(lo.x, f[0], 0); cvt4(lo.y, f[0], 1);
  cvt4(lo.z, f[1], 0); cvt4(lo.w, f[1], 1);
  cvt4(hi.x, f[2], 0); cvt4(hi.y, f[2], 1);
  cvt4(hi.z, f[3], 0); cvt4(hi.w, f[3], 1);
}

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

// Byte offset of 16-byte chunk `chunk` of tile row `row` in LDS.
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// Stage rows [0, ROWS) of a tile (row r = global row r0 + r, clamped to rmax)
// for scale block lb into LDS at `dst`.  One wave instruction moves 8 rows
// (1 KB); lane L writes LDS bytes [16L, 16L+16) of its instruction's 1 KB,
// i.e. row 8u + L/8, slot L%8, which must hold global chunk (L%8) ^ (L/8).
// Clamped rows (beyond the last valid row) only feed output rows that are
// never stored.
template <int ROWS>
__device__ __forceinline__ void stage(const uint8_t* __restrict__ G, int64_t ld, int64_t r0, int64_t rmax,
                                      int lb, uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int u = wave; u < ROWS / 8; u += 4) {
    int64_t row = r0 + 8 * u + (lane >> 3);
    row = row < rmax ? row : rmax;
    const int chunk = (lane & 7) ^ (lane >> 3);
    const uint8_t* src = G + row * ld + (int64_t)lb * BK + chunk * 16;
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(dst + u * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void frag_codes(const uint8_t* tile, int row, int ch, uint4& lo, uint4& hi) {
  lo = *reinterpret_cast<const uint4*>(tile + swz(row, ch));
  hi = *reinterpret_cast<const uint4*>(tile + swz(row, ch + 1));
}

// Stage N scale values SC[lb * ld + r0 + r], r < N (indices clamped to rmax),
// into LDS at dst with 4-byte direct loads: one wave instruction moves 64.
template <int N>
__device__ __forceinline__ void stage_scales(const float* __restrict__ SC, int64_t ld, int64_t r0, int64_t rmax,
                                             int lb, float* dst, int wave, int lane, int first_wave) {
#pragma unroll
  for (int u = 0; u < N / 64; ++u) {
    if (wave == (first_wave + u) % 4) {
      int64_t r = r0 + 64 * u + lane;
      r = r < rmax ? r : rmax;
      const float* src = SC + (int64_t)lb * ld + r;
      __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(dst + 64 * u), 4, 0, 0);
    }
  }
}

template <int BM, int BN, int WM, int WN, int SB_MODE, int OUT, int PREC>
__global__ __launch_bounds__(kThreads, (BM + BN) * BK * 2 <= 80 * 1024 ? 2 : 1) void block_gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ SA, int64_t ldsa,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ SB, int64_t ldsb,
    int64_t I, int64_t L, void* __restrict__ Cout, int64_t ldc, int tilesM, int tilesN) {
  constexpr int WGM = BM / WM, WGN = BN / WN;
  static_assert(WGM * WGN == 4, "four waves per workgroup");
  constexpr int MI = WM / 16, NI = WN / 16;
  // Per buffer: A tile, B tile, BM row scales of A, BN row scales of B (SB_ROWS).
  constexpr int kSaOff = (BM + BN) * BK;
  constexpr int kSbOff = kSaOff + BM * 4;
  constexpr int kBufBytes = kSbOff + (SB_MODE == SB_ROWS ? BN * 4 : 0);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kBufBytes];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  const int wm = wave / WGN, wn = wave % WGN;
  const int nLB = (int)(L / BK);
  const int64_t last_row = I - 1;

  v4f acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  // This lane's outputs in sub-tile (mi, ni): rows rbase + 16 mi + r (r < 4), column cbase + 16 ni.
  const int64_t rbase = i0 + wm * WM + (lane >> 4) * 4;
  const int64_t cbase = j0 + wn * WN + (lane & 15);

  auto stage_all = [&](int lb, uint8_t* buf) {
    stage<BM>(A, lda, i0, last_row, lb, buf, wave, lane);
    stage<BN>(B, ldb, j0, j0 + BN - 1, lb, buf + BM * BK, wave, lane);
    stage_scales<BM>(SA, ldsa, i0, last_row, lb, reinterpret_cast<float*>(buf + kSaOff), wave, lane, 0);
    if (SB_MODE == SB_ROWS)
      stage_scales<BN>(SB, ldsb, j0, j0 + BN - 1, lb, reinterpret_cast<float*>(buf + kSbOff), wave, lane,
                       BM / 64);
  };

  stage_all(0, lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int ch = (lane >> 4) * 2;
  for (int lb = 0; lb < nLB; ++lb) {
    uint8_t* cur = lds + (lb & 1) * kBufBytes;
    const uint8_t* ta = cur;
    const uint8_t* tb = cur + BM * BK;
    if (lb + 1 < nLB) stage_all(lb + 1, lds + ((lb + 1) & 1) * kBufBytes);

    // Scales of this block: rows of A from LDS; B's block scale (fwd/dgrad)
    // is uniform over the tile and folded into the row scales.
    float sa[MI][4], sb[NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const float4 v = *reinterpret_cast<const float4*>(cur + kSaOff + (wm * WM + mi * 16 + (lane >> 4) * 4) * 4);
      sa[mi][0] = v.x; sa[mi][1] = v.y; sa[mi][2] = v.z; sa[mi][3] = v.w;
    }
    if (SB_MODE == SB_BLOCK) {
      const float s = SB[(j0 / 128) * nLB + lb];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[mi][r] *= s;
    } else {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        sb[ni] = reinterpret_cast<const float*>(cur + kSbOff)[wn * WN + ni * 16 + (lane & 15)];
    }

    if (PREC == PREC_FP8) {
      v8i fa[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        uint4 lo, hi;
        frag_codes(ta, wm * WM + mi * 16 + (lane & 15), ch, lo, hi);
        fa[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        uint4 lo, hi;
        frag_codes(tb, wn * WN + ni * 16 + (lane & 15), ch, lo, hi);
        const v8i fb = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[mi], fb, v4f{0.f, 0.f, 0.f, 0.f},
                                                                         0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = (SB_MODE == SB_BLOCK) ? sa[mi][r] : sa[mi][r] * sb[ni];
            acc[mi][ni][r] = fmaf(p[r], s, acc[mi][ni][r]);
          }
        }
        // Keep at most one column of partials live (register budget).
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      v8h fa[MI][4];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        uint4 lo, hi;
        frag_codes(ta, wm * WM + mi * 16 + (lane & 15), ch, lo, hi);
        cvt_frag(lo, hi, fa[mi]);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        uint4 lo, hi;
        frag_codes(tb, wn * WN + ni * 16 + (lane & 15), ch, lo, hi);
        v8h fb[4];
        cvt_frag(lo, hi, fb);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          v4f p = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) p = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[mi][c], fb[c], p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = (SB_MODE == SB_BLOCK) ? sa[mi][r] : sa[mi][r] * sb[ni];
            acc[mi][ni][r] = fmaf(p[r], s, acc[mi][ni][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    __builtin_amdgcn_s_waitcnt(0);   // this wave's staging of block lb+1 has landed
    __syncthreads();                  // ... and everyone's; block lb is no longer read
  }

  // Epilogue: lane owns rows rbase + 16 mi + r, columns cbase + 16 ni.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = rbase + mi * 16 + r;
      if (row >= I) continue;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
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

template <int BM, int BN, int WM, int WN, int SB_MODE, int OUT, int PREC>
void launch_cfg(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, hipStream_t st) {
  const int tilesM = (int)((I + BM - 1) / BM), tilesN = (int)(J / BN);
  hipLaunchKernelGGL((block_gemm_kernel<BM, BN, WM, WN, SB_MODE, OUT, PREC>), dim3(tilesM * tilesN),
                     dim3(kThreads), 0, st, A, lda, SA, ldsa, B, ldb, SB, ldsb, I, L, C, ldc, tilesM, tilesN);
}

template <int SB_MODE, int OUT, int PREC>
void launch_prec(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                 const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb,
                 int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, hipStream_t st) {
  launch_cfg<128, 128, 64, 64, SB_MODE, OUT, PREC>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, st);
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
#define FP8BLK_GEMM_CASE(SBM, OM)                                                              \
  if (sb_mode == SBM && out_mode == OM) {                                                      \
    if (prec == PREC_FP8)                                                                      \
      launch_prec<SBM, OM, PREC_FP8>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, st); \
    else                                                                                       \
      launch_prec<SBM, OM, PREC_F16>(A, lda, SA, ldsa, B, ldb, SB, ldsb, I, J, L, C, ldc, st); \
    return;                                                                                    \
  }
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_F32)
  FP8BLK_GEMM_CASE(SB_BLOCK, OUT_BF16)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32)
  FP8BLK_GEMM_CASE(SB_ROWS, OUT_F32_ACC)
#undef FP8BLK_GEMM_CASE
}

}  // namespace fp8blk
