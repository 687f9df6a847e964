// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// Launchers: arguments were validated by the ABI layer; these only enqueue.
void launch_quant_rows(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st);
void launch_quant_tokens(const uint16_t* x, int64_t M, int64_t C, int64_t ldx,
                         uint8_t* qT, int64_t ldq, float* s, int64_t lds, hipStream_t st);
void launch_quant_blocks(const uint16_t* w, int64_t R, int64_t C, int64_t ldw,
                         uint8_t* q, int64_t ldq, float* s,
                         uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st);
void launch_quant_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds,
                       uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, hipStream_t st);
void launch_swiglu_quant_dual(const uint16_t* g, int64_t ldg, const uint16_t* u, int64_t ldu, int64_t R, int64_t C,
                              uint8_t* q, int64_t ldq, float* s, int64_t lds,
                              uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                              uint16_t* h, int64_t ldh, hipStream_t st);
void launch_rmsnorm_quant_dual(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t R, int64_t C,
                               float* rstd, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                               uint16_t* y, int64_t ldy, hipStream_t st);
void launch_encode(const float* x, uint8_t* q, int64_t n, hipStream_t st);

// Scale modes of the second GEMM operand.
enum SbMode { SB_BLOCK = 0, SB_ROWS = 1 };
// Output modes.
enum OutMode { OUT_F32 = 0, OUT_BF16 = 1, OUT_F32_ACC = 2 };

// How a block GEMM is laid out over the CUs: 256 x 128 tiles or 128 x 128
// tiles; with a workspace, 256 x 128 tiles split in two along the contraction
// (on request) or 128 x 128 tiles split 2, 4 or 8 ways (small grids), with
// counters and partial tiles in the workspace.
struct SplitPlan {
  bool big_tiles = false;        // unsplit: 256 x 128 tiles (else 128 x 128)
  int splits = 1;
  bool split_big_tiles = false;  // split: 256 x 128 tiles (else 128 x 128)
  bool kgroups = false;          // unsplit 128 x 128 exact path: 8 waves in two K groups (at most one tile per CU)
  unsigned* counters = nullptr;
  float* part = nullptr;
};
// Workspace bytes for `splits` splits of an I x J output on 256 x 128 tiles
// (0 for one split).
size_t split_workspace_bytes(int64_t I, int64_t J, int splits);
// The default split of I x J x L (1, 2, 4 or 8; see gemm.hip) and its
// workspace bytes on 128 x 128 tiles.
int small_grid_splits(int64_t I, int64_t J, int64_t L);
size_t small_split_workspace_bytes(int64_t I, int64_t J, int splits);
// The plan for a call: with `force`, split in two on 256 x 128 tiles when the
// workspace holds split_workspace_bytes(I, J, 2); otherwise the default split
// when the workspace holds its bytes; else one split (with `kgroups` for
// grids of at most one 128 x 128 tile per CU and an even number of blocks).
SplitPlan plan_split(int64_t I, int64_t J, int64_t L, void* ws, size_t ws_bytes, bool force);

// C[I, J] = sum_lb SA(i, lb) SB(j, lb) sum_{l in lb} A[i, l] B[j, l]
//   A [I, lda] codes, SA[lb * ldsa + i];
//   B [J, ldb] codes; SB_BLOCK: SB[(j / 128) * nLB + lb]; SB_ROWS: SB[lb * ldsb + j].
// J and L are multiples of 128; I is arbitrary.
void launch_block_gemm(const uint8_t* A, int64_t lda, const float* SA, int64_t ldsa,
                       const uint8_t* B, int64_t ldb, const float* SB, int64_t ldsb, int sb_mode,
                       int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int out_mode,
                       int prec, const SplitPlan& plan, hipStream_t st);

// Zero n 32-bit words at p (a fill kernel: usable inside a captured graph).
void launch_clear_u32(unsigned* p, int64_t n, hipStream_t st);

// C[I, J] = sum_l A[i, l] B[j, l] over BF16 operands (A [I, lda], B [J, ldb]);
// J a multiple of 128, L a multiple of 64; out_mode OUT_F32 or OUT_BF16.
void launch_bf16_gemm(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      int64_t I, int64_t J, int64_t L, void* C, int64_t ldc, int out_mode, hipStream_t st);

}  // namespace fp8blk
