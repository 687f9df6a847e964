// C ABI of libfp8blk: argument validation, device check, launches.
// The semantics of each call are documented in include/fp8blk.h.
#include <string.h>

#include <mutex>

#include "fp8blk.h"
#include "internal.h"

namespace {

using namespace fp8blk;

// Per-device cache of "is gfx950" (0 = unknown, 1 = yes, 2 = no).  Benign race:
// every writer stores the same value.
constexpr int kMaxDevices = 64;
// Row strides (bytes) of GEMM operands: a 256-row tile spans less than 2^31.
constexpr int64_t kMaxGemmLd = (int64_t)1 << 23;
// Workgroups of a one-dimensional grid.
constexpr int64_t kMaxGrid = ((int64_t)1 << 31) - 1;
int g_arch_ok[kMaxDevices];

bool device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < kMaxDevices && g_arch_ok[dev] != 0) return g_arch_ok[dev] == 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev] = ok ? 1 : 2;
  return ok;
}

// Largest dimension accepted (far beyond any tensor that fits in memory);
// checked before any arithmetic on the dimensions.
constexpr int64_t kMaxDim = (int64_t)1 << 40;

// Whether a one-dimensional grid of ceil(rows / rb) x ceil(cols / cb)
// workgroups fits (rows, cols >= 0).  Each factor is bounded first, so the
// product cannot overflow.
inline bool grid_fits(int64_t rows, int64_t rb, int64_t cols, int64_t cb) {
  if (rows >= kMaxGrid * rb || cols >= kMaxGrid * cb) return false;
  return ((rows + rb - 1) / rb) * ((cols + cb - 1) / cb) < kMaxGrid;
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int finish() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BLK_OK : FP8BLK_LAUNCH_FAILED;
}

// Common checks for a GEMM operand pair; see fp8blk.h for the contract.
int check_gemm(int64_t I, int64_t J, int64_t L, const void* A, int64_t lda, const float* SA, int64_t ldsa,
               const void* B, int64_t ldb, const float* SB, int64_t ldsb, bool sb_rows,
               const void* C, int64_t ldc, int out_mode, int64_t L_valid_rows_sa) {
  if (I < 0 || J < 0 || L < 0) return FP8BLK_INVALID_ARG;
  if (J % 128 != 0 || L % 128 != 0) return FP8BLK_UNSUPPORTED_SHAPE;
  if (I == 0 || J == 0) return -1;  // valid no-op
  if (C == nullptr) return FP8BLK_INVALID_ARG;
  if (ldc < J) return FP8BLK_INVALID_ARG;
  if (out_mode == OUT_BF16 ? (!al16(C) || ldc % 8 != 0) : (!al16(C) || ldc % 4 != 0)) return FP8BLK_MISALIGNED;
  if (L == 0) return 0;
  if (A == nullptr || B == nullptr || SA == nullptr || SB == nullptr) return FP8BLK_INVALID_ARG;
  if (lda < L || ldb < L || ldsa < L_valid_rows_sa) return FP8BLK_INVALID_ARG;
  // The kernels address the rows of a tile with 32-bit byte offsets from the
  // tile's first row, and number the tiles in one grid dimension.
  if (lda >= kMaxGemmLd || ldb >= kMaxGemmLd) return FP8BLK_UNSUPPORTED_SHAPE;
  if (!grid_fits(I, 128, J, 128)) return FP8BLK_UNSUPPORTED_SHAPE;
  if (sb_rows && ldsb < J) return FP8BLK_INVALID_ARG;
  if (!al16(A) || !al16(B) || lda % 16 != 0 || ldb % 16 != 0) return FP8BLK_MISALIGNED;
  if (!al16(SA) || ldsa % 4 != 0) return FP8BLK_MISALIGNED;
  if (!al4(SB) || (sb_rows && (!al16(SB) || ldsb % 4 != 0))) return FP8BLK_MISALIGNED;
  return 0;
}

}  // namespace

extern "C" {

int fp8_quant_1x128(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                    int transpose_out, uint8_t* q, int64_t ld_q,
                    float* scales, int64_t ld_s, void* stream) {
  if (rows < 0 || cols < 0 || (transpose_out != 0 && transpose_out != 1)) return FP8BLK_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8BLK_OK;
  if (rows >= kMaxDim || cols >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  if (x_bf16 == nullptr || q == nullptr || scales == nullptr) return FP8BLK_INVALID_ARG;
  if (ld_x < cols) return FP8BLK_INVALID_ARG;
  if (transpose_out == 0) {
    if (ld_q < cols || ld_s < rows) return FP8BLK_INVALID_ARG;
  } else {
    const int64_t mpad = (rows + 127) / 128 * 128;
    if (ld_q < mpad || ld_s < cols) return FP8BLK_INVALID_ARG;
  }
  // Grids: row blocks x column groups (at most 65535) for the row-wise
  // kernel, one dimension of (token group, 256-feature block) otherwise.
  if (transpose_out == 0 ? (cols > (int64_t)65535 * 128 || !grid_fits(rows, 32, 1, 1))
                         : !grid_fits(rows, 128, cols, 256))
    return FP8BLK_UNSUPPORTED_SHAPE;
  if (!al16(x_bf16) || ld_x % 8 != 0 || !al16(q) || ld_q % 16 != 0 || !al4(scales)) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (transpose_out == 0)
    launch_quant_rows(static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, q, ld_q, scales, ld_s, st);
  else
    launch_quant_tokens(static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, q, ld_q, scales, ld_s, st);
  return finish();
}

int fp8_quant_1x128_dual(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                         uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                         uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT, void* stream) {
  if (rows < 0 || cols < 0) return FP8BLK_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8BLK_OK;
  if (rows >= kMaxDim || cols >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  if (x_bf16 == nullptr || q == nullptr || scales == nullptr || qT == nullptr || scalesT == nullptr)
    return FP8BLK_INVALID_ARG;
  const int64_t mpad = (rows + 127) / 128 * 128;
  if (ld_x < cols || ld_q < cols || ld_s < rows || ld_qT < mpad || ld_sT < cols) return FP8BLK_INVALID_ARG;
  if (!grid_fits(rows, 128, cols, 128)) return FP8BLK_UNSUPPORTED_SHAPE;
  if (!al16(x_bf16) || ld_x % 8 != 0 || !al16(q) || ld_q % 16 != 0 || !al16(qT) || ld_qT % 16 != 0 ||
      !al4(scales) || !al4(scalesT))
    return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_quant_dual(static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, q, ld_q, scales, ld_s,
                    qT, ld_qT, scalesT, ld_sT, static_cast<hipStream_t>(stream));
  return finish();
}

namespace {
// Output checks shared by the fused dual quantisers (as fp8_quant_1x128_dual).
int check_dual_outputs(int64_t rows, int64_t cols, const uint8_t* q, int64_t ld_q, const float* scales, int64_t ld_s,
                       const uint8_t* qT, int64_t ld_qT, const float* scalesT, int64_t ld_sT,
                       const void* bf16_out, int64_t ld_out) {
  if (q == nullptr || scales == nullptr || qT == nullptr || scalesT == nullptr) return FP8BLK_INVALID_ARG;
  const int64_t mpad = (rows + 127) / 128 * 128;
  if (ld_q < cols || ld_s < rows || ld_qT < mpad || ld_sT < cols) return FP8BLK_INVALID_ARG;
  if (bf16_out != nullptr && ld_out < cols) return FP8BLK_INVALID_ARG;
  if (!grid_fits(rows, 128, cols, 128)) return FP8BLK_UNSUPPORTED_SHAPE;
  if (!al16(q) || ld_q % 16 != 0 || !al16(qT) || ld_qT % 16 != 0 || !al4(scales) || !al4(scalesT)) return FP8BLK_MISALIGNED;
  if (bf16_out != nullptr && (!al16(bf16_out) || ld_out % 8 != 0)) return FP8BLK_MISALIGNED;
  return FP8BLK_OK;
}
}  // namespace

int fp8_swiglu_quant_1x128_dual(const void* gate, int64_t ld_gate, const void* up, int64_t ld_up,
                                int64_t rows, int64_t cols, uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT,
                                void* h_bf16, int64_t ld_h, void* stream) {
  if (rows < 0 || cols < 0) return FP8BLK_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8BLK_OK;
  if (rows >= kMaxDim || cols >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  if (gate == nullptr || up == nullptr || ld_gate < cols || ld_up < cols) return FP8BLK_INVALID_ARG;
  const int rc = check_dual_outputs(rows, cols, q, ld_q, scales, ld_s, qT, ld_qT, scalesT, ld_sT, h_bf16, ld_h);
  if (rc != FP8BLK_OK) return rc;
  if (!al16(gate) || !al16(up) || ld_gate % 8 != 0 || ld_up % 8 != 0) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_swiglu_quant_dual(static_cast<const uint16_t*>(gate), ld_gate, static_cast<const uint16_t*>(up), ld_up,
                           rows, cols, q, ld_q, scales, ld_s, qT, ld_qT, scalesT, ld_sT,
                           static_cast<uint16_t*>(h_bf16), ld_h, static_cast<hipStream_t>(stream));
  return finish();
}

int fp8_rmsnorm_quant_1x128_dual(const void* x, int64_t ld_x, const void* gamma, float eps,
                                 int64_t rows, int64_t cols, float* rstd,
                                 uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                 uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT,
                                 void* y_bf16, int64_t ld_y, void* stream) {
  if (rows < 0 || cols < 0 || !(eps >= 0.0f)) return FP8BLK_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8BLK_OK;
  if (rows >= kMaxDim || cols >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  if (x == nullptr || gamma == nullptr || rstd == nullptr || ld_x < cols) return FP8BLK_INVALID_ARG;
  const int rc = check_dual_outputs(rows, cols, q, ld_q, scales, ld_s, qT, ld_qT, scalesT, ld_sT, y_bf16, ld_y);
  if (rc != FP8BLK_OK) return rc;
  if (!al16(x) || ld_x % 8 != 0 || !al16(gamma) || !al4(rstd)) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_rmsnorm_quant_dual(static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(gamma), eps,
                            rows, cols, rstd, q, ld_q, scales, ld_s, qT, ld_qT, scalesT, ld_sT,
                            static_cast<uint16_t*>(y_bf16), ld_y, static_cast<hipStream_t>(stream));
  return finish();
}

int fp8_quant_128x128(const void* w_bf16, int64_t rows, int64_t cols, int64_t ld_w,
                      uint8_t* q, int64_t ld_q, float* scales,
                      uint8_t* qT, int64_t ld_qT, float* scalesT, void* stream) {
  if (rows < 0 || cols < 0) return FP8BLK_INVALID_ARG;
  if ((qT == nullptr) != (scalesT == nullptr)) return FP8BLK_INVALID_ARG;
  if (rows == 0 || cols == 0) return FP8BLK_OK;
  if (rows >= kMaxDim || cols >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  if (w_bf16 == nullptr || q == nullptr || scales == nullptr) return FP8BLK_INVALID_ARG;
  if (ld_w < cols || ld_q < cols || (qT != nullptr && ld_qT < rows)) return FP8BLK_INVALID_ARG;
  if (!grid_fits(rows, 128, cols, 128)) return FP8BLK_UNSUPPORTED_SHAPE;
  if (!al16(w_bf16) || ld_w % 8 != 0 || !al16(q) || ld_q % 16 != 0 || !al4(scales)) return FP8BLK_MISALIGNED;
  if (qT != nullptr && (!al16(qT) || ld_qT % 16 != 0 || !al4(scalesT))) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_quant_blocks(static_cast<const uint16_t*>(w_bf16), rows, cols, ld_w, q, ld_q, scales, qT, ld_qT,
                      scalesT, static_cast<hipStream_t>(stream));
  return finish();
}

}  // extern "C"

namespace {

// Shared body of the GEMM entry points.  Operand naming follows the generic
// entry point: a/sa is the row-scaled operand, b/sb the second one.
// The GEMM's output rows, columns and contraction length (I, J, L) for op.
void gemm_dims(int op, int64_t M, int64_t N, int64_t K, int64_t& I, int64_t& J, int64_t& L) {
  if (op == FP8BLK_OP_WGRAD) {
    I = N; J = K; L = (M + 127) / 128 * 128;
  } else {
    I = M;
    J = op == FP8BLK_OP_FWD ? N : K;
    L = op == FP8BLK_OP_FWD ? K : N;
  }
}

// Validated description of a GEMM call (see gemm_validate).
struct GemmCall {
  int64_t I = 0, J = 0, L = 0;
  int sb_mode = SB_BLOCK, out = OUT_F32, prec = 0;
  bool force_split = false;
};

// Every argument check of the GEMM entry points, before anything is launched.
// Returns FP8BLK_OK with g filled in, -1 for a valid no-op, or an error status.
int gemm_validate(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                  const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
                  int64_t M, int64_t N, int64_t K, const void* c, int64_t ld_c, int c_dtype, int accumulate,
                  GemmCall& g) {
  if (op != FP8BLK_OP_FWD && op != FP8BLK_OP_DGRAD && op != FP8BLK_OP_WGRAD) return FP8BLK_INVALID_ARG;
  const int path = flags & ~FP8BLK_GEMM_SPLIT2;
  if (path != FP8BLK_GEMM_EXACT_BLOCKS && path != FP8BLK_GEMM_FP8_MATRIX_CORE) return FP8BLK_INVALID_ARG;
  g.force_split = (flags & FP8BLK_GEMM_SPLIT2) != 0;
  if (c_dtype != FP8BLK_OUT_F32 && c_dtype != FP8BLK_OUT_BF16) return FP8BLK_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return FP8BLK_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return FP8BLK_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FP8BLK_UNSUPPORTED_SHAPE;
  g.prec = path == FP8BLK_GEMM_FP8_MATRIX_CORE ? 1 : 0;
  // wgrad: C = dW [N, K], contraction over M_pad tokens; fwd: C = Y [M, N]
  // over K; dgrad: C = dX [M, K] over N.
  gemm_dims(op, M, N, K, g.I, g.J, g.L);
  if (op == FP8BLK_OP_WGRAD) {
    if (c_dtype != FP8BLK_OUT_F32) return FP8BLK_INVALID_ARG;
    if (N % 128 != 0) return FP8BLK_UNSUPPORTED_SHAPE;
    g.sb_mode = SB_ROWS;
    g.out = accumulate ? OUT_F32_ACC : OUT_F32;
  } else {
    if (accumulate) return FP8BLK_INVALID_ARG;
    g.sb_mode = SB_BLOCK;
    g.out = c_dtype == FP8BLK_OUT_BF16 ? OUT_BF16 : OUT_F32;
  }
  return check_gemm(g.I, g.J, g.L, a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, g.sb_mode == SB_ROWS, c, ld_c, g.out, g.I);
}

int gemm_impl(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
              const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
              int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype, int accumulate,
              void* ws, size_t ws_bytes, hipStream_t st) {
  GemmCall g;
  const int rc = gemm_validate(op, flags, a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, M, N, K, c, ld_c, c_dtype,
                               accumulate, g);
  if (rc == -1) return FP8BLK_OK;
  if (rc != 0) return rc;
  if (ws != nullptr && !al16(ws)) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  const SplitPlan plan = plan_split(g.I, g.J, g.L, ws, ws_bytes, g.force_split);
  launch_block_gemm(a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, g.sb_mode, g.I, g.J, g.L, c, ld_c, g.out, g.prec, plan,
                    st);
  return finish();
}

// Scratch of the allocation-free split GEMM: a file-scope device array, one
// copy per GPU, holding the 64 KiB counter region and the partial tiles of up
// to 128 output tiles of 256 x 128 (e.g. a 2048 x 2048 weight gradient).  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current and kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)64 * 1024 + (size_t)128 * 2 * 256 * 128 * 4;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// This device's address of `scratch` (nullptr if the lookup fails).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int fp8_block_gemm_fwd(const uint8_t* xq, int64_t ld_xq, const float* sx, int64_t ld_sx,
                       const uint8_t* wq, int64_t ld_wq, const float* sw,
                       int64_t M, int64_t N, int64_t K,
                       void* y, int64_t ld_y, int y_dtype,
                       void* ws, size_t ws_bytes, void* stream) {
  return gemm_impl(FP8BLK_OP_FWD, FP8BLK_GEMM_EXACT_BLOCKS, xq, ld_xq, sx, ld_sx, wq, ld_wq, sw, 0, M, N, K,
                   y, ld_y, y_dtype, 0, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_dgrad(const uint8_t* dyq, int64_t ld_dyq, const float* sdy, int64_t ld_sdy,
                         const uint8_t* wqT, int64_t ld_wqT, const float* swT,
                         int64_t M, int64_t N, int64_t K,
                         void* dx, int64_t ld_dx, int dx_dtype,
                         void* ws, size_t ws_bytes, void* stream) {
  return gemm_impl(FP8BLK_OP_DGRAD, FP8BLK_GEMM_EXACT_BLOCKS, dyq, ld_dyq, sdy, ld_sdy, wqT, ld_wqT, swT, 0,
                   M, N, K, dx, ld_dx, dx_dtype, 0, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_wgrad(const uint8_t* dyqT, int64_t ld_dyqT, const float* sdyT, int64_t ld_sdyT,
                         const uint8_t* xqT, int64_t ld_xqT, const float* sxT, int64_t ld_sxT,
                         int64_t M, int64_t N, int64_t K,
                         float* dw, int64_t ld_dw, int accumulate,
                         void* ws, size_t ws_bytes, void* stream) {
  return gemm_impl(FP8BLK_OP_WGRAD, FP8BLK_GEMM_EXACT_BLOCKS, dyqT, ld_dyqT, sdyT, ld_sdyT, xqT, ld_xqT, sxT,
                   ld_sxT, M, N, K, dw, ld_dw, FP8BLK_OUT_F32, accumulate, ws, ws_bytes,
                   static_cast<hipStream_t>(stream));
}

int fp8_block_gemm(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                   const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
                   int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype, int accumulate,
                   void* ws, size_t ws_bytes, void* stream) {
  return gemm_impl(op, flags, a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, M, N, K, c, ld_c, c_dtype, accumulate,
                   ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_split2_noalloc(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa,
                                  int64_t ld_sa, const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
                                  int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype,
                                  int accumulate, void* stream) {
  GemmCall g;
  const int rc = gemm_validate(op, flags | FP8BLK_GEMM_SPLIT2, a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, M, N, K, c,
                               ld_c, c_dtype, accumulate, g);
  if (rc == -1) return FP8BLK_OK;
  if (rc != 0) return rc;
  const size_t need = split_workspace_bytes(g.I, g.J, 2);
  if (need == 0 || need > kScratchBytes) return FP8BLK_WORKSPACE_TOO_SMALL;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  void* ws = scratch_address();
  if (ws == nullptr) return FP8BLK_LAUNCH_FAILED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // The counters must start at zero; every call leaves them so, but a call
  // that never completed may not have: clear the ones this call uses (a fill
  // kernel, so the call can also be captured into a graph).
  const int64_t tiles = ((g.I + 255) / 256) * (g.J / 128);
  launch_clear_u32(static_cast<unsigned*>(ws), tiles, st);
  const SplitPlan plan = plan_split(g.I, g.J, g.L, ws, kScratchBytes, true);
  launch_block_gemm(a, ld_a, sa, ld_sa, b, ld_b, sb, ld_sb, g.sb_mode, g.I, g.J, g.L, c, ld_c, g.out, g.prec, plan,
                    st);
  return finish();
}

int bf16_gemm_nt(const void* a, int64_t ld_a, const void* b, int64_t ld_b,
                 int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8BLK_INVALID_ARG;
  if (c_dtype != FP8BLK_OUT_F32 && c_dtype != FP8BLK_OUT_BF16) return FP8BLK_INVALID_ARG;
  if (N % 128 != 0 || K % 64 != 0) return FP8BLK_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return FP8BLK_OK;
  if (c == nullptr || ld_c < N) return FP8BLK_INVALID_ARG;
  const int out = c_dtype == FP8BLK_OUT_BF16 ? OUT_BF16 : OUT_F32;
  if (!al16(c) || ld_c % (out == OUT_BF16 ? 8 : 4) != 0) return FP8BLK_MISALIGNED;
  if (K > 0) {
    if (a == nullptr || b == nullptr || ld_a < K || ld_b < K) return FP8BLK_INVALID_ARG;
    if (ld_a >= kMaxGemmLd / 2 || ld_b >= kMaxGemmLd / 2) return FP8BLK_UNSUPPORTED_SHAPE;
    if (!grid_fits(M, 128, N, 128)) return FP8BLK_UNSUPPORTED_SHAPE;
    if (!al16(a) || !al16(b) || ld_a % 8 != 0 || ld_b % 8 != 0) return FP8BLK_MISALIGNED;
  }
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_bf16_gemm(static_cast<const uint16_t*>(a), ld_a, static_cast<const uint16_t*>(b), ld_b, M, N, K, c, ld_c,
                   out, static_cast<hipStream_t>(stream));
  return finish();
}

size_t fp8_block_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K) {
  if (op != FP8BLK_OP_FWD && op != FP8BLK_OP_DGRAD && op != FP8BLK_OP_WGRAD) return 0;
  if (M <= 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
  int64_t I, J, L;
  gemm_dims(op, M, N, K, I, J, L);
  if (J % 128 != 0 || L % 128 != 0 || (op == FP8BLK_OP_WGRAD && I % 128 != 0) || !grid_fits(I, 128, J, 128))
    return 0;
  return small_split_workspace_bytes(I, J, small_grid_splits(I, J, L));
}

size_t fp8_block_gemm_split2_workspace_size(int op, int64_t M, int64_t N, int64_t K) {
  if (op != FP8BLK_OP_FWD && op != FP8BLK_OP_DGRAD && op != FP8BLK_OP_WGRAD) return 0;
  if (M <= 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return 0;
  int64_t I, J, L;
  gemm_dims(op, M, N, K, I, J, L);
  if (J % 128 != 0 || L % 128 != 0 || (op == FP8BLK_OP_WGRAD && I % 128 != 0) || !grid_fits(I, 128, J, 128))
    return 0;
  return split_workspace_bytes(I, J, 2);
}

int fp8_e4m3_encode(const float* x, uint8_t* q, int64_t n, void* stream) {
  if (n < 0) return FP8BLK_INVALID_ARG;
  if (n == 0) return FP8BLK_OK;
  if (x == nullptr || q == nullptr) return FP8BLK_INVALID_ARG;
  if (!al4(x)) return FP8BLK_MISALIGNED;
  if (!device_ok()) return FP8BLK_DEVICE_UNSUPPORTED;
  launch_encode(x, q, n, static_cast<hipStream_t>(stream));
  return finish();
}

const char* fp8blk_status_string(int status) {
  switch (status) {
    case FP8BLK_OK: return "ok";
    case FP8BLK_INVALID_ARG: return "invalid argument";
    case FP8BLK_UNSUPPORTED_SHAPE: return "unsupported shape (GEMM N and K must be multiples of 128)";
    case FP8BLK_MISALIGNED: return "misaligned pointer or leading dimension";
    case FP8BLK_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FP8BLK_DEVICE_UNSUPPORTED: return "device is not gfx950";
    case FP8BLK_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* fp8blk_version(void) { return "fp8blk 0.1.0 (gfx950)"; }

}  // extern "C"
