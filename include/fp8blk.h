/*
 * fp8blk -- blockwise-FP8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp8blk.so.  The library implements the numerics that the
 * Puro-2B report applies to its linear layers:
 *   - arxiv-wiki summary "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090
 *     within $5090", section "접근 방법" (approach), item (4): the main linear
 *     operations run in blockwise FP8 E4M3, with one scale per 1-D group of
 *     128 activation values and one scale per 128x128 weight block; master
 *     weights and optimizer state stay BF16/FP32;
 *   - paperlayer.ai summary of arXiv 2608.27370v1, appendix C
 *     "生産学習の詳細", item "FP8実装pipeline": the FP8 GEMMs are the
 *     forward, data-gradient and weight-gradient products of each linear
 *     layer; gradients stay FP32, the hidden/residual flow stays BF16.
 *
 * Numerics (readings where the pages are silent; the CPU oracle follows the
 * same readings):
 *   - E4M3 is the OCP encoding (largest finite 448, subnormals kept, 0x7F NaN);
 *   - a group's scale is the binary32 dequantisation multiplier
 *     s = fl32(amax / 448), amax = max |x| over the group's valid elements;
 *   - code = E4M3_RNE_saturating(fl32(x / s)); an all-zero group has s = 0 and
 *     codes 0x00; binary32 denormals are not flushed;
 *   - GEMMs form each 128-wide block product on the matrix cores (exactly up
 *     to FP32 rounding by default, see FP8BLK_GEMM_*), multiply it by the
 *     product of the two block scales in FP32 and add it to an FP32
 *     accumulator; BF16 outputs are rounded to nearest even.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees, synchronises or keeps state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Device faults surface at the caller's
 *     next synchronisation.
 *   - Matrices are row-major with an explicit leading dimension `ld_*` in
 *     elements (BF16: 2 bytes, codes: 1 byte, FP32: 4 bytes).
 *   - Arguments are validated before anything is launched; on error nothing is
 *     written and a non-zero fp8blk_status is returned.  Problems with a zero
 *     dimension are valid no-ops.
 *   - Code and BF16 matrices must start on 16-byte boundaries and have leading
 *     dimensions that are multiples of 16 bytes; quantiser scale outputs and
 *     128x128 block scales need 4-byte alignment; the per-row scale inputs of
 *     the GEMMs (sx, sdy, sdyT, sxT) need 16-byte alignment and a leading
 *     dimension that is a multiple of 4; FP32 outputs 16-byte alignment with ld
 *     a multiple of 4, BF16 outputs ld a multiple of 8.
 *   - Calls on one stream are ordered; calls on different streams that write
 *     the same buffers race.
 *   - GEMM workspace (ws, ws_bytes): optional caller-owned device memory,
 *     16-byte aligned, used only when a call splits its contraction.  Two
 *     plans do that, and both add the parts in a fixed order (part 0 +
 *     part 1 + ...), so results are deterministic; no floating-point atomics
 *     are used:
 *       - small grids, by default: an output of at most 64 tiles of 128 x 128
 *         (a quarter of the 256 CUs or less) is split into S = 8, 4 or 2 parts
 *         of its scale blocks, the largest S with S * tiles <= 256 and at least
 *         two blocks per part, whenever the workspace holds
 *         fp8_block_gemm_workspace_size bytes: a 64 KiB region it leaves
 *         untouched (the counters of the other plan), then S FP32 partial
 *         planes of the output, which a second kernel adds and stores;
 *       - on request (FP8BLK_GEMM_SPLIT2), any shape split in two on 256 x 128
 *         tiles, when the workspace holds fp8_block_gemm_split2_workspace_size
 *         bytes: a fixed 64 KiB region of arrival counters (one per output
 *         tile, so shapes with more than 16384 tiles are not split), then two
 *         FP32 partial tiles of 256 x 128 per output tile; the half that
 *         finishes second adds the two.  The counters must be zero before a
 *         workspace is first used (e.g. allocate it zeroed); every call leaves
 *         them zero again, and because the counter region has a fixed size one
 *         workspace may serve calls of different shapes in turn.
 *     One workspace serves one call at a time: calls that overlap in time
 *     (different streams) need their own.  The Puro-2B layer's shapes (256
 *     tiles or more) are not split by default: there the split kernels
 *     measured slower than the unsplit ones.  With too small a workspace (or
 *     NULL) a call runs unsplit.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8blk_status {
  FP8BLK_OK = 0,
  FP8BLK_INVALID_ARG = 1,        /* null pointer, negative size, ld too small, bad enum */
  FP8BLK_UNSUPPORTED_SHAPE = 2,  /* GEMM: N or K not a multiple of 128, or a size limit below */
  FP8BLK_MISALIGNED = 3,         /* pointer or leading dimension alignment */
  FP8BLK_WORKSPACE_TOO_SMALL = 4,
  FP8BLK_DEVICE_UNSUPPORTED = 5, /* current device is not gfx950 */
  FP8BLK_LAUNCH_FAILED = 6       /* hipGetLastError() after a launch */
} fp8blk_status;

enum { FP8BLK_OUT_F32 = 0, FP8BLK_OUT_BF16 = 1 };
enum { FP8BLK_OP_FWD = 0, FP8BLK_OP_DGRAD = 1, FP8BLK_OP_WGRAD = 2 };
/* How the 128-wide block products are formed (fp8_block_gemm flags):
 *   FP8BLK_GEMM_EXACT_BLOCKS (default of the named GEMM calls): the E4M3
 *     operands are converted exactly to F16 and multiplied on the F16 matrix
 *     path; each block product is exact up to FP32 rounding, so results stay
 *     within 1e-5 * sum|a*b| of the exact blockwise definition for any input.
 *   FP8BLK_GEMM_FP8_MATRIX_CORE: the block products use the FP8 matrix path
 *     (v_mfma_f32_32x32x64_f8f6f4), whose peak rate is twice the F16 one;
 *     at the layer shapes the GEMMs run about 1.4 times faster.  On gfx950 that
 *     instruction adds products in groups of 8 after aligning them to the
 *     group's largest product and truncating 13 bits below it, so a block
 *     product can be off by up to ~7 * 2^-13 of its largest term when values
 *     inside a group of 8 differ widely in magnitude.
 *   FP8BLK_GEMM_SPLIT2 (or-ed with either path): split the contraction in two
 *     (see "GEMM workspace" above) whenever the workspace holds
 *     fp8_block_gemm_split2_workspace_size bytes. */
enum { FP8BLK_GEMM_EXACT_BLOCKS = 0, FP8BLK_GEMM_FP8_MATRIX_CORE = 1, FP8BLK_GEMM_SPLIT2 = 2 };

/*
 * 1x128 group quantiser of a BF16 matrix x [rows, cols] (ld_x >= cols).
 * Source: arxiv-wiki Puro-2B summary, section "접근 방법" item (4) (1-D
 * activation groups of 128, E4M3 values).
 *
 * transpose_out = 0 (row-wise; the fwd operand X and the dgrad operand dY):
 *   groups are 128 consecutive columns of a row (the last group of a row may be
 *   shorter); q [rows, ld_q >= cols] holds the codes in x's layout;
 *   scales are group-major: scales[g * ld_s + r] for group g of row r,
 *   ld_s >= rows, g < ceil(cols/128).
 * transpose_out = 1 (token-dimension; the wgrad operands X^T and dY^T):
 *   rows are tokens; groups are 128 consecutive rows (tokens) of a column;
 *   q [cols, ld_q >= round_up(rows, 128)] holds the codes transposed (tokens
 *   contiguous), with the padding tokens rows..round_up(rows,128)-1 written as
 *   0x00; scales[g * ld_s + c] for token group g of column c, ld_s >= cols,
 *   g < ceil(rows/128).
 */
int fp8_quant_1x128(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                    int transpose_out, uint8_t* q, int64_t ld_q,
                    float* scales, int64_t ld_s, void* stream);

/*
 * Both 1x128 orientations of x [rows, cols] from a single read: the outputs of
 * fp8_quant_1x128 with transpose_out = 0 (q, scales, ld_q, ld_s) and with
 * transpose_out = 1 (qT, scalesT, ld_qT, ld_sT), bit for bit, for 2 bytes of
 * HBM read per element instead of 4.  Source: arxiv-wiki Puro-2B summary,
 * section "접근 방법" item (4) (1-D groups of 128) and paperlayer.ai summary,
 * appendix C, item "FP8実装pipeline" (X feeds both the forward and the
 * weight-gradient GEMM, dY both the data- and the weight-gradient GEMM).
 * Layouts, leading-dimension rules and padding as in fp8_quant_1x128; all
 * five pointers are required; q and qT 16-byte aligned with ld_q and ld_qT
 * multiples of 16.
 */
int fp8_quant_1x128_dual(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                         uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                         uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT, void* stream);

/*
 * Producer fusion: SwiGLU straight into both 1x128 orientations.  The BF16
 * value h = silu(g) * u (binary32: g / (1 + e^-g) * u, rounded once to BF16 to
 * nearest even) of the gate g and up u halves of the gate_up projection is
 * formed in registers and quantised exactly as fp8_quant_1x128_dual would
 * quantise a BF16 tensor holding it -- the down projection's operands for the
 * forward (q) and weight-gradient (qT) GEMMs, without writing h.  Source:
 * paperlayer.ai Puro-2B summary, appendix C, item "FP8実装pipeline" (the BF16
 * hidden flow feeding the FP8 linear GEMMs; the model is the Qwen3-1.7B
 * architecture, arxiv-wiki summary, "접근 방법" item (1), whose MLP is SwiGLU).
 * gate [rows, ld_gate >= cols], up [rows, ld_up >= cols] BF16, 16-byte aligned,
 * ld multiples of 8; outputs as in fp8_quant_1x128_dual; h_bf16 (nullable)
 * [rows, ld_h >= cols] receives h itself (16-byte aligned, ld_h % 8 == 0).
 */
int fp8_swiglu_quant_1x128_dual(const void* gate, int64_t ld_gate, const void* up, int64_t ld_up,
                                int64_t rows, int64_t cols, uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT,
                                void* h_bf16, int64_t ld_h, void* stream);

/*
 * Producer fusion: RMSNorm straight into both 1x128 orientations.  Per row,
 * rstd = 1 / sqrt(mean(x^2) + eps) (binary32, written to rstd[rows] for the
 * backward pass); y = x * rstd * gamma in binary32, rounded once to BF16, is
 * formed in registers and quantised as fp8_quant_1x128_dual would quantise a
 * BF16 tensor holding it (the qkv and gate_up inputs), without writing y.
 * Source: paperlayer.ai Puro-2B summary, appendix C, item "FP8実装pipeline"
 * (normalisation in the BF16 flow ahead of the FP8 GEMMs).  x [rows, ld_x >=
 * cols] BF16 and gamma [cols] BF16, 16-byte aligned, ld_x % 8 == 0; eps >= 0;
 * rstd 4-byte aligned; outputs as in fp8_quant_1x128_dual; y_bf16 (nullable)
 * receives y.  Two launches on the stream: row statistics, then the fused pass.
 */
int fp8_rmsnorm_quant_1x128_dual(const void* x, int64_t ld_x, const void* gamma, float eps,
                                 int64_t rows, int64_t cols, float* rstd,
                                 uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                 uint8_t* qT, int64_t ld_qT, float* scalesT, int64_t ld_sT,
                                 void* y_bf16, int64_t ld_y, void* stream);

/*
 * 128x128 block quantiser of a BF16 weight w [rows, cols] (ld_w >= cols).
 * Source: arxiv-wiki Puro-2B summary, section "접근 방법" item (4) (one scale
 * per 128x128 weight block); the transposed copy serves the data-gradient GEMM
 * (paperlayer.ai summary, appendix C, item "FP8実装pipeline").
 *
 * q [rows, ld_q >= cols]; scales dense row-major [ceil(rows/128), ceil(cols/128)].
 * If qT is non-NULL, also writes Q(w^T): qT [cols, ld_qT >= rows] with
 * qT[c * ld_qT + r] = q[r * ld_q + c], and scalesT dense row-major
 * [ceil(cols/128), ceil(rows/128)] (the transpose of scales).  qT and scalesT
 * are both NULL or both non-NULL.  Edge blocks use only their valid elements.
 */
int fp8_quant_128x128(const void* w_bf16, int64_t rows, int64_t cols, int64_t ld_w,
                      uint8_t* q, int64_t ld_q, float* scales,
                      uint8_t* qT, int64_t ld_qT, float* scalesT, void* stream);

/*
 * Forward GEMM  Y[M, N] = sum_kb Sx[m, kb] * Sw[n/128, kb] * sum_{k in kb} X[m, k] W[n, k].
 * Source: paperlayer.ai Puro-2B summary, appendix C, item "FP8実装pipeline"
 * (forward GEMM in blockwise E4M3).
 *
 * xq [M, ld_xq >= K] codes with row-wise scales sx[kb * ld_sx + m] (the
 *   transpose_out = 0 layout of fp8_quant_1x128, ld_sx >= M);
 * wq [N, ld_wq >= K] codes with block scales sw dense [N/128, K/128];
 * y  [M, ld_y >= N], FP32 or BF16 (y_dtype).
 * N and K must be multiples of 128; M is arbitrary.  ws/ws_bytes: optional
 * workspace (see the conventions above; NULL/0 is always valid).
 */
int fp8_block_gemm_fwd(const uint8_t* xq, int64_t ld_xq, const float* sx, int64_t ld_sx,
                       const uint8_t* wq, int64_t ld_wq, const float* sw,
                       int64_t M, int64_t N, int64_t K,
                       void* y, int64_t ld_y, int y_dtype,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Data-gradient GEMM  dX[M, K] = dY[M, N] . W[N, K], contraction over N.
 * Source: paperlayer.ai Puro-2B summary, appendix C, item "FP8実装pipeline"
 * (data-gradient GEMM in blockwise E4M3).
 *
 * dyq [M, ld_dyq >= N] codes with row-wise scales sdy[nb * ld_sdy + m];
 * wqT [K, ld_wqT >= N] = Q(W^T) codes with block scales swT dense [K/128, N/128]
 *   (the qT/scalesT outputs of fp8_quant_128x128 on W);
 * dx [M, ld_dx >= K], FP32 or BF16.
 * N and K must be multiples of 128; M is arbitrary.
 */
int fp8_block_gemm_dgrad(const uint8_t* dyq, int64_t ld_dyq, const float* sdy, int64_t ld_sdy,
                         const uint8_t* wqT, int64_t ld_wqT, const float* swT,
                         int64_t M, int64_t N, int64_t K,
                         void* dx, int64_t ld_dx, int dx_dtype,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Weight-gradient GEMM  dW[N, K] (+)= dY^T[N, M] . X[M, K], contraction over
 * the M tokens in groups of 128 (padded to round_up(M, 128) with zero codes).
 * Source: paperlayer.ai Puro-2B summary, appendix C, item "FP8実装pipeline"
 * (weight-gradient GEMM in blockwise E4M3, gradients in FP32).
 *
 * dyqT [N, ld_dyqT >= round_up(M,128)] token-dimension codes of dY with scales
 *   sdyT[mb * ld_sdyT + n]; xqT [K, ld_xqT >= round_up(M,128)] token-dimension
 *   codes of X with scales sxT[mb * ld_sxT + k] (fp8_quant_1x128 with
 *   transpose_out = 1);
 * dw [N, ld_dw >= K] FP32; accumulate = 0 overwrites, 1 adds to dw.
 * N and K must be multiples of 128; M is arbitrary.
 */
int fp8_block_gemm_wgrad(const uint8_t* dyqT, int64_t ld_dyqT, const float* sdyT, int64_t ld_sdyT,
                         const uint8_t* xqT, int64_t ld_xqT, const float* sxT, int64_t ld_sxT,
                         int64_t M, int64_t N, int64_t K,
                         float* dw, int64_t ld_dw, int accumulate,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Generic block-scaled GEMM: the three calls above with an explicit op and a
 * choice of matrix path (flags, see FP8BLK_GEMM_*).  Source: paperlayer.ai
 * Puro-2B summary, appendix C, item "FP8実装pipeline" (the three GEMMs).
 *   op = FP8BLK_OP_FWD:   a = xq, sa = sx, b = wq,  sb = sw  (ld_sb unused), C = Y  [M, N];
 *   op = FP8BLK_OP_DGRAD: a = dyq, sa = sdy, b = wqT, sb = swT (ld_sb unused), C = dX [M, K];
 *   op = FP8BLK_OP_WGRAD: a = dyqT, sa = sdyT, b = xqT, sb = sxT, C = dW [N, K] (FP32 only).
 * Layouts, alignment and shape rules are those of the named call.  accumulate
 * (0/1) is accepted for the weight gradient only.
 */
int fp8_block_gemm(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                   const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
                   int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype, int accumulate,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_block_gemm with the contraction split in two (FP8BLK_GEMM_SPLIT2) and no
 * workspace argument: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The split's counters and partial tiles live in a static device
 * array of the library, 64 KiB + 32 MiB per GPU, held until the process ends;
 * the call allocates nothing and clears the counters it uses with a fill
 * kernel.  Problems needing more than that -- more than 128 output tiles of
 * 256 x 128 (fp8_block_gemm_split2_workspace_size > 33619968 bytes), e.g. a
 * weight gradient larger than 2048 x 2048 -- return
 * FP8BLK_WORKSPACE_TOO_SMALL before anything is launched.  All calls on one
 * GPU share the array, so calls that overlap in time on one GPU (different
 * streams or threads) race; calls on one stream are ordered and safe.
 * Arguments, layouts and results are those of fp8_block_gemm (flags selects
 * the matrix path; FP8BLK_GEMM_SPLIT2 is implied).
 */
int fp8_block_gemm_split2_noalloc(int op, int flags, const uint8_t* a, int64_t ld_a, const float* sa,
                                  int64_t ld_sa, const uint8_t* b, int64_t ld_b, const float* sb, int64_t ld_sb,
                                  int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype,
                                  int accumulate, void* stream);

/*
 * Plain BF16 GEMM  C[M, N] = A[M, K] . B[N, K]^T  (no quantisation, FP32
 * accumulation), the BF16 baseline against which the FP8 GEMMs are compared:
 * the pages report the FP8 recipe's throughput relative to BF16 training
 * (paperlayer.ai Puro-2B summary, appendix D "MuonH Scaling-Ladder Analysis",
 * 1.36x at 1.7B; ailog.hnlab.kr post, FP8 linear layers are 72% of compute).
 * a [M, ld_a >= K], b [N, ld_b >= K] BF16 bit patterns, row-major, 16-byte
 * aligned, ld_a and ld_b multiples of 8 elements; c [M, ld_c >= N], FP32 or
 * BF16 (c_dtype, rounded to nearest even), 16-byte aligned, ld_c a multiple
 * of 4 (FP32) or 8 (BF16).  N must be a multiple of 128 and K of 64 (else
 * FP8BLK_UNSUPPORTED_SHAPE); M is arbitrary; K = 0 writes zeros.  Rows of a
 * and b must be shorter than 2^23 bytes (ld_a, ld_b < 2^22 elements).
 */
int bf16_gemm_nt(const void* a, int64_t ld_a, const void* b, int64_t ld_b,
                 int64_t M, int64_t N, int64_t K, void* c, int64_t ld_c, int c_dtype, void* stream);

/*
 * Workspace bytes a GEMM call of (op, M, N, K) uses without flags: nonzero
 * only for the small grids that are split by default (see "GEMM workspace"),
 * 0 otherwise and for invalid arguments.  The M, N, K meaning is that of the
 * named call for op.
 */
size_t fp8_block_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K);

/* Workspace bytes that FP8BLK_GEMM_SPLIT2 needs to split (op, M, N, K) in two
 * (0 for invalid arguments). */
size_t fp8_block_gemm_split2_workspace_size(int op, int64_t M, int64_t N, int64_t K);

/*
 * The library's binary32 -> E4M3 encoder applied elementwise: q[i] = E4M3(x[i])
 * with round-to-nearest-even, saturation at +-448 (infinities included), the
 * sign kept, and NaN -> 0x7F with its sign (OCP E4M3, the format named in the
 * arxiv-wiki Puro-2B summary, "접근 방법" item (4)).  Exposed so the device
 * encoder can be checked on every binary32 input.
 * x: n floats, q: n bytes, both device pointers (no alignment requirement).
 */
int fp8_e4m3_encode(const float* x, uint8_t* q, int64_t n, void* stream);

/* Human-readable name of a status code (static string). */
const char* fp8blk_status_string(int status);

/* Library version string (static). */
const char* fp8blk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8BLK_H */
