"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before touching a GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")


def _lib():
    from blockwise_fp8_linear_quant_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libfp8blk.so is not built (run __graft_entry__.build())")
    return L.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("fp8", "bf16"))))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp8_quant_1x128", "fp8_quant_128x128", "fp8_block_gemm_fwd", "fp8_block_gemm_dgrad",
              "fp8_block_gemm_wgrad", "fp8_block_gemm_workspace_size", "fp8blk_status_string",
              "bf16_gemm_nt"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    from blockwise_fp8_linear_quant_amd import _lib as L
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding lacks a signature for {n}"


def test_status_strings_and_version():
    lib = _lib()
    assert lib.fp8blk_status_string(0) == b"ok"
    assert b"128" in lib.fp8blk_status_string(2)
    assert lib.fp8blk_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.fp8blk_version()
    assert lib.fp8_block_gemm_workspace_size(0, 4096, 4096, 2048) == 0


def test_workspace_sizes():
    """The layer's shapes are not split by default (workspace size 0); grids of at most
    64 output tiles of 128 x 128 are split 8, 4 or 2 ways (the largest split with at most
    256 workgroups and two scale blocks per split), which needs a 64 KiB region it
    leaves alone (the other plan's counters) plus S FP32 partial planes of the I x J
    output.  The forced split needs a 64 KiB counter region plus two FP32
    partial tiles of 256 x 128 per output tile."""
    lib = _lib()
    FWD, DGRAD, WGRAD = 0, 1, 2
    size, size2 = lib.fp8_block_gemm_workspace_size, lib.fp8_block_gemm_split2_workspace_size
    tiles = lambda I, J: ((I + 255) // 256) * (J // 128)
    need = lambda I, J: 65536 + tiles(I, J) * 2 * 256 * 128 * 4
    out_dims = {FWD: lambda M, N, K: (M, N), DGRAD: lambda M, N, K: (M, K), WGRAD: lambda M, N, K: (N, K)}
    small = lambda op, M, N, K, s: 65536 + s * 4 * out_dims[op](M, N, K)[0] * out_dims[op](M, N, K)[1]
    for n, k in ((4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)):
        for op in (FWD, DGRAD, WGRAD):
            assert size(op, 4096, n, k) == 0
            assert size(op, 8192, n, k) == 0
        assert size2(FWD, 4096, n, k) == need(4096, n)
        assert size2(DGRAD, 4096, n, k) == need(4096, k)
        assert size2(WGRAD, 4096, n, k) == need(n, k)
    # Small grids: (op, M, N, K) -> (output tiles of 128 x 128, splits).
    for op, M, N, K, t, s in ((FWD, 256, 2048, 2048, 32, 8),     # 16 scale blocks
                              (DGRAD, 256, 2048, 2048, 32, 8),
                              (FWD, 256, 2048, 2304, 32, 8),     # 18 blocks: splits of 2 and 3
                              (DGRAD, 256, 2048, 2304, 36, 4),   # 36 tiles: 8 splits would pass 256
                              (FWD, 300, 1024, 1024, 24, 4),     # 8 blocks
                              (FWD, 512, 2048, 2048, 64, 4),     # 64 tiles: the largest split grid
                              (FWD, 300, 256, 512, 6, 2),        # 4 blocks
                              (FWD, 1000, 128, 640, 8, 2),       # 5 blocks: splits of 2 and 3
                              (WGRAD, 2048, 256, 1024, 16, 8),   # 16 token blocks
                              (WGRAD, 1000, 128, 640, 5, 4)):    # 1000 tokens pad to 8 blocks
        assert size(op, M, N, K) == small(op, M, N, K, s), (op, M, N, K, t)
    assert size(FWD, 640, 1664, 2048) == 0        # 65 tiles
    assert size(FWD, 300, 256, 384) == 0          # 3 blocks: fewer than two per split
    assert size(WGRAD, 256, 2048, 2048) == 0      # 256 tiles
    assert size2(WGRAD, 4096, 2048, 2048) == 65536 + 128 * 2 * 256 * 128 * 4    # 128 tiles: 32 MiB + counters
    assert size2(FWD, 300, 256, 384) == 65536 + 4 * 2 * 256 * 128 * 4           # 2 x 2 tiles
    # More than 16384 output tiles (the counter region's capacity): never split.
    assert size2(FWD, 256 * 129, 128 * 128, 384) == 0
    # Invalid arguments give 0.
    assert size2(7, 4096, 2048, 2048) == 0 and size2(WGRAD, -1, 2048, 2048) == 0
    assert size2(WGRAD, 4096, 2000, 2048) == 0 and size2(FWD, 300, 250, 384) == 0


def test_noalloc_split_rejects_problems_beyond_its_scratch():
    """The allocation-free split GEMM holds 128 output tiles of 256 x 128: a 2048 x 6144
    weight gradient (384 tiles) is refused before anything is launched; argument
    errors keep their own status."""
    lib = _lib()
    P = ctypes.c_void_p(16)
    f = lib.fp8_block_gemm_split2_noalloc
    assert f(2, 0, P, 4096, P, 2048, P, 4096, P, 6144, 4096, 2048, 6144, P, 6144, 0, 0, None) == 4
    assert f(0, 0, P, 2048, P, 8192, P, 2048, P, 0, 8192, 4096, 2048, P, 4096, 1, 0, None) == 4
    assert f(2, 0, P, 4096, P, 2048, P, 4096, P, 2000, 4096, 2000, 2048, P, 2048, 0, 0, None) == 2
    assert f(7, 0, P, 4096, P, 2048, P, 4096, P, 2048, 4096, 2048, 2048, P, 2048, 0, 0, None) == 1
    assert f(2, 0, None, 0, None, 0, None, 0, None, 0, 4096, 0, 2048, None, 0, 0, 0, None) == 0   # empty


def test_misaligned_workspace_rejected_before_launch():
    lib = _lib()
    P = ctypes.c_void_p(16)
    Q = ctypes.c_void_p(24)      # 8-byte aligned only
    # wgrad 2048 x 2048 over 4096 tokens with a misaligned workspace
    assert lib.fp8_block_gemm_wgrad(P, 4096, P, 2048, P, 4096, P, 2048, 4096, 2048, 2048, P, 2048, 0,
                                    Q, 1 << 30, None) == 3
    # the generic entry point: unknown flag bits are invalid
    assert lib.fp8_block_gemm(0, 4, P, 2048, P, 256, P, 2048, P, 0, 256, 256, 2048, P, 256, 0, 0,
                              None, 0, None) == 1


def test_validation_happens_before_launch():
    lib = _lib()
    P = ctypes.c_void_p(16)       # aligned dummy address, never dereferenced on the error paths
    Q = ctypes.c_void_p(17)       # misaligned
    # negative sizes / bad enum
    assert lib.fp8_quant_1x128(P, -1, 128, 128, 0, P, 128, P, 16, None) == 1
    assert lib.fp8_quant_1x128(P, 16, 128, 128, 2, P, 128, P, 16, None) == 1
    # ld too small
    assert lib.fp8_quant_1x128(P, 16, 128, 64, 0, P, 128, P, 16, None) == 1
    assert lib.fp8_quant_1x128(P, 300, 128, 128, 1, P, 256, P, 128, None) == 1   # ld_q < round_up(300,128)
    # null pointers
    assert lib.fp8_quant_1x128(None, 16, 128, 128, 0, P, 128, P, 16, None) == 1
    # misalignment
    assert lib.fp8_quant_1x128(Q, 16, 128, 128, 0, P, 128, P, 16, None) == 3
    assert lib.fp8_quant_1x128(P, 16, 128, 132, 0, P, 128, P, 16, None) == 3
    # zero-size problems are valid no-ops, even with null pointers
    assert lib.fp8_quant_1x128(None, 0, 128, 128, 0, None, 128, None, 16, None) == 0
    assert lib.fp8_quant_128x128(None, 5, 0, 0, None, 0, None, None, 0, None, None) == 0
    # qT / scalesT must come together
    assert lib.fp8_quant_128x128(P, 128, 128, 128, P, 128, P, P, 128, None, None) == 1
    # GEMM shapes: N, K multiples of 128
    assert lib.fp8_block_gemm_fwd(P, 256, P, 16, P, 256, P, 16, 200, 256, P, 200, 0, None, 0, None) == 2
    assert lib.fp8_block_gemm_fwd(P, 256, P, 16, P, 256, P, 16, 256, 200, P, 256, 0, None, 0, None) == 2
    assert lib.fp8_block_gemm_dgrad(P, 256, P, 16, P, 256, P, 16, 100, 256, P, 100, 1, None, 0, None) == 2
    assert lib.fp8_block_gemm_wgrad(P, 128, P, 16, P, 128, P, 128, 100, 130, 128, P, 128, 0, None, 0, None) == 2
    # bad dtype / accumulate flags
    assert lib.fp8_block_gemm_fwd(P, 256, P, 16, P, 256, P, 16, 256, 256, P, 256, 7, None, 0, None) == 1
    assert lib.fp8_block_gemm_wgrad(P, 128, P, 128, P, 128, P, 128, 100, 128, 128, P, 128, 2, None, 0, None) == 1
    # GEMM ld checks
    assert lib.fp8_block_gemm_fwd(P, 128, P, 16, P, 256, P, 16, 256, 256, P, 256, 0, None, 0, None) == 1
    assert lib.fp8_block_gemm_fwd(P, 256, P, 8, P, 256, P, 16, 256, 256, P, 256, 0, None, 0, None) == 1
    # GEMM misalignment (ld_sx not a multiple of 4, odd pointer)
    assert lib.fp8_block_gemm_fwd(P, 256, P, 18, P, 256, P, 16, 256, 256, P, 256, 0, None, 0, None) == 3
    assert lib.fp8_block_gemm_fwd(Q, 256, P, 16, P, 256, P, 16, 256, 256, P, 256, 0, None, 0, None) == 3
    # zero-size GEMMs are no-ops
    assert lib.fp8_block_gemm_fwd(None, 0, None, 0, None, 0, None, 0, 0, 256, None, 0, 0, None, 0, None) == 0
    assert lib.fp8_e4m3_encode(None, None, 0, None) == 0
    assert lib.fp8_e4m3_encode(P, P, -1, None) == 1


def test_size_limits_are_per_row_and_per_grid():
    """Operands past 2 GiB and more than 65535 token groups pass the size checks.

    Each such call is stopped by a deliberately misaligned pointer, which is
    checked after the sizes: status 3 (MISALIGNED) instead of 2
    (UNSUPPORTED_SHAPE) shows the sizes passed, and nothing is launched.
    """
    lib = _lib()
    P = ctypes.c_void_p(16)
    Q = ctypes.c_void_p(17)
    M = (1 << 20) + 300                     # 2^20 + 300 rows of 2048 codes: 2.15 GB
    Mp = -(-M // 128) * 128
    assert lib.fp8_block_gemm_fwd(Q, 2048, P, M, P, 2048, P, M, 256, 2048, P, 256, 1, None, 0, None) == 3
    assert lib.fp8_block_gemm_wgrad(Q, Mp, P, 2048, P, Mp, P, 256, M, 2048, 256, P, 256, 0, None, 0, None) == 3
    T = 65536 * 128 + 300                   # 65539 token groups
    Tp = -(-T // 128) * 128
    assert lib.fp8_quant_1x128_dual(Q, T, 128, 128, P, 128, P, T, P, Tp, P, 128, None) == 3
    assert lib.fp8_quant_1x128(Q, T, 128, 128, 1, P, Tp, P, 128, None) == 3
    assert lib.fp8_quant_128x128(Q, T, 128, 128, P, 128, P, None, 0, None, None) == 3
    assert lib.bf16_gemm_nt(Q, 2048, P, 2048, M, 256, 2048, P, 256, 0, None) == 3
    # the limits themselves: a row of 2^23 bytes, a row-wise grid of 65536
    # column groups, more than 2^31 - 1 workgroups
    assert lib.fp8_block_gemm_fwd(P, 1 << 23, P, 16, P, 2048, P, 16, 256, 2048, P, 256, 1, None, 0, None) == 2
    assert lib.fp8_block_gemm_wgrad(P, 1 << 23, P, 256, P, 1 << 23, P, 256, 1 << 23, 256, 256, P, 256, 0, None, 0,
                                    None) == 2
    assert lib.bf16_gemm_nt(P, 1 << 22, P, 2048, 16, 256, 2048, P, 256, 0, None) == 2
    big = 1 << 23
    assert lib.fp8_quant_1x128(P, 4, big, big, 0, P, big, P, 4, None) == 2
    assert lib.fp8_quant_1x128_dual(P, big, big, big, P, big, P, big, P, big, P, big, None) == 2
    assert lib.fp8_quant_128x128(P, big, big, big, P, big, P, None, 0, None, None) == 2
    # absurd sizes are rejected before any arithmetic on them can overflow
    huge = 1 << 62
    assert lib.fp8_quant_1x128(P, huge, 128, 128, 1, P, huge, P, 128, None) == 2
    assert lib.fp8_quant_1x128_dual(P, huge, 128, 128, P, 128, P, huge, P, huge, P, 128, None) == 2
    assert lib.fp8_block_gemm_wgrad(P, 128, P, 256, P, 128, P, 256, huge, 256, 256, P, 256, 0, None, 0, None) == 2
    assert lib.fp8_block_gemm_fwd(P, 2048, P, huge, P, 2048, P, huge, 256, 2048, P, 256, 1, None, 0, None) == 2
    assert lib.bf16_gemm_nt(P, huge, P, 2048, 16, 256, 2048, P, 256, 0, None) == 2


def test_binding_raises_without_library(tmp_path):
    from blockwise_fp8_linear_quant_amd import _lib as L
    saved = L._lib
    try:
        L._lib = None
        with pytest.raises(ImportError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved


def test_generic_gemm_validation():
    lib = _lib()
    P = ctypes.c_void_p(16)
    # bad op, bad flags, accumulate on a forward, BF16 weight gradient
    assert lib.fp8_block_gemm(7, 0, P, 256, P, 16, P, 256, P, 0, 16, 256, 256, P, 256, 0, 0, None, 0, None) == 1
    assert lib.fp8_block_gemm(0, 5, P, 256, P, 16, P, 256, P, 0, 16, 256, 256, P, 256, 0, 0, None, 0, None) == 1
    assert lib.fp8_block_gemm(0, 1, P, 256, P, 16, P, 256, P, 0, 16, 256, 256, P, 256, 0, 1, None, 0, None) == 1
    assert lib.fp8_block_gemm(2, 1, P, 256, P, 16, P, 256, P, 256, 16, 256, 256, P, 256, 1, 0, None, 0, None) == 1
    # shape rules are those of the named calls
    assert lib.fp8_block_gemm(0, 1, P, 256, P, 16, P, 256, P, 0, 16, 200, 256, P, 256, 0, 0, None, 0, None) == 2
    assert lib.fp8_block_gemm(0, 1, None, 0, None, 0, None, 0, None, 0, 0, 256, 256, None, 0, 0, 0, None, 0,
                              None) == 0


def test_bf16_gemm_validation():
    lib = _lib()
    P = ctypes.c_void_p(16)
    # bad dtype, negative size, N not a multiple of 128, K not a multiple of 64
    assert lib.bf16_gemm_nt(P, 64, P, 64, 16, 128, 64, P, 128, 5, None) == 1
    assert lib.bf16_gemm_nt(P, 64, P, 64, -1, 128, 64, P, 128, 0, None) == 1
    assert lib.bf16_gemm_nt(P, 64, P, 64, 16, 100, 64, P, 128, 0, None) == 2
    assert lib.bf16_gemm_nt(P, 96, P, 96, 16, 128, 96, P, 128, 0, None) == 2
    # leading dimensions: too small, not a multiple of 8 elements, misaligned pointer
    assert lib.bf16_gemm_nt(P, 32, P, 64, 16, 128, 64, P, 128, 0, None) == 1
    assert lib.bf16_gemm_nt(P, 68, P, 64, 16, 128, 64, P, 128, 0, None) == 3
    assert lib.bf16_gemm_nt(ctypes.c_void_p(18), 64, P, 64, 16, 128, 64, P, 128, 0, None) == 3
    assert lib.bf16_gemm_nt(P, 64, P, 64, 16, 128, 64, P, 132, 1, None) == 3
    # empty outputs are no-ops
    assert lib.bf16_gemm_nt(None, 0, None, 0, 0, 128, 64, None, 0, 0, None) == 0


def test_dual_quantiser_validation():
    lib = _lib()
    P = ctypes.c_void_p(16)
    # missing output, leading dimensions too small, misaligned qT
    assert lib.fp8_quant_1x128_dual(P, 100, 256, 256, P, 256, P, 100, None, 128, P, 256, None) == 1
    assert lib.fp8_quant_1x128_dual(P, 100, 256, 256, P, 256, P, 100, P, 112, P, 256, None) == 1
    assert lib.fp8_quant_1x128_dual(P, 100, 256, 256, P, 256, P, 99, P, 128, P, 256, None) == 1
    assert lib.fp8_quant_1x128_dual(P, 100, 256, 256, P, 256, P, 100, ctypes.c_void_p(24), 128, P, 256, None) == 3
    assert lib.fp8_quant_1x128_dual(P, 100, 256, 256, P, 256, P, 100, P, 136, P, 256, None) == 3
    # empty input is a no-op
    assert lib.fp8_quant_1x128_dual(None, 0, 256, 256, None, 0, None, 0, None, 0, None, 0, None) == 0


def test_fused_producer_validation():
    lib = _lib()
    P = ctypes.c_void_p(16)
    # SwiGLU: missing up, ld too small, misaligned optional BF16 output
    assert lib.fp8_swiglu_quant_1x128_dual(P, 256, None, 256, 100, 256, P, 256, P, 100, P, 128, P, 256,
                                           None, 0, None) == 1
    assert lib.fp8_swiglu_quant_1x128_dual(P, 128, P, 256, 100, 256, P, 256, P, 100, P, 128, P, 256,
                                           None, 0, None) == 1
    assert lib.fp8_swiglu_quant_1x128_dual(P, 256, P, 256, 100, 256, P, 256, P, 100, P, 128, P, 256,
                                           ctypes.c_void_p(20), 256, None) == 3
    # RMSNorm: negative eps, missing rstd, misaligned gamma
    assert lib.fp8_rmsnorm_quant_1x128_dual(P, 256, P, -1.0, 100, 256, P, P, 256, P, 100, P, 128, P, 256,
                                            None, 0, None) == 1
    assert lib.fp8_rmsnorm_quant_1x128_dual(P, 256, P, 1e-6, 100, 256, None, P, 256, P, 100, P, 128, P, 256,
                                            None, 0, None) == 1
    assert lib.fp8_rmsnorm_quant_1x128_dual(P, 256, ctypes.c_void_p(18), 1e-6, 100, 256, P, P, 256, P, 100,
                                            P, 128, P, 256, None, 0, None) == 3
    assert lib.fp8_rmsnorm_quant_1x128_dual(None, 0, None, 1e-6, 0, 256, None, None, 0, None, 0, None, 0, None, 0,
                                            None, 0, None) == 0
