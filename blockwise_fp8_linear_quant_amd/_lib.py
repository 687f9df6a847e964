"""ctypes loader for libfp8blk.so (the gfx950 HIP library).

There is no fallback: if the shared library is missing or cannot be loaded,
importing the binding raises, so no result can silently come from anywhere
but the HIP kernels.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8blk.so")

# Every symbol include/fp8blk.h declares, with its ctypes signature.
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "fp8_quant_1x128": (_i32, [_vp, _i64, _i64, _i64, _i32, _vp, _i64, _vp, _i64, _vp]),
    "fp8_quant_1x128_dual": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "fp8_swiglu_quant_1x128_dual": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                           _vp, _i64, _vp, _i64, _vp]),
    "fp8_rmsnorm_quant_1x128_dual": (_i32, [_vp, _i64, _vp, ctypes.c_float, _i64, _i64, _vp, _vp, _i64, _vp, _i64,
                                            _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "fp8_quant_128x128": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp]),
    "fp8_block_gemm_fwd": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                  _vp, _i64, _i32, _vp, _sz, _vp]),
    "fp8_block_gemm_dgrad": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                    _vp, _i64, _i32, _vp, _sz, _vp]),
    "fp8_block_gemm_wgrad": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                                    _vp, _i64, _i32, _vp, _sz, _vp]),
    "fp8_block_gemm": (_i32, [_i32, _i32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                              _vp, _i64, _i32, _i32, _vp, _sz, _vp]),
    "fp8_block_gemm_split2_noalloc": (_i32, [_i32, _i32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                             _i64, _vp, _i64, _i32, _i32, _vp]),
    "bf16_gemm_nt": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _i32, _vp]),
    "fp8_block_gemm_workspace_size": (_sz, [_i32, _i64, _i64, _i64]),
    "fp8_block_gemm_split2_workspace_size": (_sz, [_i32, _i64, _i64, _i64]),
    "fp8_e4m3_encode": (_i32, [_vp, _vp, _i64, _vp]),
    "fp8blk_status_string": (ctypes.c_char_p, [_i32]),
    "fp8blk_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path=LIB_PATH):
    """Load libfp8blk.so once and attach the declared signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class Fp8BlkError(RuntimeError):
    pass


def check(status, what):
    if status != 0:
        msg = load().fp8blk_status_string(status).decode()
        raise Fp8BlkError(f"{what} failed with status {status}: {msg}")
