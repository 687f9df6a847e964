"""CPU checks of the device codec header (compiled for the host with g++).

1. The exact-quotient shortcut used by the quantiser kernels equals IEEE
   division fl32(x / fl32(amax/448)) -- same E4M3 code for every pair of BF16
   values with |x| <= amax (about 1.07e9 pairs), same binary32 quotient
   whenever it is >= 2^-12.
2. The device E4M3 encoder equals the oracle's encoder on every positive
   binary32 in [2^-12, 2^10) and on a random sample of all bit patterns.
3. The table-driven group setup the kernels use for BF16 group maxima gives
   the same four constants as the direct one for every BF16 magnitude.
4. The two-operation quotient (reciprocal rounded down plus its exact
   residual term) gives the same E4M3 code as IEEE division for every pair
   of BF16 values with |x| <= amax, both signs, wherever its reciprocal is
   finite; the maxima where it is not are all below 1.4e-36 and keep the
   normalised quotient.
"""

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import e4m3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "codec_check.cpp")
INC = os.path.join(ROOT, "blockwise_fp8_linear_quant_amd", "csrc")


@pytest.fixture(scope="module")
def codec_lib(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("codec") / "libcodec.so")
    subprocess.run([gxx, "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-I", INC, SRC, "-o", out],
                   check=True)
    lib = ctypes.CDLL(out)
    lib.codec_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.codec_quotient_scan.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint64)]
    lib.codec_quotient_scan.restype = ctypes.c_int
    lib.codec_setup_table_scan.restype = ctypes.c_int
    lib.codec_quotient2_scan.argtypes = [ctypes.POINTER(ctypes.c_uint64)] * 3
    lib.codec_quotient2_scan.restype = ctypes.c_int
    return lib


def test_table_setup_equals_direct_setup_for_every_bf16_amax(codec_lib):
    assert codec_lib.codec_setup_table_scan() == 0


def test_exact_quotient_equals_ieee_division_for_all_bf16_pairs(codec_lib):
    n = ctypes.c_uint64(0)
    bad = codec_lib.codec_quotient_scan(1, 0x7F80, ctypes.byref(n))
    assert n.value > 1_000_000_000
    assert bad == 0


def test_two_operation_quotient_gives_the_ieee_codes_for_all_bf16_pairs(codec_lib):
    n, qdiff, skipped = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint64(0)
    bad = codec_lib.codec_quotient2_scan(ctypes.byref(n), ctypes.byref(qdiff), ctypes.byref(skipped))
    assert bad == 0
    assert n.value > 1_000_000_000
    # The maxima without a finite reciprocal: every BF16 magnitude below
    # 0x03E1 (about 1.32e-36) and nothing above it.
    assert skipped.value == 0x03E1 - 1
    # The binary32 quotients differ in some pairs (so the check is not vacuous),
    # never their codes.
    assert qdiff.value > 0


def _encode(lib, v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib.codec_encode(v.ctypes.data, out.ctypes.data, v.size)
    return out


def test_device_encoder_matches_oracle_exhaustively(codec_lib):
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(2.0 ** 10).view(np.uint32))
    chunk = 1 << 23
    for start in range(lo, hi, chunk):
        v = np.arange(start, min(start + chunk, hi), dtype=np.uint32).view(np.float32)
        a = _encode(codec_lib, v)
        b = e4m3.encode(v)
        assert np.array_equal(a, b), start


def test_device_encoder_matches_oracle_on_random_bits(codec_lib):
    rng = np.random.default_rng(99)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    v = np.concatenate([v, np.array([0.0, -0.0, np.inf, -np.inf, 448, -448, 464, 1e-45], dtype=np.float32)])
    assert np.array_equal(_encode(codec_lib, v), e4m3.encode(v))
