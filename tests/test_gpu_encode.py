"""GPU parity of the device E4M3 encoder (through fp8_e4m3_encode) against the
oracle, on every binary32 of magnitude in [2^-12, 2^10) (both signs) and on
random bit patterns.  The encoder shares the hardware conversion the
quantisers use, so this also pins that conversion."""

import numpy as np
import pytest

from oracle import e4m3
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_device_encoder_exhaustive_decision_range():
    import torch
    from blockwise_fp8_linear_quant_amd import binding as B
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(2.0 ** 10).view(np.uint32))
    chunk = 1 << 24
    for start in range(lo, hi, chunk):
        say("encode chunk", hex(start))
        v = np.arange(start, min(start + chunk, hi), dtype=np.uint32).view(np.float32)
        got = B.fp8_e4m3_encode(torch.from_numpy(v).cuda()).cpu().numpy()
        ref = e4m3.encode(v)
        assert np.array_equal(got, ref), hex(start)
        neg = B.fp8_e4m3_encode(torch.from_numpy(-v).cuda()).cpu().numpy()
        assert np.array_equal(neg, ref | 0x80), hex(start)


def test_device_encoder_random_and_specials():
    import torch
    from blockwise_fp8_linear_quant_amd import binding as B
    rng = np.random.default_rng(2024)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    sp = np.array([0.0, -0.0, np.inf, -np.inf, 448, -448, 449, 464, 480, 1e-45, -1e-45,
                   2.0 ** -10, 2.0 ** -9, 7.5 * 2.0 ** -9], dtype=np.float32)
    v = np.concatenate([v, sp])
    got = B.fp8_e4m3_encode(torch.from_numpy(v).cuda()).cpu().numpy()
    assert np.array_equal(got, e4m3.encode(v))
