"""GPU parity of the device E4M3 encoder (through fp8_e4m3_encode) against the
oracle: on every binary32 of magnitude in [2^-12, 2^10) (both signs) against
the oracle's encoder itself, on random bit patterns, and on all 2^32 bit
patterns against the oracle's decision boundaries (tests/encode_rule.py).  The encoder shares the hardware conversion the
quantisers use, so this also pins that conversion."""

import numpy as np
import pytest

from oracle import e4m3
from tests.encode_rule import decision_midpoints, expected_codes_torch
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


def test_device_encoder_all_binary32():
    """Every one of the 2^32 binary32 bit patterns through the device encoder."""
    import torch
    from blockwise_fp8_linear_quant_amd import binding as B
    mids = torch.from_numpy(decision_midpoints()).cuda()
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        say("encode all-binary32 chunk", hex(start))
        b64 = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        bits = torch.where(b64 >= 2 ** 31, b64 - 2 ** 32, b64).to(torch.int32)   # the same 32 bits, signed
        got = B.fp8_e4m3_encode(bits.view(torch.float32)).to(torch.int64)
        want = expected_codes_torch(torch, bits, mids)
        bad = int((got != want).sum())
        assert bad == 0, (hex(start), bad)
