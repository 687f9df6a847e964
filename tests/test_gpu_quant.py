"""GPU parity of the quantisers: codes and scales bit-exact against the oracle.

Covers ragged and tiny shapes, the special families (power-of-two tie, signed
zeros, zero groups, denormal scales, saturation stress) and the full tensor
sizes of the workload configurations (quantiser parity is always checked on
every element).
"""

import os

import numpy as np
import pytest

from blockwise_fp8_linear_quant_amd import workloads as W
from oracle import compare, quant
from tests.gpu_util import dev_bf16, host, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd import binding
    return binding


def rows_gpu(B, bits):
    q, s = B.fp8_quant_1x128(dev_bf16(bits))
    return host(q), host(s)


def check_rows(B, bits, label):
    say("quant rows", label, bits.shape)
    q, s = rows_gpu(B, bits)
    oq, os_ = quant.quant_1x128_rows(bits)
    ok, n = compare.check_exact(q, oq)
    assert ok, f"{label}: {n} codes differ"
    ok, n = compare.check_exact(np.ascontiguousarray(s), np.ascontiguousarray(os_.T))
    assert ok, f"{label}: {n} scales differ"


def check_tokens(B, bits, label):
    say("quant tokens", label, bits.shape)
    M = bits.shape[0]
    q, s = B.fp8_quant_1x128(dev_bf16(bits), transpose_out=True)
    q, s = host(q), host(s)
    oq, os_ = quant.quant_1x128_tokens(bits)
    assert q.shape[1] == -(-M // 128) * 128
    ok, n = compare.check_exact(np.ascontiguousarray(q[:, :M]), oq)
    assert ok, f"{label}: {n} codes differ"
    assert np.all(q[:, M:] == 0), f"{label}: padding bytes not zero"
    ok, n = compare.check_exact(np.ascontiguousarray(s), np.ascontiguousarray(os_.T))
    assert ok, f"{label}: {n} scales differ"


def check_dual(B, bits, label):
    """Single-read dual quantiser: both orientations bit-exact against the oracle."""
    say("quant dual", label, bits.shape)
    M = bits.shape[0]
    q, s, qT, sT = (host(t) for t in B.fp8_quant_1x128_dual(dev_bf16(bits)))
    oq, os_ = quant.quant_1x128_rows(bits)
    oqT, osT = quant.quant_1x128_tokens(bits)
    assert qT.shape[1] == -(-M // 128) * 128
    assert np.all(qT[:, M:] == 0), f"{label}: padding bytes not zero"
    for name, got, ref in (("q", q, oq), ("s", s, os_.T), ("qT", qT[:, :M], oqT), ("sT", sT, osT.T)):
        ok, n = compare.check_exact(np.ascontiguousarray(got), np.ascontiguousarray(ref))
        assert ok, f"{label}: {name}: {n} entries differ"


def check_blocks(B, bits, label):
    say("quant 128x128", label, bits.shape)
    q, s, qT, sT = B.fp8_quant_128x128(dev_bf16(bits), with_transpose=True)
    q, s, qT, sT = host(q), host(s), host(qT), host(sT)
    oq, os_ = quant.quant_128x128(bits)
    for name, got, ref in (("q", q, oq), ("s", s, os_), ("qT", qT, oq.T), ("sT", sT, os_.T)):
        ok, n = compare.check_exact(np.ascontiguousarray(got), np.ascontiguousarray(ref))
        assert ok, f"{label}: {name}: {n} entries differ"
    # The transposed copy is also Q(W^T) computed from the transposed input.
    oqt, ost = quant.quant_128x128(np.ascontiguousarray(bits.T))
    assert np.array_equal(qT, oqt) and np.array_equal(sT.view(np.uint32), ost.view(np.uint32))


SMALL_SHAPES = [(1, 1), (1, 128), (3, 5), (7, 127), (8, 129), (33, 300), (300, 256), (257, 2048), (129, 136)]


@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_and_ragged_shapes(B, shape):
    bits = W.normal_bf16(shape, 1.0, W.seed_for(90, shape[0], 0, "x"))
    check_rows(B, bits, "small")
    check_tokens(B, bits, "small")
    check_dual(B, bits, "small")
    check_blocks(B, bits, "small")


@pytest.mark.parametrize("shape", [(256, 136), (384, 1000), (128, 8), (200, 264)])
def test_ragged_columns_dual_and_blocks(B, shape):
    """Column counts that are not multiples of 128, with whole and partial
    128-row tiles: the transposed outputs of the dual and 128x128 quantisers
    leave through a staged tile that must skip the missing columns."""
    bits = W.normal_bf16(shape, 1.0, W.seed_for(91, shape[0], shape[1], "x"))
    check_dual(B, bits, "ragged columns")
    check_blocks(B, bits, "ragged columns")
    check_dual(B, bits, "small")
    check_blocks(B, bits, "small")


def test_pow2_tie_case(B):
    g = {}
    for line in open(os.path.join(GOLDEN, "quant_pow2_tie.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()[:2]
            g[k] = int(v, 16)
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0], x[0, 1] = g["x_bits_0"], g["x_bits_1"]
    q, s = rows_gpu(B, x)
    assert s.view(np.uint32)[0, 0] == g["scale_bits"]
    assert q[0, 0] == g["code_0"] and q[0, 1] == g["code_1"] and np.all(q[0, 2:] == 0)


def test_special_values(B):
    rng = np.random.default_rng(5)
    x = W.normal_bf16((64, 512), 1.0, 77)
    x[0, :] = 0x8000                      # all negative zeros -> zero group, codes 0x00
    x[1, :128] = 0                        # a zero group
    x[2, :] = 0x8000
    x[2, 5] = 0x3F80                      # -0 inside a non-zero group keeps its sign (0x80)
    x[3, 0:128] = 0x0001                  # smallest BF16 subnormals -> denormal scale
    x[3, 1] = 0x8001
    x[4, 130] = 0x7F7F                    # largest finite BF16
    x[5, 256:384] = 0x4400                # block-constant group
    x[6, 300] = 0x47C3                    # 1e5-ish spike
    for r in range(8, 64):                # all BF16 magnitudes as group maxima
        x[r, 384 + (r % 128)] = (r * 583) & 0x7F7F
    check_rows(B, x, "specials")
    check_tokens(B, x, "specials")
    check_dual(B, x, "specials")
    check_blocks(B, x, "specials")
    q, s = rows_gpu(B, x)
    assert np.all(q[0] == 0) and s[0, 0] == 0
    assert q[2, 0] == 0x80 and q[2, 5] == 0x7E
    assert 0 < s[0, 3] < np.finfo(np.float32).tiny


def test_maxima_without_finite_reciprocal(B):
    """Groups whose maximum is below about 1.3e-36 have no finite binary32
    reciprocal of their scale; a wave or tile holding one takes the normalised
    quotient instead of the two-operation one.  Block (0, 0) holds only such
    values (so do the token groups of its columns and the row groups of its
    rows), the rest of the tensor is ordinary, so both forms meet in one call."""
    rng = np.random.default_rng(17)
    x = W.normal_bf16((256, 384), 1.0, W.seed_for(92, 0, 0, "x"))
    tiny = rng.integers(1, 0x03E1, size=(128, 128)).astype(np.uint16)
    tiny |= (rng.integers(0, 2, size=(128, 128)).astype(np.uint16) << 15)
    x[:128, :128] = tiny
    x[5, 7] = 0x03E0                          # the largest magnitude of that range
    check_rows(B, x, "tiny maxima")
    check_tokens(B, x, "tiny maxima")
    check_dual(B, x, "tiny maxima")
    check_blocks(B, x, "tiny maxima")


def test_every_bf16_magnitude_as_amax(B):
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((bits.size, 128), dtype=np.uint16)
    x[:, 3] = bits
    x[:, 4] = bits | 0x8000
    x[:, 5] = bits >> 3
    x[:, 6] = (bits >> 1) | 0x8000
    check_rows(B, x, "all-amax")
    check_dual(B, x, "all-amax")


def test_config1_tensors(B):
    x = W.normal_bf16((256, 2048), 1.0, W.seed_for(1, 0, "o", "x"))
    w = W.normal_bf16((2048, 2048), 0.02, W.seed_for(1, 0, "o", "w"))
    check_rows(B, x, "cfg1 X")
    check_blocks(B, w, "cfg1 W")


@pytest.mark.parametrize("lin", [n for n, _, _ in W.LINEARS])
def test_layer_tensors_M4096(B, lin):
    """Configurations 2 and 3: one decoder layer at 4096 tokens, full tensors."""
    _, k, n = [l for l in W.LINEARS if l[0] == lin][0]
    x = W.normal_bf16((4096, k), 1.0, W.seed_for(2, 0, lin, "x"))
    w = W.normal_bf16((n, k), 0.02, W.seed_for(2, 0, lin, "w"))
    dy = W.normal_bf16((4096, n), 1e-3, W.seed_for(2, 0, lin, "dy"))
    check_rows(B, x, f"{lin} X")
    check_tokens(B, x, f"{lin} X")
    check_blocks(B, w, f"{lin} W")
    check_rows(B, dy, f"{lin} dY")
    check_tokens(B, dy, f"{lin} dY")
    check_dual(B, x, f"{lin} X")
    check_dual(B, dy, f"{lin} dY")


def check_both_orientations(B, bits, label):
    """Row-wise and token-dimension kernels and the single-read dual kernel, all
    against one oracle evaluation per orientation (large tensors)."""
    say("quant rows/tokens/dual", label, bits.shape)
    M = bits.shape[0]
    oq, os_ = quant.quant_1x128_rows(bits)
    oqT, osT = quant.quant_1x128_tokens(bits)
    x = dev_bf16(bits)
    q, s = (host(t) for t in B.fp8_quant_1x128(x))
    qt, st = (host(t) for t in B.fp8_quant_1x128(x, transpose_out=True))
    dq, ds, dqT, dsT = (host(t) for t in B.fp8_quant_1x128_dual(x))
    for kern, qT_, sT_, q_, s_ in (("separate", qt, st, q, s), ("dual", dqT, dsT, dq, ds)):
        assert np.all(qT_[:, M:] == 0), f"{label} {kern}: padding bytes not zero"
        for name, got, ref in (("q", q_, oq), ("s", s_, os_.T), ("qT", qT_[:, :M], oqT), ("sT", sT_, osT.T)):
            ok, n = compare.check_exact(np.ascontiguousarray(got), np.ascontiguousarray(ref))
            assert ok, f"{label} {kern}: {name}: {n} entries differ"


@pytest.mark.parametrize("layer", [0, 27])
@pytest.mark.parametrize("lin", [n for n, _, _ in W.LINEARS])
def test_outlier_layer_tensors_M8192(B, layer, lin):
    """Configuration 4: every quantised tensor of the first and last layers' four
    linears at 8192 tokens (X with 1% of channels x32, W, dY), full tensors."""
    x, w, dy = W.layer_tensors(4, layer, lin, 8192, outliers=True)
    K = x.shape[1]
    big = np.abs(quant.bf16_bits_to_f32(x)).max(axis=0) > 16
    assert big.sum() >= round(0.01 * K)           # the outlier channels are there
    check_both_orientations(B, x, f"cfg4 L{layer} {lin} X")
    check_blocks(B, w, f"cfg4 L{layer} {lin} W")
    check_both_orientations(B, dy, f"cfg4 L{layer} {lin} dY")


def test_stress_ragged_M3000(B):
    """Configuration 5: 3000 tokens, Student-t(3), zero groups, spikes, a denormal scale."""
    x = W.student_t_stress((3000, 6144), W.seed_for(5, 0, "down", "x"))
    dy = W.normal_bf16((3000, 2048), 1e-3, W.seed_for(5, 0, "down", "dy"))
    w = W.normal_bf16((2048, 6144), 0.02, W.seed_for(5, 0, "down", "w"))
    check_rows(B, x, "cfg5 X")
    check_tokens(B, x, "cfg5 X")
    check_tokens(B, dy, "cfg5 dY")
    check_dual(B, x, "cfg5 X")
    check_dual(B, dy, "cfg5 dY")
    check_blocks(B, w, "cfg5 W")
    _, s = quant.quant_1x128_rows(x)
    assert np.any(s == 0) and np.any((s > 0) & (s < np.finfo(np.float32).tiny))


def test_determinism(B):
    x = W.normal_bf16((1000, 1024), 1.0, 3)
    a = rows_gpu(B, x)
    b = rows_gpu(B, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
