"""GPU parity past the sizes where 32-bit offsets or a 65535-tile grid axis would break.

* Forward GEMM with X codes of 2^20 + 300 rows x 2048 (2.15 GB, beyond 2 GiB)
  and a ragged last tile.
* Weight-gradient GEMM contracting over 2^20 + 300 tokens (dYqT 2048 x
  1048832 codes, 2.15 GB).
* Dual and token-dimension quantisers over 65536 * 128 + 300 tokens (more
  than 65535 token groups; input 2.15 GB, 44 valid tokens in the last group).
* The BF16 comparison GEMM with A of 2^20 + 300 rows x 1024 BF16 (2.15 GB).

Inputs repeat a small seeded block with a period along the long dimension;
each period's scales (GEMM) or values (quantisers) are multiplied by its own
power of two, which is exact, so a tile read or written at a wrong row shows
up as a wrong result.  Outputs are checked on sampled rows, columns and
groups, which the oracle computes one by one: GEMM outputs to the FP32
tolerance, quantiser codes and scales bit-exact.  Output buffers start filled
with a code the quantisers never produce (0x7F) so that an unwritten tile
cannot pass.
"""

import numpy as np
import pytest

from blockwise_fp8_linear_quant_amd import workloads as W
from oracle import compare, gemm, quant
from tests.gpu_util import host, sample_index, say

pytestmark = pytest.mark.gpu

LONG = (1 << 20) + 300           # rows / tokens past 2 GiB at 2048 bytes per row
TOKENS = 65536 * 128 + 300       # token groups past 65535


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd import binding
    return binding


def _period_pow2(n, period, spread):
    """2^((r // period) % spread - spread // 2) for r in [0, n), float32."""
    p = (np.arange(n, dtype=np.int64) // period) % spread - spread // 2
    return np.ldexp(np.float32(1.0), p).astype(np.float32)


def test_forward_gemm_operand_past_2_gib(B):
    import torch
    rng = np.random.default_rng(71)
    M, K, N, P = LONG, 2048, 256, 4096
    xq0, sx0 = quant.quant_1x128_rows(W.normal_bf16((P, K), 1.0, seed=711))
    wq, sw = quant.quant_128x128(W.normal_bf16((N, K), 0.02, seed=712))
    sx = sx0[np.arange(M) % P] * _period_pow2(M, P, 7)[:, None]        # [M, K/128]
    say("large fwd gemm", M, N, K)
    xq_d = torch.from_numpy(xq0).cuda().repeat(-(-M // P), 1)[:M]
    assert xq_d.is_contiguous() and xq_d.numel() >= 1 << 31
    sx_d = torch.from_numpy(np.ascontiguousarray(sx.T)).cuda()            # [K/128, M]
    y = B.fp8_block_gemm_fwd(xq_d, sx_d, torch.from_numpy(wq).cuda(), torch.from_numpy(sw).cuda(),
                             out_dtype=torch.float32)
    rows = sample_index(M, 48, rng, must=(0, P - 1, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, M // 2,
                                          (M // 128) * 128 - 1, (M // 128) * 128, M - 1))
    got = host(y[torch.from_numpy(rows).cuda()])
    want, bnd = gemm.block_gemm(xq0[rows % P], sx[rows], wq, quant.expand_block_scales(sw, N))
    ok, rep = compare.check_fp32(got, want, bnd)
    assert ok, rep


def test_weight_gradient_contraction_past_2_gib(B):
    import torch
    rng = np.random.default_rng(72)
    M, N, K, P = LONG, 2048, 256, 8192
    Mp = -(-M // 128) * 128
    G = Mp // 128
    # Token-dimension operands: dYqT [N, Mp], XqT [K, Mp]; one P-token block
    # repeated, its scales per 128-token group times a power of two per period.
    dyq0, sdy0 = quant.quant_1x128_tokens(W.normal_bf16((P, N), 1e-3, seed=721))   # [N, P], [N, P/128]
    xq0, sx0 = quant.quant_1x128_tokens(W.normal_bf16((P, K), 1.0, seed=722))
    g_per = P // 128
    mult = _period_pow2(G, g_per, 5)
    sdy = sdy0[:, np.arange(G) % g_per] * mult[None, :]                    # [N, G]
    sx = sx0[:, np.arange(G) % g_per] * mult[None, :]

    def full_codes(c0):
        # columns past M are padding: zero codes
        c = np.tile(c0, (1, Mp // P + 1))[:, :Mp]
        c[:, M:] = 0
        return c

    say("large wgrad gemm", M, N, K)
    dyq_d = torch.from_numpy(dyq0).cuda().repeat(1, Mp // P + 1)[:, :Mp].contiguous()
    dyq_d[:, M:] = 0
    xq_d = torch.from_numpy(xq0).cuda().repeat(1, Mp // P + 1)[:, :Mp].contiguous()
    xq_d[:, M:] = 0
    assert dyq_d.numel() >= 1 << 31
    sdy_d = torch.from_numpy(np.ascontiguousarray(sdy.T)).cuda()          # [G, N]
    sx_d = torch.from_numpy(np.ascontiguousarray(sx.T)).cuda()            # [G, K]
    dw = B.fp8_block_gemm_wgrad(dyq_d, sdy_d, xq_d, sx_d, M=M)
    rows = sample_index(N, 12, rng, must=(0, N - 1, 1024, 2047))
    cols = sample_index(K, 12, rng, must=(0, K - 1, 128))
    got = host(dw)[np.ix_(rows, cols)]
    want, bnd = gemm.block_gemm(full_codes(dyq0[rows]), sdy[rows], full_codes(xq0[cols]), sx[cols])
    ok, rep = compare.check_fp32(got, want, bnd)
    assert ok, rep


def test_bf16_gemm_operand_past_2_gib(B):
    import torch
    rng = np.random.default_rng(74)
    M, K, N, P = LONG, 1024, 256, 4096
    a0 = W.normal_bf16((P, K), 1.0, seed=741)
    b = W.normal_bf16((N, K), 0.02, seed=742)
    mult = _period_pow2(M, P, 7)
    say("large bf16 gemm", M, N, K)
    a_d = torch.from_numpy(a0.view(np.int16)).cuda().view(torch.bfloat16).repeat(-(-M // P), 1)[:M]
    a_d.mul_(torch.from_numpy(mult).cuda().to(torch.bfloat16)[:, None])       # powers of two: exact
    assert a_d.numel() * 2 >= 1 << 31
    c = B.bf16_gemm_nt(a_d, torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16),
                       out_dtype=torch.float32)
    rows = sample_index(M, 48, rng, must=(0, P - 1, (1 << 20) - 1, 1 << 20, M // 2, (M // 128) * 128, M - 1))
    got = host(c[torch.from_numpy(rows).cuda()])
    a_rows = W.f32_to_bf16_bits(quant.bf16_bits_to_f32(a0[rows % P]) * mult[rows][:, None])
    want, bnd = gemm.bf16_gemm(a_rows, b)
    ok, rep = compare.check_fp32(got, want, bnd)
    assert ok, rep


@pytest.fixture(scope="module")
def long_tokens(B):
    """BF16 [TOKENS, 128] on the device: a seeded 16000-token block repeated, each
    repetition times its own power of two; and a host function giving rows."""
    import torch
    P, C = 16000, 128
    base = W.normal_bf16((P, C), 1.0, seed=731)
    mult = _period_pow2(TOKENS, P, 5)
    say("long token tensor", TOKENS, C)
    x = torch.from_numpy(base.view(np.int16)).cuda().view(torch.bfloat16).repeat(-(-TOKENS // P), 1)[:TOKENS]
    m = torch.from_numpy(mult).cuda().to(torch.bfloat16)
    x.mul_(m[:, None])                    # power-of-two factors: exact in BF16

    def rows(r0, r1):
        r = np.arange(r0, r1)
        v = quant.bf16_bits_to_f32(base[r % P]) * mult[r][:, None]
        return W.f32_to_bf16_bits(v)

    return x, rows


def _filled(shape, torch, dtype, value):
    return torch.full(shape, value, dtype=dtype, device="cuda")


def test_dual_quantiser_past_65535_token_groups(B, long_tokens):
    import torch
    x, rows = long_tokens
    R, C = x.shape
    Mp = -(-R // 128) * 128
    q = _filled((R, C), torch, torch.uint8, 0x7F)
    qT = _filled((C, Mp), torch, torch.uint8, 0x7F)
    say("large dual quantiser", R, C)
    q, s, qT, sT = B.fp8_quant_1x128_dual(x, q=q, qT=qT)
    ntg = Mp // 128
    for g in sorted({0, 1, 65534, 65535, 65536, ntg - 2, ntg - 1}):
        r0, r1 = g * 128, min(R, g * 128 + 128)
        bits = rows(r0, r1)
        oq, os_ = quant.quant_1x128_rows(bits)
        ok, n = compare.check_exact(host(q[r0:r1]), oq)
        assert ok, ("row-wise codes", g, n)
        ok, n = compare.check_exact(host(s[:, r0:r1]).T.copy(), os_)
        assert ok, ("row-wise scales", g, n)
        oqT, osT = quant.quant_1x128_tokens(bits)
        got = host(qT[:, r0:r0 + 128])
        ok, n = compare.check_exact(np.ascontiguousarray(got[:, :r1 - r0]), oqT)
        assert ok, ("token codes", g, n)
        assert np.all(got[:, r1 - r0:] == 0), ("padding", g)
        ok, n = compare.check_exact(host(sT[g]), osT[:, 0])
        assert ok, ("token scales", g, n)


def test_token_quantiser_past_65535_token_groups(B, long_tokens):
    import torch
    x, rows = long_tokens
    R, C = x.shape
    Mp = -(-R // 128) * 128
    qT = _filled((C, Mp), torch, torch.uint8, 0x7F)
    say("large token quantiser", R, C)
    qT, sT = B.fp8_quant_1x128(x, transpose_out=True, q=qT)
    ntg = Mp // 128
    for g in sorted({0, 65535, 65536, 65537, ntg - 1}):
        r0, r1 = g * 128, min(R, g * 128 + 128)
        oqT, osT = quant.quant_1x128_tokens(rows(r0, r1))
        got = host(qT[:, r0:r0 + 128])
        ok, n = compare.check_exact(np.ascontiguousarray(got[:, :r1 - r0]), oqT)
        assert ok, ("token codes", g, n)
        assert np.all(got[:, r1 - r0:] == 0), ("padding", g)
        ok, n = compare.check_exact(host(sT[g]), osT[:, 0])
        assert ok, ("token scales", g, n)
