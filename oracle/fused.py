"""Producers fused into the 1x128 quantisers: SwiGLU and RMSNorm.  TEST INFRASTRUCTURE.

Pages: paperlayer.ai summary of arXiv 2608.27370v1, appendix C "生産学習の詳細",
item "FP8実装pipeline" -- the hidden flow and the normalisation run in BF16
ahead of the FP8 linear GEMMs; arxiv-wiki summary, section "접근 방법" item (1)
-- the model follows the Qwen3-1.7B architecture (RMSNorm before the attention
and MLP blocks, a SwiGLU MLP).

The pages fix neither the arithmetic of these producers nor their rounding.
Reading used here (the plain one): the BF16 value a producer hands to the
quantiser is the exact real result rounded once to BF16 (nearest, ties to
even):

    SwiGLU   h = RNE_bf16( g * u / (1 + exp(-g)) )
    RMSNorm  rstd = 1 / sqrt(mean_c x[r, c]^2 + eps),  y = RNE_bf16( x * rstd * gamma )

evaluated here in float64 (whose error is far below a BF16 half-ulp except at
exact ties, which the tests tolerate as one ulp).  The quantisation of the
result is the oracle's 1x128 quantiser, unchanged.
"""

import numpy as np

from .gemm import round_to_bf16
from .quant import bf16_bits_to_f32


def f64_to_bf16_bits(values):
    """float64 values already on the BF16 grid (or +-inf) -> BF16 bit patterns."""
    return (np.asarray(values, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def swiglu_bf16(g_bits, u_bits):
    """BF16 bits of silu(g) * u for BF16 bit arrays g, u of one shape."""
    g = bf16_bits_to_f32(g_bits).astype(np.float64)
    u = bf16_bits_to_f32(u_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return f64_to_bf16_bits(round_to_bf16(h))


def rmsnorm_bf16(x_bits, gamma_bits, eps):
    """(BF16 bits of y, rstd float64 [rows]) for x [rows, cols], gamma [cols]."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    gamma = bf16_bits_to_f32(np.asarray(gamma_bits)).astype(np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(np.float32(eps)))
    y = x * rstd[:, None] * gamma[None, :]
    return f64_to_bf16_bits(round_to_bf16(y)), rstd
