"""Reference forward pass of the decoder layer with blockwise-FP8 linears.  TEST INFRASTRUCTURE.

Pages: arxiv-wiki summary of Puro-2B, section "접근 방법" item (1) (Qwen3-1.7B
architecture); paperlayer.ai summary, appendix C, item "FP8実装pipeline"
(blockwise E4M3 linear GEMMs in a BF16 hidden flow, FP32 softmax).

Plain numpy in float64, with the values rounded to BF16 at the points where the
layer hands BF16 tensors from one operation to the next (every operation's
output).  The linears are the oracle's blockwise-FP8 GEMMs (1x128 activations,
128x128 weights) on those BF16 inputs.  The attention is written out as
softmax(q k^T / sqrt(d) + causal mask) v.  Each stage is a function of its
own, so that a test can hand it the GPU's input to that stage and compare
stage by stage; the chained forward() reproduces no GPU summation order, and
FP8 rounding turns ulp-level differences upstream into whole FP8 steps
downstream, so its output is comparable norm-wise only.
"""

import numpy as np

from . import gemm, quant
from .fused import f64_to_bf16_bits
from .gemm import round_to_bf16

HIDDEN, HEADS, KV_HEADS, HEAD_DIM, INTER = 2048, 16, 8, 128, 6144
EPS, ROPE_THETA = 1e-6, 1e6


def _bf(x):
    return round_to_bf16(x)


def bf16_values(bits):
    """BF16 bit patterns -> float64 values."""
    return quant.bf16_bits_to_f32(bits).astype(np.float64)


def rms_norm(x):
    """x * (mean(x^2) + eps)^-1/2 over the last axis, rounded once to BF16 (unit gain,
    as the layer's norms are initialised)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)
    return _bf(x * r)


def fp8_linear(h, w_bits, budget=False):
    """BF16 values h [M, K] -> (Y [M, N] float64, Bnd) through the blockwise-FP8 forward GEMM:
    h in 1x128 groups, the weight in 128x128 blocks.  Y is not rounded."""
    hq, sh = quant.quant_1x128_rows(f64_to_bf16_bits(h))
    wq, sw = quant.quant_128x128(w_bits)
    return gemm.fwd(hq, sh, wq, sw, budget=budget)


def split_heads(qkv):
    """qkv [s, 4096] -> q [16, s, 128], k [8, s, 128], v [8, s, 128]."""
    s = qkv.shape[0]
    nq, nk = HEADS * HEAD_DIM, KV_HEADS * HEAD_DIM
    q = qkv[:, :nq].reshape(s, HEADS, HEAD_DIM).transpose(1, 0, 2)
    k = qkv[:, nq:nq + nk].reshape(s, KV_HEADS, HEAD_DIM).transpose(1, 0, 2)
    v = qkv[:, nq + nk:].reshape(s, KV_HEADS, HEAD_DIM).transpose(1, 0, 2)
    return q, k, v


def rope(t):
    """t [heads, seq, dim] BF16 values; rotate-half RoPE (theta 1e6) in float64.
    Returns (BF16 result, magnitude |t| + |rotated t| bounding the result)."""
    seq, dim = t.shape[1], t.shape[2]
    inv = 1.0 / (ROPE_THETA ** (np.arange(0, dim, 2) / dim))
    ang = np.arange(seq)[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=-1)
    half = dim // 2
    rot = np.concatenate([-t[..., half:], t[..., :half]], axis=-1)
    return _bf(t * np.cos(ang) + rot * np.sin(ang)), np.abs(t) + np.abs(rot)


def attention(q, k, v):
    """Causal softmax(q k^T / sqrt(128)) v with each key/value head shared by two
    consecutive query heads.  q [16, s, 128], k, v [8, s, 128].  Returns
    (BF16 result [s, 2048], P|v| [s, 2048] bounding it)."""
    s = q.shape[1]
    rep = HEADS // KV_HEADS
    k, v = np.repeat(k, rep, axis=0), np.repeat(v, rep, axis=0)
    sc = q @ k.transpose(0, 2, 1) / np.sqrt(HEAD_DIM)
    sc = np.where(np.tril(np.ones((s, s), dtype=bool))[None], sc, -np.inf)
    p = np.exp(sc - sc.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    merge = lambda t: t.transpose(1, 0, 2).reshape(s, HEADS * HEAD_DIM)
    return merge(_bf(p @ v)), merge(p @ np.abs(v))


def swiglu(gu):
    """gu [s, 12288] BF16 values -> silu(gate) * up rounded once to BF16.

    This is the reading the fused producer follows: the BF16 value handed to
    the down projection's quantiser is the exact product rounded once (the
    pages fix no rounding for the activation).  It is the layer's default
    composition."""
    g, u = gu[:, :INTER], gu[:, INTER:]
    return _bf(g / (1.0 + np.exp(-g)) * u)


def swiglu_separate_ops(gu):
    """gu [s, 12288] BF16 values -> silu(gate) rounded to BF16, times up,
    rounded to BF16 again: the composition of two separate BF16 operations
    (a SiLU, then a multiply), as in the layer variant whose producers are
    not fused.  It differs from swiglu() by at most about one BF16 ulp."""
    gate, up = gu[:, :INTER], gu[:, INTER:]
    return _bf(_bf(gate / (1.0 + np.exp(-gate))) * up)


def forward(x_bits, w_qkv, w_o, w_gu, w_down):
    """x_bits [s, 2048] BF16 (one sequence); weights BF16 bits [N, K] (norm gains 1).
    Returns the layer output as float64 BF16 values."""
    x = bf16_values(x_bits)
    qkv = _bf(fp8_linear(rms_norm(x), w_qkv)[0])
    q, k, v = split_heads(qkv)
    q, k = rope(rms_norm(q))[0], rope(rms_norm(k))[0]
    a = attention(q, k, v)[0]
    x1 = _bf(x + _bf(fp8_linear(a, w_o)[0]))
    act = swiglu(_bf(fp8_linear(rms_norm(x1), w_gu)[0]))
    return _bf(x1 + _bf(fp8_linear(act, w_down)[0]))
