"""Seeded synthetic inputs shaped like the Puro-2B linear layers.

This module only draws random BF16 tensors and describes shapes; it contains
none of the quantisation or GEMM arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it without sharing any of the method.

Shapes (arxiv-wiki Puro-2B summary, section "접근 방법" item (1): a Qwen3-1.7B
style decoder with untied embeddings, sequence length 4096; paperlayer.ai
summary, appendix C: micro-batch 2): hidden 2048, intermediate 6144, 16 query
and 8 key/value heads of width 128, 28 layers.  Per layer the four linears are
    qkv      2048 -> 4096   (16*128 + 2*8*128)
    o        2048 -> 2048
    gate_up  2048 -> 12288  (2 * 6144)
    down     6144 -> 2048
Activations ~ N(0, 1), weights ~ N(0, 0.02), output gradients ~ N(0, 1e-3)
(standard deviations); values are drawn in float32 and rounded to BF16 to
nearest even.
"""

import numpy as np

HIDDEN = 2048
INTER = 6144
LAYERS = 28
# (name, in_features K, out_features N)
LINEARS = (("qkv", 2048, 4096), ("o", 2048, 2048), ("gate_up", 2048, 12288), ("down", 6144, 2048))

BASE_SEED = 0x50902608
_TENSOR_IDS = {"x": 1, "w": 2, "dy": 3}


def seed_for(config, layer, linear, tensor):
    """Deterministic seed per (configuration, layer, linear, tensor)."""
    lin = [n for n, _, _ in LINEARS].index(linear) if isinstance(linear, str) else int(linear)
    return np.random.SeedSequence([BASE_SEED, int(config), int(layer), lin, _TENSOR_IDS[tensor]])


def f32_to_bf16_bits(x):
    """float32 -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def normal_bf16(shape, std, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def with_outlier_channels(x_bits, frac, factor, seed):
    """Multiply round(frac * K) distinct columns by `factor` (a power of two: exact in BF16)."""
    K = x_bits.shape[1]
    n = int(round(frac * K))
    rng = np.random.default_rng(seed)
    cols = np.sort(rng.choice(K, size=n, replace=False))
    e = int(np.log2(factor))
    assert 2 ** e == factor
    out = x_bits.copy()
    sub = out[:, cols].astype(np.uint32)
    expo = (sub >> 7) & 0xFF
    ok = (expo != 0) & (expo + e < 0xFF)
    sub = np.where(ok, sub + (e << 7), sub)          # exponent + e for normal values
    out[:, cols] = sub.astype(np.uint16)
    return out, cols


def student_t_stress(shape, seed, tail_tokens=None):
    """Heavy-tailed activations with zero groups, huge values and one tiny group.

    * Student-t(nu=3) values;
    * about 1% of 128x128-aligned tiles zeroed (zero groups in both the row
      and the token orientation), at least one touching the last token rows;
    * about 1% more row-wise 1x128 groups zeroed;
    * in about 0.1% of row-wise groups one element set to +-U(1e3, 1e5);
    * one row-wise group scaled down so its maximum is below 5e-36 (a binary32
      denormal scale).
    """
    rng = np.random.default_rng(seed)
    M, K = shape
    x = rng.standard_t(3.0, size=shape).astype(np.float32)
    tm, tk = -(-M // 128), K // 128
    tiles = rng.random((tm, tk)) < 0.01
    tiles[tm - 1, rng.integers(tk)] = True            # a zero tile in the ragged tail
    for a, b in zip(*np.nonzero(tiles)):
        x[a * 128:(a + 1) * 128, b * 128:(b + 1) * 128] = 0.0
    groups = rng.random((M, tk)) < 0.01
    for r, g in zip(*np.nonzero(groups)):
        x[r, g * 128:(g + 1) * 128] = 0.0
    big = rng.random((M, tk)) < 0.001
    for r, g in zip(*np.nonzero(big)):
        x[r, g * 128 + rng.integers(128)] = rng.choice([-1.0, 1.0]) * rng.uniform(1e3, 1e5)
    r, g = int(rng.integers(M)), int(rng.integers(tk))
    x[r, g * 128:(g + 1) * 128] = rng.standard_normal(128).astype(np.float32) * np.float32(1e-37)
    x[r, g * 128] = np.float32(3e-36)
    return f32_to_bf16_bits(x)


def layer_tensors(config, layer, linear, M, outliers=False):
    """(X, W, dY) BF16 bit arrays of one linear of one layer at M tokens.

    X [M, K] ~ N(0, 1), W [N, K] ~ N(0, 0.02), dY [M, N] ~ N(0, 1e-3), each from
    its own seed.  outliers=True (the 8192-token sweep) scales round(1% of K)
    input channels of X by 32 (exact in BF16)."""
    _, k, n = [l for l in LINEARS if l[0] == linear][0]
    sx = seed_for(config, layer, linear, "x")
    x = normal_bf16((M, k), 1.0, sx)
    if outliers:
        x, _ = with_outlier_channels(x, 0.01, 32, sx.spawn(1)[0])
    w = normal_bf16((n, k), 0.02, seed_for(config, layer, linear, "w"))
    dy = normal_bf16((M, n), 1e-3, seed_for(config, layer, linear, "dy"))
    return x, w, dy


def layer_shapes(M):
    """[(name, X shape, W shape, dY shape)] of one decoder layer at M tokens."""
    return [(n, (M, k), (nout, k), (M, nout)) for n, k, nout in LINEARS]


def gemm_flops_per_layer(M):
    """2*M*N*K summed over the forward, dgrad and wgrad GEMMs of one layer."""
    return 3 * sum(2 * M * n * k for _, k, n in LINEARS)
