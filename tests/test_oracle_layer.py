"""Pins for the decoder-layer reference (oracle/layer.py), CPU only.

Closed forms and special cases that a wiring slip would break:
* RoPE: identity at position 0; at position p the pair (i, i+64) turns by
  p * 1e6^(-i/64) radians (checked against math.cos/sin at p = 1, 3);
* attention: the first query sees only the first key (its output is that
  value row); equal keys give the running mean of the values; query heads
  2h and 2h+1 read key/value head h (a distinct value per head shows it);
  scores are scaled by 1/sqrt(128): scores 0 and sqrt(128) ln 3 give the
  weights 1/4 and 3/4 exactly;
* RMSNorm of a constant row is +-1; silu(gate) (up = 1) equals the pinned
  fused reference; the two SwiGLU compositions (the product rounded once, as
  the fused producer forms it, and silu rounded before the multiply, as two
  separate BF16 operations do) each equal a 60-digit evaluation rounded to the
  nearest BF16 at the same points;
* the whole layer with zero output projections is the identity (residuals),
  and with a zero down projection it is x + o(attention) alone.
"""

import math
from decimal import Decimal, getcontext

import numpy as np

from oracle import fused, gemm
from oracle import layer as L


def bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_rope_position_zero_and_rotation_angle():
    rng = np.random.default_rng(1)
    t = gemm.round_to_bf16(rng.standard_normal((1, 4, 128)))
    out, _ = L.rope(t)
    assert np.array_equal(out[0, 0], t[0, 0])
    for p in (1, 3):
        for i in (0, 5, 63):
            ang = p * L.ROPE_THETA ** (-i / 64)
            a, b = t[0, p, i], t[0, p, i + 64]
            want_a = a * math.cos(ang) - b * math.sin(ang)
            want_b = b * math.cos(ang) + a * math.sin(ang)
            assert out[0, p, i] == gemm.round_to_bf16(want_a)
            assert out[0, p, i + 64] == gemm.round_to_bf16(want_b)


def test_attention_first_query_and_equal_keys():
    rng = np.random.default_rng(2)
    s = 6
    q = rng.standard_normal((16, s, 128))
    k = np.ones((8, s, 128))
    v = gemm.round_to_bf16(rng.standard_normal((8, s, 128)))
    out, _ = L.attention(q, k, v)
    out = out.reshape(s, 16, 128)
    for h in range(16):
        assert np.array_equal(out[0, h], v[h // 2, 0])
        for i in range(s):
            np.testing.assert_allclose(out[i, h], gemm.round_to_bf16(v[h // 2, :i + 1].mean(axis=0)),
                                       rtol=2.0 ** -7, atol=1e-12)


def test_attention_head_sharing():
    s = 3
    q = np.zeros((16, s, 128))
    k = np.zeros((8, s, 128))
    v = np.zeros((8, s, 128))
    for h in range(8):
        v[h, :, :] = h + 1.0
    out, _ = L.attention(q, k, v)
    out = out.reshape(s, 16, 128)
    for h in range(16):
        assert np.all(out[:, h] == h // 2 + 1.0)


def test_attention_softmax_temperature_closed_form():
    # Query 1 sees keys 0 and 1 with q.k = 0 and sqrt(128) ln 3: after the
    # 1/sqrt(128) scaling the softmax weights are 1/4 and 3/4, so values 4 and
    # 8 average to 7 (exact in BF16), and P|v| is 7 as well.
    s = 2
    q = np.zeros((16, s, 128))
    k = np.zeros((8, s, 128))
    v = np.zeros((8, s, 128))
    q[:, 1, 0] = 1.0
    k[:, 1, 0] = math.sqrt(128.0) * math.log(3.0)
    v[:, 0, :], v[:, 1, :] = 4.0, 8.0
    out, mag = L.attention(q, k, v)
    out, mag = out.reshape(s, 16, 128), mag.reshape(s, 16, 128)
    np.testing.assert_allclose(out[1], 7.0, rtol=2.0 ** -8)
    np.testing.assert_allclose(mag[1], 7.0, rtol=1e-12)
    assert np.all(out[0] == 4.0)


def test_rms_norm_constant_rows_and_swiglu():
    x = np.array([[3.0] * 64, [-0.25] * 64])
    y = L.rms_norm(x)
    assert np.allclose(y[0], 1.0, atol=2.0 ** -8) and np.allclose(y[1], -1.0, atol=2.0 ** -8)
    rng = np.random.default_rng(4)
    g = bf16_bits(rng.standard_normal((2, L.INTER)).astype(np.float32))
    one = bf16_bits(np.ones((2, L.INTER), dtype=np.float32))
    gu = np.concatenate([L.bf16_values(g), L.bf16_values(one)], axis=1)
    silu = L.swiglu(gu)           # up = 1: silu(gate) rounded once
    assert np.array_equal(silu, L.bf16_values(fused.swiglu_bf16(g, one)))
    assert np.array_equal(L.swiglu_separate_ops(gu), silu)   # with up = 1 the second rounding is exact
    u = bf16_bits(rng.standard_normal((2, L.INTER)).astype(np.float32))
    gu = np.concatenate([L.bf16_values(g), L.bf16_values(u)], axis=1)
    assert np.array_equal(L.swiglu_separate_ops(gu), gemm.round_to_bf16(silu * L.bf16_values(u)))


def _dec(v):
    return Decimal(float(v))


def _nearest_bf16_value(d):
    """Exact nearest BF16 value (ties to even) to the Decimal d, as a float."""
    if d == 0:
        return 0.0
    b0 = int((np.asarray([float(d)], dtype=np.float32).view(np.uint32) >> 16)[0])
    val = lambda b: Decimal(float(np.uint32(b << 16).view(np.float32)))
    return float(val(min((b0 - 1, b0, b0 + 1), key=lambda b: (abs(val(b) - d), b & 1))))


def test_swiglu_compositions_against_high_precision():
    """Both SwiGLU compositions against a 60-digit evaluation with exact nearest-BF16
    rounding: swiglu() rounds silu(g) * u once, swiglu_separate_ops() rounds silu(g)
    first and the product again; on these inputs the two differ somewhere."""
    getcontext().prec = 60
    rng = np.random.default_rng(9)
    n = 48
    g = L.bf16_values(bf16_bits(rng.standard_normal((1, n)).astype(np.float32) * 3))
    u = L.bf16_values(bf16_bits(rng.standard_normal((1, n)).astype(np.float32)))
    inter = L.INTER
    gu = np.zeros((1, 2 * inter))
    gu[0, :n], gu[0, inter:inter + n] = g[0], u[0]
    once, twice = L.swiglu(gu)[0, :n], L.swiglu_separate_ops(gu)[0, :n]
    for i in range(n):
        gd, ud = _dec(g[0, i]), _dec(u[0, i])
        silu = gd / (1 + (-gd).exp())
        assert once[i] == _nearest_bf16_value(silu * ud), i
        assert twice[i] == _nearest_bf16_value(_dec(_nearest_bf16_value(silu)) * ud), i
    assert (once != twice).any()


def _weights(rng, zero=()):
    shapes = [(4096, 2048), (2048, 2048), (12288, 2048), (2048, 6144)]
    out = []
    for i, sh in enumerate(shapes):
        w = np.zeros(sh, dtype=np.float32) if i in zero else rng.standard_normal(sh).astype(np.float32) * 0.02
        out.append(bf16_bits(w))
    return out


def test_forward_residual_paths():
    rng = np.random.default_rng(5)
    x = bf16_bits(rng.standard_normal((8, 2048)).astype(np.float32) * 0.5)
    xv = L.bf16_values(x)
    w = _weights(rng, zero=(1, 3))
    assert np.array_equal(L.forward(x, *w), xv)
    w = _weights(rng, zero=(3,))
    qkv = gemm.round_to_bf16(L.fp8_linear(L.rms_norm(xv), w[0])[0])
    q, k, v = L.split_heads(qkv)
    a = L.attention(L.rope(L.rms_norm(q))[0], L.rope(L.rms_norm(k))[0], v)[0]
    want = gemm.round_to_bf16(xv + gemm.round_to_bf16(L.fp8_linear(a, w[1])[0]))
    assert np.array_equal(L.forward(x, *w), want)
