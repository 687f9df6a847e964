"""The decoder layer with FP8 linears, stage by stage against the float64 reference.

Each stage of the GPU layer is compared with the reference stage applied to
the GPU's own input to that stage (the tensors the layer records in its trace):
* the four FP8 linears: the GEMM acceptance rule (one BF16 ulp, or the FP32
  error budget under cancellation), every element;
* RMSNorms, residual adds: within one BF16 ulp;
* head norm + RoPE: within two BF16 ulps of the terms' magnitude (PyTorch
  evaluates them in binary32 with its own exp/sin/cos);
* SwiGLU: the fused producer's value within one BF16 ulp of silu(g) * u
  rounded once; the separate PyTorch operations' value within one ulp of
  silu(g) rounded to BF16, times |u|, plus one ulp of the product rounded
  again (the two compositions round differently);
* attention (PyTorch's fused kernel): within 2^-6 of P|v| plus one ulp, and
  below 1% norm-wise.
The chained output is then compared norm-wise only: FP8 rounding turns a
one-ulp difference upstream into a whole FP8 step downstream (on the CPU, one
BF16 ulp added to 10% of the layer's input moves the reference output by 4%
norm-wise), so the bound is 8%; wiring mistakes (a swapped split, a wrong
key/value head, a missing mask) are off by order one.
The same stage checks run with the producers (RMSNorm, SwiGLU) as separate
PyTorch operations and fused into the linears' quantisers (the default), and
with the FP8 matrix-instruction linears, whose GEMMs are held to the derived
bound (2^-10 + 1e-5) * sum |a*b| instead.
The backward pass is checked against the same layer with BF16 nn.Linear
weights: finite gradients and cosine similarity above 0.99 for the input
gradient, every weight gradient (the FP8 linears' main_grad) and the two
RMSNorm gains.
"""

import numpy as np
import pytest

from oracle import compare
from oracle import layer as ref
from tests.gpu_util import host, say

pytestmark = pytest.mark.gpu


def _vals(t):
    """BF16 device tensor -> float64 values (any layout)."""
    return ref.bf16_values(host(t.contiguous()))


def _within(got, want, bound, label):
    err = np.abs(got - want)
    bad = ~(err <= bound)
    assert not bad.any(), (label, int(bad.sum()), float(err.max()))


def _cos(a, b):
    a, b = a.double().flatten(), b.double().flatten()
    return float((a @ b) / (a.norm() * b.norm()))


@pytest.fixture(scope="module")
def run():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from blockwise_fp8_linear_quant_amd.layer import DecoderLayer
    s = 256
    g = torch.Generator().manual_seed(11)
    x0 = (torch.randn((1, s, 2048), generator=g) * 0.5).to(torch.bfloat16).cuda()
    out = {}
    for kind in ("fp8", "fp8_unfused", "fp8_matrix_core", "bf16"):
        if kind == "fp8_unfused":
            lay = DecoderLayer(linears="fp8", seed=3, fused=False)
        else:
            lay = DecoderLayer(linears=kind, seed=3)
        x = x0.clone().requires_grad_(True)
        tr = {}
        say("decoder layer forward", kind, s)
        y = lay(x, trace=tr)
        say("decoder layer backward", kind, s)
        y.float().pow(2).mean().backward()
        torch.cuda.synchronize()
        grads = [l.weight.grad if kind == "bf16" else l.weight.main_grad for l in lay.linears()]
        norms = [lay.norm1.grad, lay.norm2.grad]
        out[kind] = dict(lay=lay, x=x, y=y.detach(), trace=tr, dx=x.grad, grads=grads, norms=norms)
    return out


FP8_PATH_RTOL = 2.0 ** -10 + 1e-5


@pytest.mark.parametrize("kind,rtol", [("fp8", compare.FP32_RTOL), ("fp8_unfused", compare.FP32_RTOL),
                                       ("fp8_matrix_core", FP8_PATH_RTOL)])
def test_layer_stages(run, kind, rtol):
    r = run[kind]
    tr, lay = r["trace"], r["lay"]
    x = _vals(r["x"].detach()[0])
    w = [host(l.weight.detach()) for l in lay.linears()]
    T = {k: _vals(v[0]) for k, v in tr.items()}
    ulp = compare.bf16_ulp

    _within(T["h"], ref.rms_norm(x), ulp(T["h"]), "rmsnorm 1")
    for name, inp, wi in (("qkv", "h", 0), ("o", "a", 1), ("gu", "h2", 2), ("down", "act", 3)):
        y, bnd = ref.fp8_linear(T[inp], w[wi], budget=True)
        ok, rep = compare.check_bf16(host(tr[name][0].contiguous()), y, bnd, rtol=rtol)
        assert ok, (name, rep)

    q, k, v = ref.split_heads(T["qkv"])
    for name, t in (("q", q), ("k", k)):
        want, mag = ref.rope(ref.rms_norm(t))
        _within(T[name], want, 2 * ulp(mag), "head norm + rope " + name)

    want, mag = ref.attention(T["q"], T["k"], v)
    a = T["a"].reshape(-1, 2048)
    _within(a, want, 2.0 ** -6 * mag + ulp(want), "attention")
    rel = np.linalg.norm(a - want) / np.linalg.norm(want)
    assert rel < 1e-2, ("attention norm-wise", rel)

    _within(T["x1"], ref.round_to_bf16(x + T["o"]), ulp(T["x1"]), "residual 1")
    _within(T["h2"], ref.rms_norm(T["x1"]), ulp(T["h2"]), "rmsnorm 2")
    g, u = T["gu"][:, :ref.INTER], T["gu"][:, ref.INTER:]
    if kind == "fp8_unfused":
        # Separate PyTorch operations: silu(g) rounded to BF16, then the product rounded again.
        want = ref.swiglu_separate_ops(T["gu"])
        silu = np.abs(g / (1.0 + np.exp(-g)))
        _within(T["act"], want, ulp(silu) * np.abs(u) + ulp(want), "swiglu (separate ops)")
    else:
        # Fused producer: the product rounded once, as the oracle's fused reading.
        want = ref.swiglu(T["gu"])
        _within(T["act"], want, ulp(np.maximum(np.abs(want), np.abs(T["act"]))), "swiglu (fused)")
    yv = _vals(r["y"][0])
    _within(yv, ref.round_to_bf16(T["x1"] + T["down"]), ulp(yv), "residual 2")


def test_layer_chained_output(run):
    r = run["fp8"]
    x = host(r["x"].detach()[0])
    w = [host(l.weight.detach()) for l in r["lay"].linears()]
    want = ref.forward(x, *w)
    got = _vals(r["y"][0])
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 8e-2, rel


@pytest.mark.parametrize("kind", ["fp8", "fp8_unfused", "fp8_matrix_core"])
def test_layer_backward_against_bf16_layer(run, kind):
    import torch
    f, b = run[kind], run["bf16"]
    assert torch.isfinite(f["dx"]).all()
    c = _cos(f["dx"], b["dx"])
    assert c > 0.99, ("dx", c)
    for i, (gf, gb) in enumerate(zip(f["grads"], b["grads"])):
        assert gf.dtype == torch.float32 and torch.isfinite(gf).all()
        c = _cos(gf, gb)
        assert c > 0.99, (i, c)
    for i, (nf, nb) in enumerate(zip(f["norms"], b["norms"])):   # RMSNorm gains
        assert nf is not None and torch.isfinite(nf).all()
        c = _cos(nf, nb)
        assert c > 0.99, ("norm", i, c)
