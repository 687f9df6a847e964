"""A whole decoder layer with blockwise-FP8 linears, for measuring their share.

Pages: arxiv-wiki summary of Puro-2B, section "접근 방법" item (1) -- the model
is a Qwen3-1.7B-style decoder (hidden 2048, untied embeddings, sequence length
4096); paperlayer.ai summary, appendix C, item "FP8実装pipeline" -- the linear
layers' GEMMs run in blockwise FP8, the hidden flow, normalisation and
embeddings in BF16, softmax in FP32; ailog.hnlab.kr post -- FP8 covers about
72% of the training compute.

Layer (Qwen3 layout, 16 query heads and 8 key/value heads of 128):
    h  = RMSNorm(x)                    q, k, v = split(qkv(h))
    q, k = RMSNorm_head(q), RMSNorm_head(k);  RoPE(q, k)
    a  = causal attention(q, k, v)     x1 = x + o(a)
    h2 = RMSNorm(x1)                   g, u = split(gate_up(h2))
    y  = x1 + down(silu(g) * u)

The four linears are Fp8Linear (this library; exact block products, or the
FP8 matrix instructions with linears="fp8_matrix_core") or, for comparison,
BF16 nn.Linear (linears="bf16").  With FP8 linears the two RMSNorms and the
SwiGLU are by default fused into the quantiser of the linear they feed
(fused=False keeps them as separate PyTorch operations).  Attention is PyTorch's scaled_dot_product_attention in BF16 (its
softmax accumulates in FP32); the other element-wise steps are PyTorch BF16
operations.  Only the linears are the subject of this library.
"""

import torch
import torch.nn.functional as F

from .linear import Fp8Linear

HIDDEN, HEADS, KV_HEADS, HEAD_DIM, INTER = 2048, 16, 8, 128, 6144
EPS, ROPE_THETA = 1e-6, 1e6


def rope_tables(seq, device, dim=HEAD_DIM, theta=ROPE_THETA):
    """cos, sin [seq, dim] (the rotate-half form) in float32."""
    inv = 1.0 / (theta ** (torch.arange(0, dim, 2, dtype=torch.float64, device=device) / dim))
    ang = torch.arange(seq, dtype=torch.float64, device=device)[:, None] * inv[None, :]
    ang = torch.cat([ang, ang], dim=-1)
    return ang.cos().float(), ang.sin().float()


def apply_rope(t, cos, sin):
    """t [b, heads, seq, dim] BF16; rotation in float32, result BF16."""
    tf = t.float()
    half = tf.shape[-1] // 2
    rot = torch.cat([-tf[..., half:], tf[..., :half]], dim=-1)
    return (tf * cos + rot * sin).to(t.dtype)


class DecoderLayer(torch.nn.Module):
    def __init__(self, linears="fp8", device="cuda", seed=0, fused=True):
        super().__init__()
        if linears not in ("fp8", "fp8_matrix_core", "bf16"):
            raise ValueError(f"linears must be 'fp8', 'fp8_matrix_core' or 'bf16', not {linears!r}")
        fp8 = linears != "bf16"
        g = torch.Generator(device="cpu").manual_seed(seed)

        def weight(n, k):
            return (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16).to(device)

        def linear(k, n):
            w = weight(n, k)
            if fp8:
                return Fp8Linear(k, n, weight=w, fp8_matrix_core=(linears == "fp8_matrix_core"))
            lin = torch.nn.Linear(k, n, bias=False, device=device, dtype=torch.bfloat16)
            with torch.no_grad():
                lin.weight.copy_(w)
            return lin

        self.fp8 = fp8
        self.fused = fused
        self.qkv = linear(HIDDEN, (HEADS + 2 * KV_HEADS) * HEAD_DIM)
        self.o = linear(HEADS * HEAD_DIM, HIDDEN)
        self.gate_up = linear(HIDDEN, 2 * INTER)
        self.down = linear(INTER, HIDDEN)
        ones = lambda n: torch.nn.Parameter(torch.ones(n, dtype=torch.bfloat16, device=device))
        self.norm1, self.norm2 = ones(HIDDEN), ones(HIDDEN)
        self.q_norm, self.k_norm = ones(HEAD_DIM), ones(HEAD_DIM)
        self._rope = {}

    def linears(self):
        return [self.qkv, self.o, self.gate_up, self.down]

    def forward(self, x, trace=None):
        """x [b, s, 2048] BF16 -> [b, s, 2048] BF16.  trace: optional dict that
        receives the intermediate tensors (detached) under the names used above.

        With FP8 linears and fused=True the two RMSNorms and the SwiGLU are
        formed inside the following linear's quantiser (their BF16 values are
        written out only when a trace is asked for)."""
        def keep(name, t):
            if trace is not None:
                trace[name] = t.detach()
            return t

        def bf16_out(cols):
            return None if trace is None else torch.empty((b * s, cols), dtype=torch.bfloat16, device=x.device)

        b, s, _ = x.shape
        if s not in self._rope:
            self._rope[s] = rope_tables(s, x.device)
        cos, sin = self._rope[s]
        fused = self.fp8 and self.fused
        if fused:
            h = bf16_out(HIDDEN)
            qkv = self.qkv.forward_rmsnorm(x, self.norm1, EPS, h_out=h)
            if trace is not None:
                keep("h", h.view(b, s, HIDDEN))
        else:
            qkv = self.qkv(keep("h", F.rms_norm(x, (HIDDEN,), self.norm1, EPS)))
        keep("qkv", qkv)
        q, k, v = qkv.split([HEADS * HEAD_DIM, KV_HEADS * HEAD_DIM, KV_HEADS * HEAD_DIM], dim=-1)
        q = F.rms_norm(q.reshape(b, s, HEADS, HEAD_DIM), (HEAD_DIM,), self.q_norm, EPS).transpose(1, 2)
        k = F.rms_norm(k.reshape(b, s, KV_HEADS, HEAD_DIM), (HEAD_DIM,), self.k_norm, EPS).transpose(1, 2)
        v = v.reshape(b, s, KV_HEADS, HEAD_DIM).transpose(1, 2)
        q, k = keep("q", apply_rope(q, cos, sin)), keep("k", apply_rope(k, cos, sin))
        a = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
        a = keep("a", a.transpose(1, 2).reshape(b, s, HEADS * HEAD_DIM))
        x1 = keep("x1", x + keep("o", self.o(a)))
        if fused:
            h2 = bf16_out(HIDDEN)
            gu = keep("gu", self.gate_up.forward_rmsnorm(x1, self.norm2, EPS, h_out=h2))
            act = bf16_out(INTER)
            down = self.down.forward_swiglu(gu, h_out=act)
            if trace is not None:
                keep("h2", h2.view(b, s, HIDDEN))
                keep("act", act.view(b, s, INTER))
        else:
            h2 = keep("h2", F.rms_norm(x1, (HIDDEN,), self.norm2, EPS))
            gu = keep("gu", self.gate_up(h2))
            gate, up = gu.split([INTER, INTER], dim=-1)
            down = self.down(keep("act", F.silu(gate) * up))
        return x1 + keep("down", down)
