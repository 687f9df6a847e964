"""Blockwise-FP8 linear layer (forward, data gradient, weight gradient).

Pages: paperlayer.ai summary of arXiv 2608.27370v1, appendix C "生産学習の詳細",
item "FP8実装pipeline" -- a linear layer's forward, data-gradient and
weight-gradient GEMMs run on blockwise E4M3 operands while the hidden flow is
BF16 and gradients and optimizer state stay FP32; arxiv-wiki summary, section
"접근 방법" item (4) -- 1x128 activation groups, 128x128 weight blocks, BF16/FP32
master weights.

The module is a thin autograd wrapper over the C ABI (every step runs in the
library's kernels):

* forward:  X (BF16) is quantised once into both 1x128 orientations
  (fp8_quant_1x128_dual); Y = Xq . Wq^T (BF16).  Only the token-dimension FP8
  copy of X (XqT, 1 byte per element plus scales) is kept for the backward
  pass instead of the BF16 activation.
* backward: dY is quantised once into both orientations; dX = dYq . WqT
  (BF16) and dW += dYqT . XqT (FP32, accumulated into ``weight.main_grad``
  across micro-batches, the FP32 gradient the optimizer reads).
* the FP8 weight, its transposed copy and their block scales are made once per
  weight value and reused by every micro-batch until the weight changes.  The
  cache is keyed on the parameter's in-place version counter and storage, so
  in-place updates through the parameter itself (an optimizer's ``p.add_``,
  ``p.copy_`` under ``no_grad``) rebuild it.  Writes that bypass the counter --
  through ``weight.data`` or another tensor aliasing the same storage, as a
  master-to-model weight copy often does -- are not seen: call
  ``Fp8Linear.invalidate_weight_cache()`` after them.

Two fused entry points put the producer of the linear's input into its
quantiser: ``forward_rmsnorm`` (RMSNorm, for the qkv and gate_up projections)
and ``forward_swiglu`` (SwiGLU, for the down projection).  Their backward
passes run the producer's backward with PyTorch's kernels from the saved inputs.

The three GEMMs form each 128-wide block product exactly by default; with
``fp8_matrix_core=True`` they use the FP8 matrix instructions instead (about
1.4 times the GEMM rate; the hardware truncates small products inside groups
of 8 positions, an error up to about 2^-10 of the block's sum of |a*b|).
"""

import torch
import torch.nn.functional as F

from . import binding as B


class _WeightCache:
    """Wq, Sw, WqT, SwT of one BF16 weight, rebuilt when the weight changes."""

    def __init__(self):
        self.version = None
        self.ptr = None
        self.tensors = None
        self.builds = 0

    def invalidate(self):
        """Force a rebuild on the next use (after writes the version counter misses)."""
        self.version = self.ptr = None

    def get(self, w):
        key = (w._version, w.data_ptr())
        if self.tensors is None or key != (self.version, self.ptr):
            q, s, qT, sT = self._reuse(w)
            self.tensors = B.fp8_quant_128x128(w.detach(), True, q, s, qT, sT)
            self.version, self.ptr = key
            self.builds += 1
        return self.tensors

    def _reuse(self, w):
        # Reuse the previous buffers when the shape is unchanged.
        if self.tensors is not None and self.tensors[0].shape == w.shape:
            return self.tensors
        return (None, None, None, None)


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, cache, mc):
        wq, sw, wqT, swT = cache.get(weight)
        xq, sx, xqT, sxT = B.fp8_quant_1x128_dual(x)
        y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, fp8_matrix_core=mc)
        ctx.save_for_backward(xqT, sxT)
        ctx.cache, ctx.weight, ctx.M, ctx.mc = cache, weight, x.shape[0], mc
        return y

    @staticmethod
    def backward(ctx, dy):
        xqT, sxT = ctx.saved_tensors
        return _linear_backward(ctx.cache, ctx.weight, xqT, sxT, ctx.M, ctx.mc, dy), None, None, None


def _linear_backward(cache, weight, xqT, sxT, M, mc, dy):
    """dY -> dX (BF16), accumulating dW into weight.main_grad (FP32)."""
    _, _, wqT, swT = cache.get(weight)
    dy = dy.contiguous()
    dyq, sdy, dyqT, sdyT = B.fp8_quant_1x128_dual(dy)
    dx = B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, fp8_matrix_core=mc)
    if getattr(weight, "main_grad", None) is None:
        weight.main_grad = torch.zeros(weight.shape, dtype=torch.float32, device=weight.device)
    B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=weight.main_grad, accumulate=True, fp8_matrix_core=mc)
    return dx


class _Fp8RMSNormLinearFn(torch.autograd.Function):
    """y = RMSNorm(x; gamma, eps) . W^T with the normalisation fused into the
    quantiser: the BF16 normalised value exists only in registers (or in the
    optional h_out).  Backward: the linear's dgrad gives dL/dh, then PyTorch's
    fused RMSNorm backward from x, gamma and the saved 1/rms."""

    @staticmethod
    def forward(ctx, x, gamma, weight, cache, mc, eps, h_out):
        wq, sw, _, _ = cache.get(weight)
        xq, sx, xqT, sxT, rstd = B.fp8_rmsnorm_quant_1x128_dual(x, gamma, eps, y_out=h_out)
        y = B.fp8_block_gemm_fwd(xq, sx, wq, sw, fp8_matrix_core=mc)
        ctx.save_for_backward(x, gamma, rstd, xqT, sxT)
        ctx.cache, ctx.weight, ctx.M, ctx.mc = cache, weight, x.shape[0], mc
        return y

    @staticmethod
    def backward(ctx, dy):
        x, gamma, rstd, xqT, sxT = ctx.saved_tensors
        dh = _linear_backward(ctx.cache, ctx.weight, xqT, sxT, ctx.M, ctx.mc, dy)
        # The producer's backward: PyTorch's fused RMSNorm backward with the
        # 1/rms the forward kernel wrote ([rows, 1] FP32, as PyTorch keeps it).
        dx, dgamma = torch.ops.aten._fused_rms_norm_backward(dh, x, [x.shape[1]], rstd.view(-1, 1), gamma,
                                                             [True, True])
        return dx, dgamma, None, None, None, None, None


class _Fp8SwiGLULinearFn(torch.autograd.Function):
    """y = (silu(gate) * up) . W^T for gu = [gate | up] with the activation
    fused into the quantiser.  Backward: the linear's dgrad gives dL/d(act),
    then PyTorch's SwiGLU backward from the saved gate and up."""

    @staticmethod
    def forward(ctx, gu, weight, cache, mc, h_out):
        wq, sw, _, _ = cache.get(weight)
        half = gu.shape[1] // 2
        gate, up = gu[:, :half], gu[:, half:]
        aq, sa, aqT, saT = B.fp8_swiglu_quant_1x128_dual(gate, up, h_out=h_out)
        y = B.fp8_block_gemm_fwd(aq, sa, wq, sw, fp8_matrix_core=mc)
        ctx.save_for_backward(gu, aqT, saT)
        ctx.cache, ctx.weight, ctx.M, ctx.mc = cache, weight, gu.shape[0], mc
        return y

    @staticmethod
    def backward(ctx, dy):
        gu, aqT, saT = ctx.saved_tensors
        da = _linear_backward(ctx.cache, ctx.weight, aqT, saT, ctx.M, ctx.mc, dy)
        # The producer's backward with PyTorch's SiLU kernels, written straight
        # into the two halves of d[gate | up].
        half = gu.shape[1] // 2
        gate, up = gu[:, :half], gu[:, half:]
        dgu = torch.empty_like(gu)
        torch.ops.aten.silu_backward.grad_input(da * up, gate, grad_input=dgu[:, :half])
        torch.mul(da, F.silu(gate), out=dgu[:, half:])
        return dgu, None, None, None, None


class Fp8Linear(torch.nn.Module):
    """y = x . W^T with blockwise-FP8 GEMMs; no bias (the decoder's linears have none).

    ``weight`` is a BF16 parameter [out_features, in_features]; both sizes
    must be multiples of 128.  Its gradient is accumulated in FP32 into
    ``weight.main_grad`` (zero it between optimizer steps); ``weight.grad`` is
    left untouched.  Inputs are [..., in_features] BF16 tensors.
    ``fp8_matrix_core`` selects the FP8 matrix-instruction GEMMs (see above).
    """

    def __init__(self, in_features, out_features, device="cuda", weight=None, fp8_matrix_core=False):
        super().__init__()
        if in_features % 128 or out_features % 128:
            raise ValueError("in_features and out_features must be multiples of 128")
        if weight is None:
            weight = torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        self.weight = torch.nn.Parameter(weight)
        self.in_features, self.out_features = in_features, out_features
        self._cache = _WeightCache()
        self.fp8_matrix_core = bool(fp8_matrix_core)

    def invalidate_weight_cache(self):
        """Requantise the weight on the next forward.  Needed after writes that do
        not bump the parameter's version counter, e.g. ``weight.data.copy_(w)``
        or a copy into a tensor that aliases the weight's storage; in-place
        operations on the parameter itself are detected without it."""
        self._cache.invalidate()

    @property
    def weight_quantisations(self):
        """How many times the FP8 weight has been (re)built."""
        return self._cache.builds

    def forward(self, x, rmsnorm=None, swiglu=False, h_out=None):
        """y = x . W^T for x [..., in_features] BF16.

        rmsnorm=(gamma, eps): y = (RMSNorm(x) * gamma) . W^T with the
        normalisation fused into the quantiser (gamma BF16 [in_features]).
        swiglu=True: x = [gate | up] (2 * in_features wide) and
        y = (silu(gate) * up) . W^T with the activation fused likewise.
        h_out: optional BF16 [rows, in_features] receiving the fused producer's value.
        """
        shape = x.shape
        if rmsnorm is not None:
            gamma, eps = rmsnorm
            y = _Fp8RMSNormLinearFn.apply(_rows(x, self.in_features), gamma, self.weight, self._cache,
                                          self.fp8_matrix_core, float(eps), h_out)
        elif swiglu:
            y = _Fp8SwiGLULinearFn.apply(_rows(x, 2 * self.in_features), self.weight, self._cache,
                                         self.fp8_matrix_core, h_out)
        else:
            y = _Fp8LinearFn.apply(_rows(x, self.in_features), self.weight, self._cache, self.fp8_matrix_core)
        return y.reshape(*shape[:-1], self.out_features)

    def forward_rmsnorm(self, x, gamma, eps, h_out=None):
        """self(RMSNorm(x) * gamma), the normalisation fused into the quantiser."""
        return self(x, rmsnorm=(gamma, eps), h_out=h_out)

    def forward_swiglu(self, gu, h_out=None):
        """self(silu(gate) * up) for gu = [gate | up], the activation fused into the quantiser."""
        return self(gu, swiglu=True, h_out=h_out)


def _rows(x, cols):
    """x as a 2-D [rows, cols] BF16 view with unit column stride and 16-byte aligned rows."""
    if x.dim() < 1 or x.shape[-1] != cols:
        raise ValueError(f"input must be [..., {cols}], got {list(x.shape)}")
    x2 = x.reshape(-1, cols)
    if x2.stride(1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    return x2
