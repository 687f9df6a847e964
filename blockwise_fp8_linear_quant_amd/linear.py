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
  weight value and reused by every micro-batch until the weight changes (the
  cache is keyed on the parameter's in-place version counter).

The three GEMMs form each 128-wide block product exactly by default; with
``fp8_matrix_core=True`` they use the FP8 matrix instructions instead (about
1.5 times the GEMM rate; the hardware truncates small products inside groups
of 8 positions, an error up to about 2^-10 of the block's sum of |a*b|).
"""

import torch

from . import binding as B


class _WeightCache:
    """Wq, Sw, WqT, SwT of one BF16 weight, rebuilt when the weight changes."""

    def __init__(self):
        self.version = None
        self.ptr = None
        self.tensors = None
        self.builds = 0

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
        weight = ctx.weight
        _, _, wqT, swT = ctx.cache.get(weight)
        dy = dy.contiguous()
        dyq, sdy, dyqT, sdyT = B.fp8_quant_1x128_dual(dy)
        dx = B.fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, fp8_matrix_core=ctx.mc)
        if getattr(weight, "main_grad", None) is None:
            weight.main_grad = torch.zeros(weight.shape, dtype=torch.float32, device=weight.device)
        B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=ctx.M, dw=weight.main_grad, accumulate=True,
                               fp8_matrix_core=ctx.mc)
        return dx, None, None, None


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

    @property
    def weight_quantisations(self):
        """How many times the FP8 weight has been (re)built."""
        return self._cache.builds

    def forward(self, x):
        shape = x.shape
        x2 = x.reshape(-1, self.in_features)
        if x2.stride(1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
            x2 = x2.contiguous()
        y = _Fp8LinearFn.apply(x2, self.weight, self._cache, self.fp8_matrix_core)
        return y.reshape(*shape[:-1], self.out_features)
