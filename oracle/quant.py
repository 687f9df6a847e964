"""Blockwise quantisers: 1x128 groups and 128x128 blocks.  TEST INFRASTRUCTURE.

Pages: arxiv-wiki summary of Puro-2B, section "접근 방법" item (4) -- activation
scales cover 1-D groups of 128 values, weight scales cover 128x128 blocks, the
values are E4M3; paperlayer.ai summary, appendix C "生産学習の詳細", item
"FP8実装pipeline" -- the forward, data-gradient and weight-gradient GEMMs all
take blockwise E4M3 operands.

Readings where the pages are silent (both the oracle and the GPU path follow
them; each is listed in the design notes):

* the scale is a binary32 dequantisation multiplier s = fl32(amax / 448),
  computed by an IEEE division; amax is the exact max |x| over the valid
  elements of the group;
* a code is E4M3(fl32(x / s)), again an IEEE binary32 division (not a
  multiply by a reciprocal), then round-to-nearest-even with saturation;
* an all-zero group has s = 0 and all codes 0x00 (no epsilon clamp);
* binary32 denormals are kept (no flush to zero) in s and in x / s;
* groups that run past the end of a dimension use only their valid elements;
* the weight-gradient operands are quantised afresh from BF16 along the token
  dimension (groups of 128 tokens per feature);
* the transposed weight for the data gradient is Q(W^T), which equals Q(W)^T
  because a block's amax does not depend on orientation.

All arrays are logical (no padding, no storage layout): codes have the shape
of the input, scales have one entry per (row, group) or per block.
"""

import numpy as np

from . import e4m3

GROUP = 128


def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32 values (exact: append 16 zero bits)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _quantise_groups(x, amax):
    """Scale and codes for values x whose group maxima are amax (broadcastable).

    s = fl32(amax / 448); codes = E4M3(fl32(x / s)); s == 0 gives codes 0x00.
    numpy float32 arithmetic is IEEE binary32 with round-to-nearest-even and
    gradual underflow, which is exactly fl32(.).
    """
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quotient = (x / s).astype(np.float32)
    codes = e4m3.encode(quotient)
    codes = np.where(s == 0, np.uint8(0), codes).astype(np.uint8)
    return s, codes


def quant_1x128_rows(x_bits):
    """Row-wise 1x128 quantisation of a BF16 matrix [R, C].

    Groups are 128 consecutive columns of one row (the contraction dimension of
    the forward and data-gradient GEMMs).  Returns (codes uint8 [R, C],
    scales float32 [R, ceil(C/128)]).
    """
    x = bf16_bits_to_f32(x_bits)
    R, C = x.shape
    G = -(-C // GROUP)
    codes = np.zeros((R, C), dtype=np.uint8)
    scales = np.zeros((R, G), dtype=np.float32)
    for g in range(G):
        c0, c1 = g * GROUP, min((g + 1) * GROUP, C)
        blk = x[:, c0:c1]
        amax = np.max(np.abs(blk), axis=1, keepdims=True)
        s, q = _quantise_groups(blk, amax)
        scales[:, g] = s[:, 0]
        codes[:, c0:c1] = q
    return codes, scales


def quant_1x128_tokens(x_bits):
    """Token-dimension 1x128 quantisation of a BF16 matrix [M, C] (tokens x features).

    Groups are 128 consecutive tokens of one feature, which is the row-wise
    quantisation of the transpose.  Returns (codes uint8 [C, M] -- already
    transposed so that tokens are contiguous, scales float32 [C, ceil(M/128)]).
    """
    xt = np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)
    return quant_1x128_rows(xt)


def quant_128x128(w_bits):
    """128x128 block quantisation of a BF16 matrix [R, C].

    Returns (codes uint8 [R, C], scales float32 [ceil(R/128), ceil(C/128)]).
    Edge blocks use only their valid elements.
    """
    w = bf16_bits_to_f32(w_bits)
    R, C = w.shape
    BR, BC = -(-R // GROUP), -(-C // GROUP)
    codes = np.zeros((R, C), dtype=np.uint8)
    scales = np.zeros((BR, BC), dtype=np.float32)
    for br in range(BR):
        r0, r1 = br * GROUP, min((br + 1) * GROUP, R)
        for bc in range(BC):
            c0, c1 = bc * GROUP, min((bc + 1) * GROUP, C)
            blk = w[r0:r1, c0:c1]
            amax = np.float32(np.max(np.abs(blk)))
            s, q = _quantise_groups(blk, amax)
            scales[br, bc] = s
            codes[r0:r1, c0:c1] = q
    return codes, scales


def expand_block_scales(block_scales, rows):
    """Per-row view of 128x128 block scales: [ceil(R/128), G] -> [R, G]."""
    return np.repeat(np.asarray(block_scales), GROUP, axis=0)[:rows]
