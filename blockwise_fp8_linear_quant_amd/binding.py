"""Thin Python binding over the C ABI of libfp8blk.so.

Functions carry the C names.  They only marshal arguments: torch tensors
provide device memory, `torch.cuda.current_stream()` provides the stream, and
every step of the computation runs in the HIP kernels behind the C ABI.
Outputs the caller does not pass in are allocated with torch.

Layouts (see include/fp8blk.h for the full contract):
  row-wise codes  q [R, C] uint8, scales [ceil(C/128), R] float32 (group-major)
  token-dim codes qT [C, round_up(M,128)] uint8, scales [ceil(M/128), C] float32
  block codes     q [R, C] uint8, scales [ceil(R/128), ceil(C/128)] float32
Scale tensors may be row-strided views (leading dimension padded to a multiple
of 4 floats so that the GEMMs can read them with 16-byte loads).
"""

import operator

import torch

from . import _lib

OUT_F32 = 0
OUT_BF16 = 1


def _stream(t):
    return ctypes_stream(torch.cuda.current_stream(t.device))


def ctypes_stream(s):
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _round_up(a, b):
    return (a + b - 1) // b * b


def _check_2d(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a 2-D {dtype} CUDA tensor")
    if t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be row-major with unit column stride")


# The C ABI sees only pointers and leading dimensions, so every tensor the
# kernels read or write is checked here: a host tensor, a tensor on another
# device or one smaller than the region the kernel covers would otherwise be
# an out-of-bounds device access.
def _check(t, dtype, name, rows, cols, device, exact=False):
    """2-D `dtype` tensor on `device`, row-major, at least (exactly, dense) rows x cols."""
    _check_2d(t, dtype, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if exact:
        if tuple(t.shape) != (rows, cols) or not t.is_contiguous():
            raise ValueError(f"{name} must be a dense [{rows}, {cols}] tensor, got {list(t.shape)}")
    elif t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} must be at least [{rows}, {cols}], got {list(t.shape)}")
    return t


def _check_out(t, name, rows, cols, device):
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be float32 or bfloat16")
    return _check(t, t.dtype, name, rows, cols, device)


def _codes(rows, cols, device):
    """uint8 [rows, cols] view of a buffer whose leading dimension is a multiple of 16 bytes."""
    ld = _round_up(max(cols, 1), 16)
    return torch.empty((rows, ld), dtype=torch.uint8, device=device)[:, :cols]


def _scales(rows, cols, device):
    """float32 [rows, cols] view of a buffer whose leading dimension is a multiple of 4."""
    ld = _round_up(max(cols, 1), 4)
    return torch.empty((rows, ld), dtype=torch.float32, device=device)[:, :cols]


def fp8_quant_1x128(x, transpose_out=False, q=None, scales=None):
    """1x128 group quantisation of BF16 x [rows, cols] -> (codes, scales)."""
    _check_2d(x, torch.bfloat16, "x")
    R, C = x.shape
    if not transpose_out:
        q = _codes(R, C, x.device) if q is None else _check(q, torch.uint8, "q", R, C, x.device)
        G = -(-C // 128)
        scales = _scales(G, R, x.device) if scales is None else _check(scales, torch.float32, "scales", G, R, x.device)
    else:
        Mp, G = _round_up(R, 128), -(-R // 128)
        if q is None:
            q = torch.empty((C, Mp), dtype=torch.uint8, device=x.device)
        _check(q, torch.uint8, "q", C, Mp, x.device)
        scales = _scales(G, C, x.device) if scales is None else _check(scales, torch.float32, "scales", G, C, x.device)
    st = _lib.load().fp8_quant_1x128(
        _ptr(x), R, C, x.stride(0), 1 if transpose_out else 0,
        _ptr(q), q.stride(0), _ptr(scales), scales.stride(0), _stream(x))
    _lib.check(st, "fp8_quant_1x128")
    return q, scales


def fp8_quant_1x128_dual(x, q=None, scales=None, qT=None, scalesT=None):
    """Row-wise and token-dimension 1x128 quantisation of x from one read.

    Returns (q, scales, qT, scalesT), identical to fp8_quant_1x128(x) and
    fp8_quant_1x128(x, transpose_out=True).
    """
    _check_2d(x, torch.bfloat16, "x")
    R, C = x.shape
    q, scales, qT, scalesT = _dual_outputs(R, C, x.device, q, scales, qT, scalesT)
    st = _lib.load().fp8_quant_1x128_dual(
        _ptr(x), R, C, x.stride(0), _ptr(q), q.stride(0), _ptr(scales), scales.stride(0),
        _ptr(qT), qT.stride(0), _ptr(scalesT), scalesT.stride(0), _stream(x))
    _lib.check(st, "fp8_quant_1x128_dual")
    return q, scales, qT, scalesT


def _dual_outputs(R, C, device, q, scales, qT, scalesT):
    """Outputs of the dual quantisers: allocated when not given, else checked."""
    G, Mp, GT = -(-C // 128), _round_up(R, 128), -(-R // 128)
    q = _codes(R, C, device) if q is None else _check(q, torch.uint8, "q", R, C, device)
    scales = _scales(G, R, device) if scales is None else _check(scales, torch.float32, "scales", G, R, device)
    if qT is None:
        qT = torch.empty((C, Mp), dtype=torch.uint8, device=device)
    _check(qT, torch.uint8, "qT", C, Mp, device)
    scalesT = _scales(GT, C, device) if scalesT is None else _check(scalesT, torch.float32, "scalesT", GT, C, device)
    return q, scales, qT, scalesT


def fp8_swiglu_quant_1x128_dual(gate, up, h_out=None, q=None, scales=None, qT=None, scalesT=None):
    """Both 1x128 orientations of silu(gate) * up, formed in registers.

    Returns (q, scales, qT, scalesT); with h_out (BF16 [R, C]) the fused BF16
    value is written there too.
    """
    _check_2d(gate, torch.bfloat16, "gate")
    R, C = gate.shape
    _check(up, torch.bfloat16, "up", R, C, gate.device)
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    if h_out is not None:
        _check(h_out, torch.bfloat16, "h_out", R, C, gate.device)
    q, scales, qT, scalesT = _dual_outputs(R, C, gate.device, q, scales, qT, scalesT)
    st = _lib.load().fp8_swiglu_quant_1x128_dual(
        _ptr(gate), gate.stride(0), _ptr(up), up.stride(0), R, C, _ptr(q), q.stride(0), _ptr(scales),
        scales.stride(0), _ptr(qT), qT.stride(0), _ptr(scalesT), scalesT.stride(0),
        _ptr(h_out), h_out.stride(0) if h_out is not None else 0, _stream(gate))
    _lib.check(st, "fp8_swiglu_quant_1x128_dual")
    return q, scales, qT, scalesT


def fp8_rmsnorm_quant_1x128_dual(x, gamma, eps=1e-6, y_out=None, rstd=None, q=None, scales=None, qT=None,
                                 scalesT=None):
    """Both 1x128 orientations of RMSNorm(x) * gamma, formed in registers.

    Returns (q, scales, qT, scalesT, rstd); with y_out (BF16 [R, C]) the
    normalised BF16 value is written there too.
    """
    _check_2d(x, torch.bfloat16, "x")
    R, C = x.shape
    if (not isinstance(gamma, torch.Tensor) or gamma.dtype != torch.bfloat16 or gamma.dim() != 1
            or gamma.shape[0] != C or not gamma.is_contiguous() or gamma.device != x.device):
        raise TypeError("gamma must be a contiguous BF16 vector of length cols on the device of x")
    if y_out is not None:
        _check(y_out, torch.bfloat16, "y_out", R, C, x.device)
    q, scales, qT, scalesT = _dual_outputs(R, C, x.device, q, scales, qT, scalesT)
    if rstd is None:
        rstd = torch.empty(R, dtype=torch.float32, device=x.device)
    elif (rstd.dtype != torch.float32 or rstd.dim() != 1 or rstd.shape[0] < R or not rstd.is_contiguous()
          or rstd.device != x.device):
        raise ValueError("rstd must be a contiguous float32 vector of at least rows entries on the device of x")
    st = _lib.load().fp8_rmsnorm_quant_1x128_dual(
        _ptr(x), x.stride(0), _ptr(gamma), float(eps), R, C, _ptr(rstd), _ptr(q), q.stride(0), _ptr(scales),
        scales.stride(0), _ptr(qT), qT.stride(0), _ptr(scalesT), scalesT.stride(0),
        _ptr(y_out), y_out.stride(0) if y_out is not None else 0, _stream(x))
    _lib.check(st, "fp8_rmsnorm_quant_1x128_dual")
    return q, scales, qT, scalesT, rstd


def fp8_quant_128x128(w, with_transpose=False, q=None, scales=None, qT=None, scalesT=None):
    """128x128 block quantisation of BF16 w [rows, cols] -> (q, scales, qT, scalesT)."""
    _check_2d(w, torch.bfloat16, "w")
    R, C = w.shape
    br, bc = -(-R // 128), -(-C // 128)
    dev = w.device
    q = _codes(R, C, dev) if q is None else _check(q, torch.uint8, "q", R, C, dev)
    if scales is None:
        scales = torch.empty((br, bc), dtype=torch.float32, device=dev)
    _check(scales, torch.float32, "scales", br, bc, dev, exact=True)
    if with_transpose:
        qT = _codes(C, R, dev) if qT is None else _check(qT, torch.uint8, "qT", C, R, dev)
        if scalesT is None:
            scalesT = torch.empty((bc, br), dtype=torch.float32, device=dev)
        _check(scalesT, torch.float32, "scalesT", bc, br, dev, exact=True)
    elif qT is not None or scalesT is not None:
        raise ValueError("qT and scalesT are written only with with_transpose=True")
    st = _lib.load().fp8_quant_128x128(
        _ptr(w), R, C, w.stride(0), _ptr(q), q.stride(0), _ptr(scales),
        _ptr(qT), qT.stride(0) if qT is not None else 0, _ptr(scalesT), _stream(w))
    _lib.check(st, "fp8_quant_128x128")
    return q, scales, qT, scalesT


def _out(shape, out_dtype, device, y):
    if y is not None:
        return _check_out(y, "output", shape[0], shape[1], device)
    return torch.empty(shape, dtype=out_dtype, device=device)


def _check_gemm_operands(op, a, sa, b, sb, M, N, K, c):
    """Shapes the kernels read and write, by operation (see the C entry points)."""
    _check_2d(a, torch.uint8, "a")
    dev = a.device
    try:
        M, N, K = operator.index(M), operator.index(N), operator.index(K)
    except TypeError:
        raise ValueError("M, N and K must be integers") from None
    if min(M, N, K) < 0:
        raise ValueError("M, N and K must be non-negative")
    if op == OP_WGRAD:
        Mp, G = _round_up(M, 128), -(-M // 128)
        _check(a, torch.uint8, "dyqT", N, Mp, dev)
        _check(sa, torch.float32, "sdyT", G, N, dev)
        _check(b, torch.uint8, "xqT", K, Mp, dev)
        _check(sb, torch.float32, "sxT", G, K, dev)
        _check(c, torch.float32, "dw", N, K, dev)
    else:
        I, J, L = (M, N, K) if op == OP_FWD else (M, K, N)
        _check(a, torch.uint8, "a", I, L, dev)
        _check(sa, torch.float32, "row scales", -(-L // 128), I, dev)
        _check(b, torch.uint8, "b", J, L, dev)
        _check(sb, torch.float32, "block scales", -(-J // 128), -(-L // 128), dev, exact=True)
        _check_out(c, "output", I, J, dev)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return OUT_F32
    if t.dtype == torch.bfloat16:
        return OUT_BF16
    raise TypeError("output must be float32 or bfloat16")


FLAG_EXACT_BLOCKS = 0
FLAG_FP8_MATRIX_CORE = 1
FLAG_SPLIT2 = 2
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2

# Split-K workspaces, one per (device, stream): zero-filled when allocated (the
# library needs its counters to start at zero and leaves them at zero), grown
# when a larger problem needs more.  Calls on one stream are ordered, so they
# can share one; calls on different streams get different ones.
_workspaces = {}


def _workspace(workspace, op, M, N, K, split2, device, stream):
    """(pointer, bytes) of the workspace a GEMM call gets: None/False -> none,
    a uint8 CUDA tensor -> that tensor, True -> the binding's per-stream one."""
    if workspace is None or workspace is False:
        return None, 0
    if isinstance(workspace, torch.Tensor):
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != device:
            raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
        return workspace.data_ptr(), workspace.numel()
    lib = _lib.load()
    need = int((lib.fp8_block_gemm_split2_workspace_size if split2 else lib.fp8_block_gemm_workspace_size)(
        op, M, N, K))
    if need == 0:
        return None, 0
    key = (device, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws.data_ptr(), ws.numel()


def fp8_block_gemm(op, a, sa, b, sb, M, N, K, c, accumulate=False, fp8_matrix_core=False, workspace=True,
                   split2=False):
    """The generic C entry point (explicit op and matrix path); c is preallocated.

    workspace: True (the binding's zero-initialised per-stream workspace),
    False/None (none) or a caller-owned uint8 tensor.  split2 forces the
    contraction split in two whenever the workspace allows it."""
    if op not in (OP_FWD, OP_DGRAD, OP_WGRAD):
        raise ValueError("op must be OP_FWD, OP_DGRAD or OP_WGRAD")
    _check_gemm_operands(op, a, sa, b, sb, M, N, K, c)
    ld_sb = sb.stride(0) if op == OP_WGRAD else 0
    stream = _stream(a)
    ws, ws_bytes = _workspace(workspace, op, M, N, K, split2, a.device, stream)
    flags = (FLAG_FP8_MATRIX_CORE if fp8_matrix_core else FLAG_EXACT_BLOCKS) | (FLAG_SPLIT2 if split2 else 0)
    st = _lib.load().fp8_block_gemm(
        op, flags, _ptr(a), a.stride(0), _ptr(sa), sa.stride(0), _ptr(b), b.stride(0), _ptr(sb), ld_sb,
        M, N, K, _ptr(c), c.stride(0), _dtype_code(c), 1 if accumulate else 0, ws, ws_bytes, stream)
    _lib.check(st, "fp8_block_gemm")
    return c


def fp8_block_gemm_split2_noalloc(op, a, sa, b, sb, M, N, K, c, accumulate=False, fp8_matrix_core=False):
    """fp8_block_gemm split in two along the contraction, with the library's static
    scratch instead of a workspace (nothing is allocated); c is preallocated."""
    if op not in (OP_FWD, OP_DGRAD, OP_WGRAD):
        raise ValueError("op must be OP_FWD, OP_DGRAD or OP_WGRAD")
    _check_gemm_operands(op, a, sa, b, sb, M, N, K, c)
    ld_sb = sb.stride(0) if op == OP_WGRAD else 0
    st = _lib.load().fp8_block_gemm_split2_noalloc(
        op, FLAG_FP8_MATRIX_CORE if fp8_matrix_core else FLAG_EXACT_BLOCKS,
        _ptr(a), a.stride(0), _ptr(sa), sa.stride(0), _ptr(b), b.stride(0), _ptr(sb), ld_sb,
        M, N, K, _ptr(c), c.stride(0), _dtype_code(c), 1 if accumulate else 0, _stream(a))
    _lib.check(st, "fp8_block_gemm_split2_noalloc")
    return c


def fp8_block_gemm_fwd(xq, sx, wq, sw, out_dtype=torch.bfloat16, y=None, fp8_matrix_core=False, workspace=True,
                       split2=False):
    """Y[M, N] = Xq . Wq^T with 1x128 row scales sx [K/128, M] and block scales sw [N/128, K/128].
    workspace / split2: as for fp8_block_gemm."""
    _check_2d(xq, torch.uint8, "xq")
    _check_2d(wq, torch.uint8, "wq")
    M, K = xq.shape
    N = wq.shape[0]
    y = _out((M, N), out_dtype, xq.device, y)
    _check_gemm_operands(OP_FWD, xq, sx, wq, sw, M, N, K, y)
    if fp8_matrix_core or split2:
        return fp8_block_gemm(OP_FWD, xq, sx, wq, sw, M, N, K, y, fp8_matrix_core=fp8_matrix_core,
                              workspace=workspace, split2=split2)
    stream = _stream(xq)
    ws, ws_bytes = _workspace(workspace, OP_FWD, M, N, K, False, xq.device, stream)
    st = _lib.load().fp8_block_gemm_fwd(
        _ptr(xq), xq.stride(0), _ptr(sx), sx.stride(0), _ptr(wq), wq.stride(0), _ptr(sw),
        M, N, K, _ptr(y), y.stride(0), _dtype_code(y), ws, ws_bytes, stream)
    _lib.check(st, "fp8_block_gemm_fwd")
    return y


def fp8_block_gemm_dgrad(dyq, sdy, wqT, swT, out_dtype=torch.bfloat16, dx=None, fp8_matrix_core=False,
                         workspace=True, split2=False):
    """dX[M, K] = dY . W from dYq [M, N] (row scales sdy [N/128, M]) and WqT [K, N] (scales swT [K/128, N/128]).
    workspace / split2: as for fp8_block_gemm."""
    _check_2d(dyq, torch.uint8, "dyq")
    _check_2d(wqT, torch.uint8, "wqT")
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = _out((M, K), out_dtype, dyq.device, dx)
    _check_gemm_operands(OP_DGRAD, dyq, sdy, wqT, swT, M, N, K, dx)
    if fp8_matrix_core or split2:
        return fp8_block_gemm(OP_DGRAD, dyq, sdy, wqT, swT, M, N, K, dx, fp8_matrix_core=fp8_matrix_core,
                              workspace=workspace, split2=split2)
    stream = _stream(dyq)
    ws, ws_bytes = _workspace(workspace, OP_DGRAD, M, N, K, False, dyq.device, stream)
    st = _lib.load().fp8_block_gemm_dgrad(
        _ptr(dyq), dyq.stride(0), _ptr(sdy), sdy.stride(0), _ptr(wqT), wqT.stride(0), _ptr(swT),
        M, N, K, _ptr(dx), dx.stride(0), _dtype_code(dx), ws, ws_bytes, stream)
    _lib.check(st, "fp8_block_gemm_dgrad")
    return dx


def fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=None, dw=None, accumulate=False, fp8_matrix_core=False,
                         workspace=True, split2=False):
    """dW[N, K] (+)= dY^T . X from token-dimension codes dyqT [N, M_pad], xqT [K, M_pad].
    workspace / split2: as for fp8_block_gemm (split2=True splits the tokens in two)."""
    _check_2d(dyqT, torch.uint8, "dyqT")
    _check_2d(xqT, torch.uint8, "xqT")
    N = dyqT.shape[0]
    K = xqT.shape[0]
    if M is None:
        M = dyqT.shape[1]
    if dw is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing dw")
        dw = torch.empty((N, K), dtype=torch.float32, device=dyqT.device)
    _check_gemm_operands(OP_WGRAD, dyqT, sdyT, xqT, sxT, M, N, K, dw)
    if fp8_matrix_core or split2:
        return fp8_block_gemm(OP_WGRAD, dyqT, sdyT, xqT, sxT, M, N, K, dw, accumulate,
                              fp8_matrix_core=fp8_matrix_core, workspace=workspace, split2=split2)
    stream = _stream(dyqT)
    ws, ws_bytes = _workspace(workspace, OP_WGRAD, M, N, K, False, dyqT.device, stream)
    st = _lib.load().fp8_block_gemm_wgrad(
        _ptr(dyqT), dyqT.stride(0), _ptr(sdyT), sdyT.stride(0), _ptr(xqT), xqT.stride(0), _ptr(sxT),
        sxT.stride(0), M, N, K, _ptr(dw), dw.stride(0), 1 if accumulate else 0, ws, ws_bytes, stream)
    _lib.check(st, "fp8_block_gemm_wgrad")
    return dw


def bf16_gemm_nt(a, b, out_dtype=torch.bfloat16, c=None):
    """C[M, N] = A[M, K] . B[N, K]^T over BF16 operands (the BF16 baseline GEMM)."""
    _check_2d(a, torch.bfloat16, "a")
    M, K = a.shape
    _check(b, torch.bfloat16, "b", 0, K, a.device)
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must have the same number of columns")
    c = _out((M, N), out_dtype, a.device, c)
    st = _lib.load().bf16_gemm_nt(_ptr(a), a.stride(0), _ptr(b), b.stride(0), M, N, K,
                                  _ptr(c), c.stride(0), _dtype_code(c), _stream(a))
    _lib.check(st, "bf16_gemm_nt")
    return c


def fp8_e4m3_encode(x, q=None):
    """Elementwise binary32 -> E4M3 codes with the library's device encoder."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 CUDA tensor")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    elif (q.dtype != torch.uint8 or q.numel() != x.numel() or not q.is_contiguous() or q.device != x.device):
        raise ValueError("q must be a contiguous uint8 tensor with x's number of elements on x's device")
    st = _lib.load().fp8_e4m3_encode(_ptr(x), _ptr(q), x.numel(), _stream(x))
    _lib.check(st, "fp8_e4m3_encode")
    return q


def fp8_block_gemm_workspace_size(op, M, N, K):
    return int(_lib.load().fp8_block_gemm_workspace_size(op, M, N, K))


def fp8_block_gemm_split2_workspace_size(op, M, N, K):
    return int(_lib.load().fp8_block_gemm_split2_workspace_size(op, M, N, K))


def fp8blk_version():
    return _lib.load().fp8blk_version().decode()
