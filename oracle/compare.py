"""Acceptance tests for GPU results against the oracle.  TEST INFRASTRUCTURE.

* Quantised codes and scales: bit-exact (one correct result exists).
* FP32 GEMM outputs: |gpu - Y| <= 1e-5 * Bnd + 1e-6 elementwise, where Y is the
  float64 oracle value and Bnd = sum_l |a_l * b_l| its error budget.  Any
  summation order and any rounding of the combined scale stays inside it.
* BF16 GEMM outputs: within one BF16 ulp of the rounded oracle value; where
  cancellation leaves |Y| far below Bnd, the FP32 budget above (plus half a
  BF16 ulp for the final rounding) is accepted instead, and such elements are
  counted separately.
"""

import numpy as np

FP32_RTOL = 1e-5
FP32_ATOL = 1e-6


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(v):
    """Spacing of BF16 values at |v| (2**-133 in the subnormal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(a)
    return np.ldexp(1.0, np.maximum(ex - 1, -126) - 7)


def check_fp32(gpu, y, bnd, rtol=FP32_RTOL, atol=FP32_ATOL):
    """Returns (ok, report).  report['worst'] = max |err| / allowed (<= 1 passes)."""
    g = np.asarray(gpu, dtype=np.float64)
    err = np.abs(g - y)
    allowed = rtol * bnd + atol
    ratio = err / allowed
    bad = ~(ratio <= 1.0)          # NaN counts as a failure
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    return (not bad.any()), {"n": int(g.size), "bad": int(bad.sum()), "worst": worst,
                             "max_abs_err": float(err.max()) if err.size else 0.0}


def check_bf16(gpu_bits, y, bnd, rtol=FP32_RTOL, atol=FP32_ATOL):
    """BF16 acceptance; gpu_bits are raw BF16 bit patterns.  Returns (ok, report)."""
    from .gemm import round_to_bf16
    g = bf16_bits_to_f64(gpu_bits)
    r = round_to_bf16(y)
    ulp_clause = np.abs(g - r) <= bf16_ulp(r)
    budget_clause = np.abs(g - y) <= rtol * bnd + atol + 0.5 * bf16_ulp(g)
    ok = ulp_clause | budget_clause
    return bool(ok.all()), {"n": int(g.size), "bad": int((~ok).sum()),
                            "budget_only": int((budget_clause & ~ulp_clause).sum()),
                            "exact": int((g == r).sum())}


def check_exact(gpu, ref):
    """Bit-exact comparison.  Returns (ok, n_mismatch).

    Both arrays must have the same shape and the same dtype; otherwise the
    result is (False, -1).  Elements are compared as their stored bit patterns
    (floating-point values through an unsigned integer view of the same
    width), so +0 and -0 differ, a denormal differs from zero, and NaNs match
    only when their payloads match -- the quantisers have exactly one correct
    output, including the sign of a zero scale or code.
    """
    a = np.asarray(gpu)
    b = np.asarray(ref)
    if a.shape != b.shape or a.dtype != b.dtype:
        return False, -1
    if a.dtype.kind not in "biu":
        width = np.dtype("u%d" % a.dtype.itemsize)
        a, b = a.view(width), b.view(width)
    mism = int(np.count_nonzero(a != b))
    return mism == 0, mism
