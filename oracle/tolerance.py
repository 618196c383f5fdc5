"""Acceptance bound for GEMM outputs (test infrastructure; see the package docstring).

The pages fix no numeric tolerance. The bound used is

    |float(C) - ref| <= 4e-3 * absref + ulp_bf16(ref)        (per element)

where ref and absref come from the float64 reference. The first term absorbs
the device's FP32 accumulation of promoted partials in any order (and any
reassociation of the two scale products); the second absorbs the final BF16
round-to-nearest-even. A wrong scale index, a missing chunk or a transposed
operand produces errors of the order of |ref| and fails it.

ulp_bf16(y) = 2^(max(floor(log2|y|), -126) - 7), and 2^-133 for y == 0.
"""

import numpy as np

REL_TOL = 4e-3


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(y):
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, x = np.frexp(np.where(y > 0, y, 1.0))
    e = np.maximum(x - 1, -126)                   # floor(log2 |y|), clamped at the normal range
    ulp = np.ldexp(1.0, e - 7)
    return np.where(y > 0, ulp, np.ldexp(1.0, -133))


def check_gemm(c_bits, ref, absref, rel_tol=REL_TOL):
    """Compare BF16 output bits with the reference.

    Returns (ok, worst) where ok is the per-element boolean mask and worst is
    the largest |err| / bound (<= 1 means pass), for regression tracking.
    """
    c = bf16_bits_to_f64(c_bits)
    if c.shape != ref.shape:
        raise ValueError(f"shape mismatch {c.shape} vs {ref.shape}")
    bound = rel_tol * np.asarray(absref) + bf16_ulp(ref)
    err = np.abs(c - ref)
    ok = np.isfinite(c) & (err <= bound)
    ratio = np.where(np.isfinite(c), err / bound, np.inf)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return ok, worst
