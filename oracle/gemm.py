"""Block-scaled FP8 GEMM reference (test infrastructure; see the package docstring).

What the method computes (DeepSeek-V3 report section 3.3.2; the promotion
scheme of Figure 7(b) as paraphrased on the why-be.why-be.co.kr page, and the
per-group scaling along the inner dimension on the innerforce.co.kr page):
the FP8 product is formed one inner-dimension interval at a time; at the end
of each interval the partial result is promoted to FP32 and multiplied by the
two operands' group scales, and the promoted, scaled partials are summed in
full precision. Reading: the interval is 128, equal to the quantization group
along K, so each chunk kb carries exactly one scale per A row and one per B
column:

    C[m][n] = sum_kb  sA(kb, m) * sB(kb, n) * P_kb[m][n]
    P_kb[m][n] = sum_{k in chunk kb} dec(A[m][k]) * dec(B[n][k])

A[M][K] and B[N][K] hold E4M3 codes with K contiguous ("TN"). sA is
[K/128][M]. sB is read in one of two modes:
  * "block" (mode 0): sB[N/128][K/128], one scale per 128x128 weight block
    (Fprop with W, Dgrad with the transposed weight copy);
  * "row" (mode 1): sB[K/128][N], one scale per column per chunk (Wgrad,
    where both operands come from the 128x1 transposed quantizer).

Each chunk sum is computed in float64 and is exact: every E4M3 value is an
integer multiple of 2^-9 of magnitude at most 448, so each product is a
multiple of 2^-18 below 2^17.62 and any partial sum of at most 128 of them is
a multiple of 2^-18 below 2^24.62, needing at most 43 significant bits. Any
summation order or blocking therefore gives the same chunk sum, and a plain
float64 matmul may serve as the step. The sum over chunks is float64.

Also returned: absref = sum_kb |sA*sB| * (|dec A| @ |dec B|^T)_kb, the
magnitude used by the acceptance bound.
"""

import numpy as np

from .e4m3 import e4m3_decode
from .quant import GROUP

MODE_BLOCK = 0
MODE_ROW = 1


def _sb_chunk(sB, mode, kb, N, K, cols):
    nkb = K // GROUP
    if mode == MODE_BLOCK:
        grid = np.asarray(sB, dtype=np.float32).reshape(N // GROUP, nkb)
        return grid[cols // GROUP, kb].astype(np.float64)
    if mode == MODE_ROW:
        grid = np.asarray(sB, dtype=np.float32).reshape(nkb, N)
        return grid[kb, cols].astype(np.float64)
    raise ValueError("unknown scale mode")


def gemm_ref_rows(A, sA, B, sB, mode, rows=None, cols=None):
    """Reference for the output rows ``rows`` and columns ``cols`` (all by default).

    Returns (ref, absref), float64 arrays of shape [len(rows)][len(cols)].
    """
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N, Kb = B.shape
    if Kb != K or K % GROUP:
        raise ValueError("inner dimensions must agree and be a multiple of 128")
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    sA = np.asarray(sA, dtype=np.float32).reshape(K // GROUP, M)
    ref = np.zeros((len(rows), len(cols)), np.float64)
    absref = np.zeros_like(ref)
    Ar = A[rows]
    Bc = B[cols]
    for kb in range(K // GROUP):
        ks = slice(kb * GROUP, (kb + 1) * GROUP)
        da = e4m3_decode(Ar[:, ks])
        db = e4m3_decode(Bc[:, ks])
        part = da @ db.T                                   # exact chunk sum (see module docstring)
        apart = np.abs(da) @ np.abs(db).T
        scale = sA[kb, rows].astype(np.float64)[:, None] * _sb_chunk(sB, mode, kb, N, K, cols)[None, :]
        ref += scale * part
        absref += np.abs(scale) * apart
    return ref, absref


def gemm_ref(A, sA, B, sB, mode=MODE_BLOCK):
    """Full reference C (float64) and its magnitude bound absref."""
    return gemm_ref_rows(A, sA, B, sB, mode)


def grouped_gemm_ref(A, sA, B, sB, offsets, rows=None, cols=None):
    """Per-expert form: rows [off[e], off[e+1]) of A use expert e's weights.

    A[M_total][K], sA[K/128][M_total], B[E][N][K], sB[E][N/128][K/128]
    (block mode), offsets[E+1] with offsets[0] = 0, non-decreasing,
    offsets[E] = M_total. Returns (ref, absref) for ``rows`` (all by default)
    and ``cols``.
    """
    A = np.asarray(A, dtype=np.uint8)
    M, K = A.shape
    B = np.asarray(B, dtype=np.uint8)
    E, N, _ = B.shape
    off = np.asarray(offsets, dtype=np.int64)
    if off.shape != (E + 1,) or off[0] != 0 or off[-1] != M or np.any(np.diff(off) < 0):
        raise ValueError("bad group offsets")
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    sA = np.asarray(sA, dtype=np.float32).reshape(K // GROUP, M)
    sB = np.asarray(sB, dtype=np.float32).reshape(E, N // GROUP, K // GROUP)
    ref = np.zeros((len(rows), len(cols)), np.float64)
    absref = np.zeros_like(ref)
    expert = np.searchsorted(off, rows, side="right") - 1
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        # the expert's rows as a small dense problem, with sA columns gathered
        r, a = gemm_ref_rows(A[rows[sel]], sA[:, rows[sel]], B[e], sB[e], MODE_BLOCK, cols=cols)
        ref[sel] = r
        absref[sel] = a
    return ref, absref
