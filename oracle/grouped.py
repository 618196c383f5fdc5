"""Per-expert Wgrad path (test infrastructure; see the package docstring).

What is computed: the FP8 Wgrad GEMM (report sections 3.3.1-3.3.2 on the
innerforce.co.kr page) contracts over tokens, so both of its operands are
quantized in groups of 128 consecutive tokens of one channel. In the MoE
experts every expert sees its own batch of tokens (report section 3.4.2, page
headed "Deepseek : The Ultimate Convenience!"), so expert e's weight gradient
dW_e = dY_e^T X_e contracts over that expert's tokens only.

Readings taken where the pages are silent:
  * an expert's tokens are cut into groups of 128 from its first token; a last
    group with fewer than 128 tokens is completed with zero tokens, which
    change neither its amax nor any product (their codes are +0);
  * the groups of all experts are numbered expert-major and stored side by
    side: P_e = sum over e' < e of ceil(M_e' / 128) groups come before expert
    e, and its group j occupies columns 128 (P_e + j) .. 128 (P_e + j) + 127
    of the transposed codes and row P_e + j of the scale grid;
  * an expert with no tokens has a zero weight gradient.
"""

import numpy as np

from .gemm import MODE_ROW, gemm_ref_rows
from .quant import GROUP, _as_f32, quant_act_128x1_T


def _check_offsets(offsets, M):
    off = np.asarray(offsets, dtype=np.int64)
    if off.ndim != 1 or len(off) < 1 or off[0] != 0 or off[-1] != M or np.any(np.diff(off) < 0):
        raise ValueError("bad group offsets")
    return off


def padded_group_starts(offsets):
    """P[e] for e = 0..E: groups before expert e (P[E] = all groups)."""
    off = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(off)
    groups = (counts + GROUP - 1) // GROUP
    P = np.zeros(len(off), np.int64)
    P[1:] = np.cumsum(groups)
    return P


def quant_act_128x1_T_grouped(x, offsets):
    """128x1 transposed quantization of every expert's rows of x.

    x: [M_total][C] float32 (or BF16 bits), rows grouped by expert with
    offsets[E+1]. Returns qT[C][128 P_E] (uint8) and sT[P_E][C] (float32).
    """
    x = _as_f32(x)
    M, C = x.shape
    off = _check_offsets(offsets, M)
    P = padded_group_starts(off)
    qT = np.zeros((C, GROUP * int(P[-1])), np.uint8)
    sT = np.zeros((int(P[-1]), C), np.float32)
    for e in range(len(off) - 1):
        rows = x[off[e]:off[e + 1]]
        n = P[e + 1] - P[e]
        if n == 0:
            continue
        padded = np.zeros((GROUP * n, C), np.float32)     # zero tokens complete the last group
        padded[:len(rows)] = rows
        q, s = quant_act_128x1_T(padded)
        qT[:, GROUP * P[e]:GROUP * P[e + 1]] = q
        sT[P[e]:P[e + 1]] = s
    return qT, sT


def grouped_wgrad_ref(A, sA, B, sB, offsets, rows=None, cols=None):
    """Per-expert Wgrad reference.

    A[N][>= 128 P_E], sA[>= P_E][N]: grouped 128x1 quantization of dY;
    B[K][>= 128 P_E], sB[>= P_E][K]: the same for X (same offsets). Returns
    (ref, absref), float64 [E][len(rows)][len(cols)]: expert e's
    C[n][k] = sum over its groups g of sA[g][n] sB[g][k] sum_{t in g} A[n][t] B[k][t].
    """
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    N, K = A.shape[0], B.shape[0]
    off = np.asarray(offsets, dtype=np.int64)
    P = padded_group_starts(off)
    E = len(off) - 1
    rows = np.arange(N) if rows is None else np.asarray(rows)
    cols = np.arange(K) if cols is None else np.asarray(cols)
    ref = np.zeros((E, len(rows), len(cols)), np.float64)
    absref = np.zeros_like(ref)
    sA = np.asarray(sA, dtype=np.float32)
    sB = np.asarray(sB, dtype=np.float32)
    for e in range(E):
        if P[e + 1] == P[e]:
            continue                                      # no tokens: zero gradient
        t = slice(GROUP * P[e], GROUP * P[e + 1])
        g = slice(P[e], P[e + 1])
        r, a = gemm_ref_rows(A[:, t], sA[g], B[:, t], sB[g], MODE_ROW, rows=rows, cols=cols)
        ref[e] = r
        absref[e] = a
    return ref, absref
