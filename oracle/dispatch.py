"""MoE dispatch payload and combine (test infrastructure; see the package docstring).

What is computed (DeepSeek-V3 report section 3.3.3, low-precision storage
and communication): the activations entering the MoE experts are quantized to
FP8 before they are dispatched (innerforce.co.kr page), so every copy of a
token sent to an expert carries the token's FP8 codes and scales; the combine
that brings the experts' outputs back to the tokens is kept in BF16
(why-be.why-be.co.kr page). The report has each token choose several experts
(page headed "Deepseek : The Ultimate Convenience!": 8 routed experts plus a
shared one), hence topk copies per token.

Readings taken where the pages are silent:
  * the payload is the 1x128 activation quantization of the token row
    (quant_act_1x128), identical for all copies of a token;
  * the copies are laid out for the grouped GEMM: rows sorted by expert,
    stably, so that inside an expert the copies follow (token, slot) order;
  * combine: out[t] = sum_j w[t][j] * Y[pos[t][j]], rounded to BF16 once.
"""

import numpy as np

from .quant import quant_act_1x128
from .tolerance import bf16_bits_to_f64, bf16_ulp


def route(topk_ids, E):
    """Stable sort of the (token, slot) pairs by expert.

    topk_ids[T][topk] ints in [0, E). Returns offsets[E+1] (expert e owns rows
    offsets[e] .. offsets[e+1]-1), pos[T][topk] (row of each pair) and
    src_row[T*topk] (token of each row).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert ids must lie in [0, E)")
    flat = ids.reshape(-1)                          # pair i = t * topk + j
    order = np.argsort(flat, kind="stable")         # rows -> pairs
    pos = np.empty(T * topk, np.int64)
    pos[order] = np.arange(T * topk)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(np.bincount(flat, minlength=E))
    return offsets, pos.reshape(T, topk), order // topk


def dispatch_quant(x, topk_ids, E):
    """The dispatched payload: (q[T*topk][K], s[K/128][T*topk], offsets, pos, src_row)."""
    offsets, pos, src = route(topk_ids, E)
    q_tok, s_tok = quant_act_1x128(x)
    return q_tok[src], np.ascontiguousarray(s_tok[:, src]), offsets, pos, src


def combine_ref(Y, pos, w):
    """ref[T][N] = sum_j w[t][j] * Y[pos[t][j]] in float64, and absref = sum |w y|.

    Y: float64-convertible values [T*topk][N] (BF16 widened exactly).
    """
    Y = np.asarray(Y, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    T, topk = pos.shape
    ref = np.zeros((T, Y.shape[1]), np.float64)
    absref = np.zeros_like(ref)
    for j in range(topk):
        term = w[:, j:j + 1] * Y[pos[:, j]]
        ref += term
        absref += np.abs(term)
    return ref, absref


def check_combine(out_bf16_bits, ref, absref, topk):
    """Acceptance bound of the combine: FP32 fused multiply-adds over topk terms
    (each rounding at most 2^-24 of the running magnitude, itself at most
    absref) and one BF16 rounding: |out - ref| <= topk 2^-24 absref + ulp_bf16(ref).

    Returns (ok mask, worst ratio of error to bound).
    """
    out = bf16_bits_to_f64(out_bf16_bits)
    bound = topk * 2.0 ** -24 * absref + bf16_ulp(ref)
    err = np.abs(out - ref)
    ok = err <= bound
    return ok, float(np.max(err / bound)) if err.size else 0.0
