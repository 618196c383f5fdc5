"""Fine-grained group quantization (test infrastructure; see the package docstring).

The method (DeepSeek-V3 report section 3.3.2, paraphrased on the
innerforce.co.kr page): elements are quantized in small groups, each group
sharing one scaling factor, so that an outlier only costs precision inside its
own group; the groups of both GEMM operands run along the inner (K) dimension.

Readings taken where the pages are silent:
  * group geometry: activations 1x128 (one row, 128 consecutive K), weights
    128x128 blocks, Wgrad operands 128x1 (128 consecutive tokens of one
    channel) with the output written transposed, because the pages call a
    transposition fused into the GEMM cumbersome (report section 3.5.2, on the
    page headed "Deepseek : The Ultimate Convenience!");
  * scale s = fl32(amax / 448) with IEEE float32 division; an all-zero group
    (or one whose scale underflows to zero) gets s = 1.0;
  * codes = E4M3(fl32(x / s)) with IEEE float32 division, not a multiply by a
    reciprocal: the float32 rounding followed by the E4M3 rounding is part of
    the definition;
  * dequantized value = decode(code) * s.

Scale-grid layouts: 1x128 -> s[K/128][M]; 128x128 -> s[N/128][K/128];
128x1 transposed -> sT[M/128][C]; every grid is row-major float32.
"""

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode

GROUP = 128


def bf16_bits_to_f32(bits):
    """Widen BF16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _as_f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    if x.dtype != np.float32:
        raise TypeError("oracle quantizers take float32 values or BF16 bits (uint16)")
    return x


def group_scale(amax):
    """s = fl32(amax / 448) (IEEE float32 division); zero -> 1.0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(E4M3_MAX)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def pow2_scale(amax):
    """Power-of-two variant: the smallest power of two not below group_scale(amax)
    (fl32(amax / 448), 1.0 for a zero group) and not below 2^-126.

    Reading for the hardware-scaled variant: gfx950's MFMA takes E8M0 (pure
    power-of-two) operand scales, and the smallest such scale that keeps the
    group's largest value inside the E4M3 range is the ceiling power of two.
    """
    r = group_scale(amax).astype(np.float64)          # exact widening
    m, e = np.frexp(r)                                # r = m 2^e, m in [0.5, 1)
    s = np.where(m == 0.5, r, np.ldexp(1.0, e))
    return np.maximum(s, 2.0 ** -126).astype(np.float32)


def _scale(amax, pow2):
    return pow2_scale(amax) if pow2 else group_scale(amax)


def _cast_group(x, s):
    """codes = E4M3(fl32(x / s)) with s broadcast over the group."""
    y = (x / s).astype(np.float32)        # numpy float32 division is IEEE, round-to-nearest-even
    return e4m3_encode(y)


def quant_act_1x128(x, pow2=False):
    """Activation quantization, one scale per (row m, 128-wide K chunk kb).

    x: [M][K] float32 (or BF16 bits). Returns q[M][K] uint8, s[K/128][M] float32.
    pow2 selects the power-of-two scale (pow2_scale).
    """
    x = _as_f32(x)
    M, K = x.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    nkb = K // GROUP
    g = x.reshape(M, nkb, GROUP)                      # group (m, kb)
    amax = np.max(np.abs(g), axis=2) if M else np.zeros((0, nkb), np.float32)
    s = _scale(amax, pow2)                            # [M][nkb]
    q = _cast_group(g, s[:, :, None]).reshape(M, K)
    return q, np.ascontiguousarray(s.T)


def quant_w_128x128(w, transposed=False, pow2=False):
    """Weight quantization, one scale per 128x128 block (nb, kb).

    w: [N][K] float32 (or BF16 bits). Returns q[N][K], s[N/128][K/128]; with
    ``transposed`` also qT[K][N] = q^T and sT[K/128][N/128] = s^T (the same
    codes and scales, laid out for the Dgrad GEMM).
    """
    w = _as_f32(w)
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    nnb, nkb = N // GROUP, K // GROUP
    blk = w.reshape(nnb, GROUP, nkb, GROUP)           # [nb][i][kb][j]
    amax = np.max(np.abs(blk), axis=(1, 3))           # [nb][kb]
    s = _scale(amax, pow2)
    q = _cast_group(blk, s[:, None, :, None]).reshape(N, K)
    if not transposed:
        return q, s
    return q, s, np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def quant_act_128x1_T(x, pow2=False):
    """Wgrad-operand quantization, one scale per (token chunk tb, channel c).

    x: [M][C] float32 (or BF16 bits), M a multiple of 128. Groups are 128
    consecutive tokens of one channel. Returns the codes transposed,
    qT[C][M], and sT[M/128][C].
    """
    x = _as_f32(x)
    M, C = x.shape
    if M % GROUP:
        raise ValueError("M must be a multiple of 128")
    ntb = M // GROUP
    g = x.reshape(ntb, GROUP, C)                      # group (tb, c) = g[tb, :, c]
    amax = np.max(np.abs(g), axis=1)                  # [ntb][C]
    s = _scale(amax, pow2)
    q = _cast_group(g, s[:, None, :]).reshape(M, C)
    return np.ascontiguousarray(q.T), s
