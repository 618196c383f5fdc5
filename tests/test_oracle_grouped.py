"""Pins for the oracle's per-expert Wgrad path (grouped 128x1 transposed
quantizer and per-expert Wgrad reference).

Checked against: an independent torch computation (float32 division and the
float8_e4m3fn cast after clamping, group by group of each expert's tokens),
the padding and layout rules stated by the reading (zero codes after an
expert's last token, experts' blocks shifting by whole groups when an expert
is prepended), the independence of experts, and for the GEMM a brute-force
float64 product of the per-element dequantized operands over each expert's
tokens (no chunking), plus the unquantized product within the quantization
error.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, grouped_wgrad_ref, padded_group_starts, quant_act_128x1_T_grouped

COUNTS = [0, 1, 127, 128, 129, 300, 0, 64]


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int64)
    off[1:] = np.cumsum(counts)
    return off


def _x(M, C, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, C)).astype(np.float32)
    x[rng.random((M, C)) < 0.01] *= 100.0
    return x


def _torch_expected(x, counts):
    """Group-by-group quantization with torch, independent of the oracle."""
    C = x.shape[1]
    blocks_q, blocks_s = [], []
    start = 0
    for n in counts:
        rows = torch.from_numpy(x[start:start + n])
        start += n
        for j in range(0, n, 128):
            grp = torch.zeros((128, C), dtype=torch.float32)
            grp[:min(128, n - j)] = rows[j:j + 128]
            amax = grp.abs().amax(dim=0)
            s = amax / torch.tensor(448.0, dtype=torch.float32)
            s = torch.where(s == 0, torch.ones_like(s), s)
            y = (grp / s).clamp(-448.0, 448.0)
            blocks_q.append(y.to(torch.float8_e4m3fn).view(torch.uint8).T.numpy())
            blocks_s.append(s.numpy())
    return np.concatenate(blocks_q, axis=1), np.stack(blocks_s)


def test_grouped_quant_matches_torch_group_by_group():
    x = _x(sum(COUNTS), 96, 0)
    qT, sT = quant_act_128x1_T_grouped(x, _offsets(COUNTS))
    q_ref, s_ref = _torch_expected(x, COUNTS)
    assert qT.shape == q_ref.shape and sT.shape == s_ref.shape
    assert np.array_equal(qT, q_ref)
    assert np.array_equal(sT.view(np.uint32), s_ref.view(np.uint32))


def test_grouped_layout_and_padding():
    counts = [129, 0, 5]
    x = _x(sum(counts), 32, 1)
    qT, sT = quant_act_128x1_T_grouped(x, _offsets(counts))
    P = padded_group_starts(_offsets(counts))
    assert list(P) == [0, 2, 2, 3]
    assert qT.shape == (32, 3 * 128) and sT.shape == (3, 32)
    assert np.all(qT[:, 129:256] == 0) and np.all(qT[:, 256 + 5:] == 0)   # padding tokens: +0 codes
    # the max element of every column of every group encodes to +-448
    for g, (lo, n) in enumerate([(0, 128), (128, 1), (129, 5)]):
        cols = x[lo:lo + n]
        arg = np.abs(cols).argmax(axis=0)
        codes = qT[np.arange(32), 128 * g + arg]
        assert np.all((codes == 0x7E) | (codes == 0xFE))


def test_grouped_quant_experts_independent_and_shift_by_whole_groups():
    counts = [200, 70, 130]
    x = _x(sum(counts), 40, 2)
    qT, sT = quant_act_128x1_T_grouped(x, _offsets(counts))
    # changing expert 1's rows leaves experts 0 and 2 unchanged
    x2 = x.copy()
    x2[200:270] *= -3.0
    qT2, sT2 = quant_act_128x1_T_grouped(x2, _offsets(counts))
    P = padded_group_starts(_offsets(counts))
    for e in (0, 2):
        c = slice(128 * P[e], 128 * P[e + 1])
        assert np.array_equal(qT[:, c], qT2[:, c]) and np.array_equal(sT[P[e]:P[e + 1]], sT2[P[e]:P[e + 1]])
    # prepending an expert of 256 tokens shifts everything by two groups
    pre = _x(256, 40, 3)
    qT3, sT3 = quant_act_128x1_T_grouped(np.concatenate([pre, x]), _offsets([256] + counts))
    assert np.array_equal(qT3[:, 256:], qT) and np.array_equal(sT3[2:], sT)


def test_grouped_quant_dequantizes_within_e4m3_rounding():
    counts = [3, 250, 128]
    x = _x(sum(counts), 24, 4)
    qT, sT = quant_act_128x1_T_grouped(x, _offsets(counts))
    P = padded_group_starts(_offsets(counts))
    off = _offsets(counts)
    for e in range(len(counts)):
        for t in range(off[e], off[e + 1]):
            g = P[e] + (t - off[e]) // 128
            col = 128 * P[e] + (t - off[e])
            deq = e4m3_decode(qT[:, col]) * sT[g].astype(np.float64)
            err = np.abs(deq - x[t])
            # RNE on a 3-bit mantissa: half a quantum, relative 2^-4 (normal), 2^-10 s (subnormal)
            assert np.all(err <= np.abs(x[t]) * 2.0 ** -4 + sT[g] * 2.0 ** -10 + 0.0)


def _codes(shape, rng):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B
    return c


def _zero_padding(qT, counts):
    off, P = _offsets(counts), padded_group_starts(_offsets(counts))
    for e, n in enumerate(counts):
        qT[:, 128 * P[e] + n:128 * P[e + 1]] = 0
    return qT


def test_grouped_wgrad_ref_matches_dequantized_brute_force():
    rng = np.random.default_rng(5)
    counts = [0, 130, 1, 256]
    P = padded_group_starts(_offsets(counts))
    G = int(P[-1])
    N, K = 64, 48
    A = _zero_padding(_codes((N, 128 * G), rng), counts)
    B = _zero_padding(_codes((K, 128 * G), rng), counts)
    sA = (2.0 ** rng.integers(-8, 9, (G, N)) * rng.uniform(0.5, 1.0, (G, N))).astype(np.float32)
    sB = (2.0 ** rng.integers(-8, 9, (G, K)) * rng.uniform(0.5, 1.0, (G, K))).astype(np.float32)
    ref, absref = grouped_wgrad_ref(A, sA, B, sB, _offsets(counts))
    assert ref.shape == (len(counts), N, K)
    # brute force: dequantize every element with its own group's scale, then
    # one float64 product over all of the expert's token columns
    grp = np.repeat(np.arange(G), 128)
    dA = torch.from_numpy(e4m3_decode(A) * sA[grp].T.astype(np.float64))
    dB = torch.from_numpy(e4m3_decode(B) * sB[grp].T.astype(np.float64))
    for e in range(len(counts)):
        c = slice(128 * P[e], 128 * P[e + 1])
        want = (dA[:, c] @ dB[:, c].T).numpy()
        assert np.allclose(ref[e], want, rtol=0, atol=1e-12 * (absref[e].max() + 1e-300))
    assert np.all(ref[0] == 0) and np.all(absref[0] == 0)


def test_grouped_wgrad_of_quantized_operands_approximates_the_exact_product():
    # end to end through the oracle: quantize dY and X per expert, then the
    # per-expert Wgrad is close to dY_e^T X_e (each operand within E4M3 rounding)
    counts = [140, 0, 256, 17]
    M = sum(counts)
    dY, X = _x(M, 128, 6), _x(M, 256, 7)
    off = _offsets(counts)
    qa, sa = quant_act_128x1_T_grouped(dY, off)
    qb, sb = quant_act_128x1_T_grouped(X, off)
    ref, _ = grouped_wgrad_ref(qa, sa, qb, sb, off)
    for e in range(len(counts)):
        r = slice(off[e], off[e + 1])
        exact = dY[r].astype(np.float64).T @ X[r].astype(np.float64)
        mag = np.abs(dY[r]).astype(np.float64).T @ np.abs(X[r]).astype(np.float64)
        assert np.all(np.abs(ref[e] - exact) <= (2 * 2.0 ** -4 + 2.0 ** -8) * mag + 1e-30)
    with pytest.raises(ValueError):
        quant_act_128x1_T_grouped(dY, [0, 5])
