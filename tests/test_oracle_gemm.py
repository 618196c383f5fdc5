"""Pins for the oracle's block-scaled GEMM reference and acceptance bound.

Checked against: exact integer matmul (every E4M3 value times 2^9 is an
integer), an exact rational (Fraction) computation on a tiny case with
arbitrary float32 scales in both scale modes, torch's float64 matmul of
torch-decoded codes for the single-chunk case, the all-code-pairs table, and
the per-expert decomposition of the grouped form. A planted mistake (wrong
scale index, transposed operand, dropped chunk) is shown to fail the bound.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import (bf16_ulp, check_gemm, e4m3_decode, gemm_ref, gemm_ref_rows,
                    grouped_gemm_ref)
from oracle.gemm import MODE_BLOCK, MODE_ROW


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x00
    return c


def _int_values(codes):
    """E4M3 value * 2^9 as exact int64, decoded by torch (independent decode)."""
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64) * 512
    out = v.numpy()
    assert np.all(out == np.round(out))
    return out.astype(np.int64)


def _f32_bits_to_frac(x):
    return Fraction(float(np.float32(x)))


def test_integer_matmul_pin_block_mode():
    rng = np.random.default_rng(10)
    M, N, K = 37, 256, 384
    A, B = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    ea = rng.integers(-3, 4, (K // 128, M))
    eb = rng.integers(-3, 4, (N // 128, K // 128))
    sA = (2.0 ** ea).astype(np.float32)
    sB = (2.0 ** eb).astype(np.float32)
    ref, _ = gemm_ref(A, sA, B, sB, MODE_BLOCK)
    ia, ib = _int_values(A), _int_values(B)
    exact = np.zeros((M, N), np.float64)
    for kb in range(K // 128):
        ks = slice(kb * 128, kb * 128 + 128)
        P = ia[:, ks] @ ib[:, ks].T                     # int64, exact
        scale = 2.0 ** (ea[kb][:, None] + eb[np.arange(N) // 128, kb][None, :])
        exact += scale * P.astype(np.float64) * 2.0 ** -18
    assert np.array_equal(ref, exact)


def test_integer_matmul_pin_row_mode():
    rng = np.random.default_rng(11)
    M, N, K = 19, 45, 256
    A, B = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    ea = rng.integers(-2, 3, (K // 128, M))
    eb = rng.integers(-2, 3, (K // 128, N))
    ref, _ = gemm_ref(A, (2.0 ** ea).astype(np.float32), B, (2.0 ** eb).astype(np.float32), MODE_ROW)
    ia, ib = _int_values(A), _int_values(B)
    exact = np.zeros((M, N))
    for kb in range(K // 128):
        ks = slice(kb * 128, kb * 128 + 128)
        exact += 2.0 ** (ea[kb][:, None] + eb[kb][None, :]) * (ia[:, ks] @ ib[:, ks].T) * 2.0 ** -18
    assert np.array_equal(ref, exact)


def _fraction_gemm(A, sA, B, sB, mode, rows, cols):
    K = A.shape[1]
    dA = [[Fraction(float(v)) for v in r] for r in e4m3_decode(A[rows])]
    dB = [[Fraction(float(v)) for v in r] for r in e4m3_decode(B[cols])]
    out = []
    for i, m in enumerate(rows):
        row = []
        for j, n in enumerate(cols):
            total = Fraction(0)
            for kb in range(K // 128):
                p = sum(dA[i][k] * dB[j][k] for k in range(kb * 128, kb * 128 + 128))
                sa = _f32_bits_to_frac(sA[kb][m])
                sb = _f32_bits_to_frac(sB[n // 128][kb] if mode == MODE_BLOCK else sB[kb][n])
                total += sa * sb * p
            row.append(total)
        out.append(row)
    return out


def test_fraction_pin_arbitrary_scales_both_modes():
    rng = np.random.default_rng(12)
    M, N, K = 5, 256, 384
    A, B = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sA = rng.uniform(1e-3, 3, (K // 128, M)).astype(np.float32)
    rows = np.array([0, 2, 4])
    cols = np.array([0, 1, 127, 128, 200, 255])
    for mode, sB in ((MODE_BLOCK, rng.uniform(1e-4, 1, (N // 128, K // 128)).astype(np.float32)),
                     (MODE_ROW, rng.uniform(1e-4, 1, (K // 128, N)).astype(np.float32))):
        ref, absref = gemm_ref_rows(A, sA, B, sB, mode, rows=rows, cols=cols)
        exact = _fraction_gemm(A, sA, B, sB, mode, rows, cols)
        for i in range(len(rows)):
            for j in range(len(cols)):
                e = exact[i][j]
                # per chunk: the scale product of two float32 is exact in float64, the
                # chunk sum is exact, so only the scaling and the chunk sum round: a few
                # float64 ulps of the magnitude sum
                assert abs(Fraction(ref[i, j]) - e) <= Fraction(absref[i, j]) * Fraction(1, 2 ** 50)
                assert absref[i, j] >= abs(ref[i, j])


def test_single_chunk_unit_scale_is_plain_matmul():
    rng = np.random.default_rng(13)
    A, B = _rand_codes(rng, (64, 128)), _rand_codes(rng, (128, 128))
    ref, absref = gemm_ref(A, np.ones((1, 64), np.float32), B, np.ones((1, 1), np.float32))
    ta = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float64)
    tb = torch.from_numpy(B).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.array_equal(ref, (ta @ tb.T).numpy())
    assert np.array_equal(absref, (ta.abs() @ tb.abs().T).numpy())


def test_all_code_pairs():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    A = np.repeat(codes[:, None], 128, axis=1)
    B = np.zeros((256, 128), np.uint8)
    B[:254] = A
    ref, _ = gemm_ref(A, np.ones((1, 254), np.float32), B, np.ones((2, 1), np.float32))
    v = _int_values(codes)
    exact = 128.0 * np.outer(v, v).astype(np.float64) * 2.0 ** -18
    assert np.array_equal(ref[:, :254], exact)
    assert np.all(ref[:, 254:] == 0)


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(14)
    counts = [0, 5, 130, 1, 0, 17]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M, N, K, E = int(off[-1]), 128, 256, len(counts)
    A = _rand_codes(rng, (M, K))
    sA = rng.uniform(0.1, 2, (K // 128, M)).astype(np.float32)
    B = _rand_codes(rng, (E, N, K))
    sB = rng.uniform(0.1, 2, (E, N // 128, K // 128)).astype(np.float32)
    ref, absref = grouped_gemm_ref(A, sA, B, sB, off)
    for e in range(E):
        r = slice(off[e], off[e + 1])
        if off[e] == off[e + 1]:
            continue
        d, da = gemm_ref(A[r], sA[:, r], B[e], sB[e])
        assert np.array_equal(ref[r], d) and np.array_equal(absref[r], da)
    # and each expert's rows use only that expert's weights: integer pin on expert 2
    ia, ib = _int_values(A[5:135]), _int_values(B[2])
    sa = sA[:, 5:135].astype(np.float64)
    exact = sum(sa[kb][:, None] * sB[2][0, kb] * (ia[:, kb * 128:(kb + 1) * 128] @ ib[:, kb * 128:(kb + 1) * 128].T)
                * 2.0 ** -18 for kb in range(2))
    assert np.allclose(ref[5:135], exact, rtol=1e-14, atol=0)


def _bf16_rne_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bound_accepts_rounded_result_and_rejects_planted_mistakes():
    rng = np.random.default_rng(15)
    M, N, K = 64, 256, 512
    A, B = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sA = rng.uniform(0.01, 1, (K // 128, M)).astype(np.float32)
    sB = rng.uniform(0.01, 1, (N // 128, K // 128)).astype(np.float32)
    ref, absref = gemm_ref(A, sA, B, sB)
    # an FP32 accumulation in a different order, then BF16 RNE, passes
    ok, worst = check_gemm(_bf16_rne_bits(ref.astype(np.float32)), ref, absref)
    assert ok.all() and worst <= 1.0
    # planted mistakes fail on a large fraction of elements
    wrong_scale, _ = gemm_ref(A, sA[::-1].copy(), B, sB)                  # chunk order of sA reversed
    wrong_t, _ = gemm_ref(A, sA, B, np.ascontiguousarray(sB[::-1]))      # weight-block rows swapped
    dropped, _ = gemm_ref(A[:, :384], sA[:3], B[:, :384], sB[:, :3].copy())  # last chunk missing
    for bad in (wrong_scale, wrong_t, dropped):
        ok, _ = check_gemm(_bf16_rne_bits(bad.astype(np.float32)), ref, absref)
        assert ok.mean() < 0.5


def test_bf16_ulp_values():
    y = np.array([1.0, 1.5, -3.0, 2.0 ** -126, 2.0 ** -130, 0.0, 448.0])
    expect = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133, 2.0 ** 1])
    assert np.array_equal(bf16_ulp(y), expect)


def test_bf16_rounding_within_one_ulp_bound():
    rng = np.random.default_rng(16)
    y = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float64)
    c = _bf16_rne_bits(y.astype(np.float32))
    ok, _ = check_gemm(c, y, np.zeros_like(y))
    assert ok.all()
    # a 2-ulp error is rejected when absref is zero
    c2 = (c.astype(np.int32) + 2).astype(np.uint16)
    ok2, _ = check_gemm(c2, y, np.zeros_like(y))
    assert not ok2.any()
