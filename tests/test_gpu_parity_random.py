"""Randomized GPU parity: seeded random shapes, modes, dtypes and value ranges
against the oracle, beyond the hand-picked cases of the other files.

* Dense GEMM: M in 1..1199, N and K multiples of 128 up to 1,536, both scale
  modes, codes over the whole E4M3 range, scales spread over 2^-8 .. 2^8;
  the whole NaN-prefilled output is checked.
* Grouped GEMM: 1..16 experts whose row counts mix empty, small (<= 32),
  medium and past-one-pass (> 256) experts, so both the weight-streaming and
  the tile kernel run, alone and together; the whole output is checked.
* Quantizers: 1x128 (any M, F32 or BF16), 128x128 (with and without the
  transposed copy) and 128x1 transposed (any C) on values whose magnitude
  varies per column and per row, with outliers, bit for bit.

Acceptance bound for the GEMMs: |C - ref| <= 4e-3 * sum_k |a_k b_k| + ulp_bf16(ref).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_codes_equal, assert_scales_equal, bf16_bits, to_oracle, u8
from oracle.gemm import MODE_BLOCK

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B          # no NaN codes
    return c


def _scales(rng, shape):
    return np.exp2(rng.uniform(-8.0, 8.0, shape)).astype(np.float32)


def _check(C, ref, absref, what):
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        c = oracle.bf16_bits_to_f64(bf16_bits(C))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound "
                             f"(worst {worst:.3g}); first at {i}: got {c[i]!r}, ref {ref[i]!r}")


@pytest.mark.parametrize("seed", range(120))
def test_random_dense_gemm(dev, seed):
    rng = np.random.default_rng(7000 + seed)
    M = int(rng.integers(1, 1200))
    N = 128 * int(rng.integers(1, 13))
    K = 128 * int(rng.integers(1, 13))
    mode = int(rng.integers(0, 2))
    A, B = _codes(rng, (M, K)), _codes(rng, (N, K))
    sA = _scales(rng, (K // 128, M))
    sB = _scales(rng, (N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N))
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(sA).to(dev), torch.from_numpy(B).to(dev),
                            torch.from_numpy(sB).to(dev), mode, out=C)
    ref, absref = oracle.gemm_ref(A, sA, B, sB, mode)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"seed {seed}: gemm {M}x{N}x{K} mode {mode}")


def _expert_counts(rng):
    E = int(rng.integers(1, 17))
    kind = rng.integers(0, 4, E)                       # empty, small, medium, past one 256-row pass
    counts = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 33, E),
                                             np.where(kind == 2, rng.integers(33, 257, E),
                                                      rng.integers(257, 600, E))))
    return counts.astype(np.int64)


@pytest.mark.parametrize("seed", range(48))
def test_random_grouped_gemm(dev, seed):
    rng = np.random.default_rng(8000 + seed)
    counts = _expert_counts(rng)
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M = int(off[-1])
    N = 128 * int(rng.integers(1, 6))
    K = 128 * int(rng.integers(1, 6))
    A, B = _codes(rng, (M, K)), _codes(rng, (E, N, K))
    sA, sB = _scales(rng, (K // 128, M)), _scales(rng, (E, N // 128, K // 128))
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(sA).to(dev),
                                    torch.from_numpy(B).to(dev), torch.from_numpy(sB).to(dev),
                                    torch.from_numpy(off).to(dev), out=C)
    if M == 0:
        return
    ref, absref = oracle.grouped_gemm_ref(A, sA, B, sB, off)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"seed {seed}: grouped counts {counts.tolist()} N={N} K={K}")


def _values(rng, shape, dtype):
    """Normals scaled per column (2^-20 .. 2^20) and per row (2^-6 .. 2^6), with
    a few outliers x1000 and some exact zeros."""
    x = rng.standard_normal(shape) * np.exp2(rng.uniform(-20, 20, (1, shape[1])))
    x *= np.exp2(rng.uniform(-6, 6, (shape[0], 1)))
    x.flat[rng.integers(0, x.size, max(1, x.size // 500))] *= 1000.0
    x.flat[rng.integers(0, x.size, max(1, x.size // 300))] = 0.0
    t = torch.from_numpy(x.astype(np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("seed", range(24))
def test_random_quant_act_1x128(dev, seed):
    rng = np.random.default_rng(9000 + seed)
    M, K = int(rng.integers(1, 1500)), 128 * int(rng.integers(1, 25))
    dtype = ("bf16", "f32")[seed % 2]
    X = _values(rng, (M, K), dtype)
    q, s = fb.fp8_quant_act_1x128(X.to(dev))
    qo, so = oracle.quant_act_1x128(to_oracle(X))
    assert_codes_equal(u8(q), qo, f"seed {seed}: 1x128 {M}x{K} {dtype} codes")
    assert_scales_equal(s.cpu().numpy(), so, f"seed {seed}: 1x128 {M}x{K} {dtype} scales")


@pytest.mark.parametrize("seed", range(24))
def test_random_quant_w_128x128(dev, seed):
    rng = np.random.default_rng(9100 + seed)
    N, K = 128 * int(rng.integers(1, 13)), 128 * int(rng.integers(1, 13))
    dtype = ("bf16", "f32")[seed % 2]
    transposed = bool(seed % 3 == 0)
    W = _values(rng, (N, K), dtype)
    out = fb.fp8_quant_w_128x128(W.to(dev), transposed=transposed)
    qo, so = oracle.quant_w_128x128(to_oracle(W))
    assert_codes_equal(u8(out[0]), qo, f"seed {seed}: 128x128 {N}x{K} {dtype} codes")
    assert_scales_equal(out[1].cpu().numpy(), so, f"seed {seed}: 128x128 {N}x{K} {dtype} scales")
    if transposed:
        assert_codes_equal(u8(out[2]), qo.T, f"seed {seed}: 128x128 {N}x{K} {dtype} transposed codes")
        assert_scales_equal(out[3].cpu().numpy(), so.T, f"seed {seed}: 128x128 {N}x{K} {dtype} transposed scales")


@pytest.mark.parametrize("seed", range(24))
def test_random_quant_act_128x1_T(dev, seed):
    rng = np.random.default_rng(9200 + seed)
    M, C = 128 * int(rng.integers(1, 13)), int(rng.integers(1, 1200))
    dtype = ("bf16", "f32")[seed % 2]
    X = _values(rng, (M, C), dtype)
    qT, sT = fb.fp8_quant_act_128x1_T(X.to(dev))
    qo, so = oracle.quant_act_128x1_T(to_oracle(X))
    assert_codes_equal(u8(qT), qo, f"seed {seed}: 128x1T {M}x{C} {dtype} codes")
    assert_scales_equal(sT.cpu().numpy(), so, f"seed {seed}: 128x1T {M}x{C} {dtype} scales")
