"""Accumulation precision of the gfx950 FP8 MFMA inside one 128-wide K chunk
(informational; the DeepSeek-V3 report section 3.3.2, on the innerforce.co.kr
page, measures about 14 bits for H800 tensor cores and promotes every 128
elements for that reason).

Each experiment is one K = 128 dot product with three non-zero products: a
cancelling pair +448*448 and -448*448 at K positions i and j, and a small
power of two 2^e at position p. The exact sum is 2^e, which BF16 holds
exactly, so the block-scaled GEMM's BF16 output shows whether the small term
survived the matrix unit's internal summation: an accumulator of W bits
aligned to the largest term loses it once 448^2 / 2^e exceeds about 2^W. The
experiments sit on the diagonal of one GEMM (row m of A and row m of B form
experiment m; off-diagonal outputs only go through the acceptance bound).
The assertion is the acceptance bound; the survival table is printed."""

import numpy as np
import pytest
import torch

import oracle
from helpers import bf16_bits

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu

E_SMALL = list(range(-18, 17))   # exponent of the small product
PER = 128                        # experiments per exponent


def _code_pow2(e):
    """E4M3 code of 2^e, e in [-9, 8]."""
    if e >= -6:
        return (e + 7) << 3
    return {-7: 0x04, -8: 0x02, -9: 0x01}[e]


def _build(seed=0):
    rng = np.random.default_rng(seed)
    n = len(E_SMALL) * PER
    A = np.zeros((n, 128), np.uint8)
    B = np.zeros((n, 128), np.uint8)
    pos = np.zeros((n, 3), np.int64)
    for b, e in enumerate(E_SMALL):
        ea = max(-9, e - 8)
        eb = e - ea
        for t in range(PER):
            m = b * PER + t
            i, j, p = rng.choice(128, 3, replace=False)
            A[m, i] = A[m, j] = 0x7E            # 448
            B[m, i], B[m, j] = 0x7E, 0xFE       # +448, -448
            A[m, p], B[m, p] = _code_pow2(ea), _code_pow2(eb)
            pos[m] = (i, j, p)
    return A, B, pos


def test_mfma_chunk_accumulation_probe(dev):
    A, B, pos = _build()
    n = A.shape[0]
    sA = np.ones((1, n), np.float32)
    sB = np.ones((n // 128, 1), np.float32)
    C = fb.fp8_gemm_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(sA).to(dev),
                                torch.from_numpy(B).to(dev), torch.from_numpy(sB).to(dev))
    torch.cuda.synchronize()
    ref, absref = oracle.gemm_ref(A, sA, B, sB, oracle.gemm.MODE_BLOCK)
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    assert ok.all(), f"probe GEMM outside the acceptance bound (worst {worst:.3g})"

    got = oracle.bf16_bits_to_f64(bf16_bits(C.diagonal().contiguous()))
    lines = ["log2(448^2 / small)  exact  zero  other  (of %d)" % PER]
    for b, e in enumerate(E_SMALL):
        g = got[b * PER:(b + 1) * PER]
        exact = int(np.sum(g == 2.0 ** e))
        zero = int(np.sum(g == 0.0))
        lines.append("%19.2f  %5d  %4d  %5d" % (np.log2(448.0 ** 2) - e, exact, zero, PER - exact - zero))
    # Where the ratio is between 2^15 and 2^24 (an FP32 sum would keep the
    # small term): losses against the K positions, for aligned K blocks of
    # g products holding the small term together with exactly one of the pair.
    lost = got != 2.0 ** np.repeat(E_SMALL, PER)
    ratio = np.log2(448.0 ** 2) - np.repeat(E_SMALL, PER)
    mid = (ratio > 15) & (ratio < 24)
    lines.append(f"ratio 2^15 .. 2^24: {int((lost & mid).sum())} of {int(mid.sum())} small terms lost")
    for gsz in (2, 4, 8, 16, 32, 64):
        bi, bj, bp = pos[:, 0] // gsz, pos[:, 1] // gsz, pos[:, 2] // gsz
        one = (bp == bi) ^ (bp == bj)
        lines.append(f"  small term in a {gsz:2d}-wide K block with one of the pair: lost "
                     f"{int((lost & mid & one).sum())} of {int((mid & one).sum())}; otherwise lost "
                     f"{int((lost & mid & ~one).sum())} of {int((mid & ~one).sum())}")
    print("\n" + "\n".join(lines))
