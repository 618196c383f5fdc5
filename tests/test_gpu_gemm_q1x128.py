"""GPU parity of the GEMM with the fused quantizing epilogues.

fp8_gemm_blockscaled_q1x128 must write exactly the oracle's 1x128
quantization (codes and scales, bit for bit) of the BF16 result that
fp8_gemm_blockscaled writes for the same operands, and
fp8_gemm_blockscaled_q1x128_q128x1T also the oracle's transposed 128x1
quantization of it; that BF16 result is held to the oracle GEMM's acceptance
bound here as well, so each pair pins the fused output to the oracle without
any GPU quantizer in between.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_codes_equal, assert_scales_equal, bf16_bits, u8
from oracle.gemm import MODE_BLOCK, MODE_ROW

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B          # no NaN codes
    return c


def _scales(shape, seed, lo=1e-3, hi=1.0):
    g = torch.Generator().manual_seed(seed)
    return (lo + (hi - lo) * torch.rand(shape, generator=g)).to(torch.float32)


def _sb_shape(mode, N, K):
    return (N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N)


def _fused_vs_oracle(dev, A, sA, B, sB, mode, what, rows=None):
    """Run both entry points; check C against the oracle GEMM and Q/sQ against
    the oracle quantization of C (all rows, or the given sample)."""
    args = (A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode)
    C = fb.fp8_gemm_blockscaled(*args)
    Q, sQ = fb.fp8_gemm_blockscaled_q1x128(*args)
    torch.cuda.synchronize()
    M, N = C.shape
    assert Q.shape == (M, N) and sQ.shape == (N // 128, M)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    if rows is None:
        ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode)
    else:
        ref, absref = oracle.gemm_ref_rows(u8(A), sA.cpu().numpy(), u8(B), sB.cpu().numpy(), mode,
                                           rows=sel)
    ok, worst = oracle.check_gemm(bf16_bits(C[sel]), ref, absref)
    assert ok.all(), f"{what}: BF16 result outside the bound (worst {worst:.3g})"
    qo, so = oracle.quant_act_1x128(bf16_bits(C[sel]))
    assert_codes_equal(u8(Q[sel]), qo, f"{what}: fused codes")
    assert_scales_equal(sQ[:, sel].cpu().numpy(), so, f"{what}: fused scales")
    return C, Q, sQ


SHAPES = [(1, 128, 128), (16, 128, 256), (17, 256, 384), (256, 256, 128), (255, 512, 1024),
          (300, 384, 640), (513, 640, 256), (1024, 1280, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_fused_q1x128_random_codes(dev, M, N, K, mode):
    A, B = _codes((M, K), 2 * M + N + K), _codes((N, K), 13 + M + 3 * N + K)
    sA = _scales((K // 128, M), 7 + M)
    sB = _scales(_sb_shape(mode, N, K), 17 + N)
    _fused_vs_oracle(dev, A, sA, B, sB, mode, f"fused {M}x{N}x{K} mode {mode}")


# Shapes for which the fused entry point picks each of its tiles on a 256-CU
# MI355X (the dense GEMM's time estimate over 256x256, 224x256, 128x256 and
# 128x128 four deep; the shapes above all take 128x128): rows of every
# 16-row band checked, both scale modes.
FUSED_TILE_SHAPES = [(64, 2048, 1024),     # 128x128, four deep
                     (1600, 2560, 512),    # 128x256 (last m-tile 64 rows)
                     (4096, 4096, 256),    # 256x256
                     (7168, 2048, 256)]    # 224x256


@pytest.mark.parametrize("M,N,K", FUSED_TILE_SHAPES)
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_fused_q1x128_every_tile(dev, M, N, K, mode):
    A, B = _codes((M, K), 5 * M + N + K + mode), _codes((N, K), 31 + M + 7 * N + K)
    sA = _scales((K // 128, M), 11 + M)
    sB = _scales(_sb_shape(mode, N, K), 19 + N)
    rows = sorted({min(16 * b + (5 * b) % 16, M - 1) for b in range(-(-M // 16))})
    _fused_vs_oracle(dev, A, sA, B, sB, mode, f"fused {M}x{N}x{K} mode {mode}", rows=rows)


def test_fused_q1x128_zero_groups(dev):
    # zero rows of A and a zero 128-column block of B give all-zero groups of
    # C: codes +0 and scale 1.0; a single nonzero column gives a group whose
    # amax sits in one element
    M, N, K = 300, 512, 256
    A, B = _codes((M, K), 1), _codes((N, K), 2)
    A[5] = 0
    A[290:] = 0
    B[128:256] = 0
    B[384:511] = 0                       # group 3 keeps only column 511
    sA, sB = _scales((K // 128, M), 3), _scales((N // 128, K // 128), 4)
    C, Q, sQ = _fused_vs_oracle(dev, A, sA, B, sB, MODE_BLOCK, "fused zero groups")
    assert torch.all(sQ[1] == 1.0) and torch.all(sQ[:, 5] == 1.0)
    assert torch.all(Q[:, 128:256] == 0)


def test_fused_q1x128_wide_range(dev):
    # scales spread over 2^-40 .. 2^40 per row and per block, so group amaxes
    # span most of the FP32 range the 1x128 scales can take
    M, N, K = 256, 384, 512
    A, B = _codes((M, K), 21), _codes((N, K), 22)
    g = torch.Generator().manual_seed(23)
    sA = torch.pow(2.0, torch.randint(-40, 41, (K // 128, M), generator=g).float())
    sB = torch.pow(2.0, torch.randint(-20, 21, (N // 128, K // 128), generator=g).float())
    _fused_vs_oracle(dev, A, sA, B, sB, MODE_BLOCK, "fused wide scale range")


def test_fused_q1x128_dense_fprop_sampled(dev):
    # the 4096x7168x7168 layer whose output feeds the next layer's GEMM
    d = workloads.dense_fprop(device=dev)
    qx, sx = fb.fp8_quant_act_1x128(d["X"])
    qw, sw = fb.fp8_quant_w_128x128(d["W"])
    C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw)
    Q, sQ = fb.fp8_gemm_blockscaled_q1x128(qx, sx, qw, sw)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 2047, 3071, 4000, 4095])
    qo, so = oracle.quant_act_1x128(bf16_bits(C[rows]))
    assert_codes_equal(u8(Q[rows]), qo, "dense fprop fused codes, sampled rows")
    assert_scales_equal(sQ[:, rows].cpu().numpy(), so, "dense fprop fused scales, sampled rows")
    ref, absref = oracle.gemm_ref_rows(u8(qx), sx.cpu().numpy(), u8(qw), sw.cpu().numpy(), MODE_BLOCK,
                                       rows=rows)
    ok, worst = oracle.check_gemm(bf16_bits(C[rows]), ref, absref)
    assert ok.all(), f"dense fprop BF16 result outside the bound (worst {worst:.3g})"
    # every row: the fused output is the two-kernel path's output
    q2, s2 = fb.fp8_quant_act_1x128(C)
    assert torch.equal(Q, q2)
    assert torch.equal(sQ.view(torch.int32), s2.view(torch.int32))


def test_fused_q1x128_empty_m(dev):
    Q, sQ = fb.fp8_gemm_blockscaled_q1x128(torch.zeros((0, 128), dtype=torch.uint8, device=dev),
                                           torch.zeros((1, 0), device=dev),
                                           torch.zeros((256, 128), dtype=torch.uint8, device=dev),
                                           torch.ones((2, 1), device=dev))
    assert Q.shape == (0, 256) and sQ.shape == (2, 0)


def test_fused_q1x128_rejects_bad_arguments(dev):
    A = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    s = torch.ones((1, 128), device=dev)
    B = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    sB = torch.ones((1, 1), device=dev)
    L = fb.lib()
    p = [t.data_ptr() for t in (A, s, B, sB)]
    Q = torch.empty((128, 128), dtype=torch.uint8, device=dev)
    sQ = torch.empty((1, 128), device=dev)
    assert L.fp8_gemm_blockscaled_q1x128(*p, 7, Q.data_ptr(), sQ.data_ptr(), 128, 128, 128, None) != 0
    assert L.fp8_gemm_blockscaled_q1x128(*p, 0, None, sQ.data_ptr(), 128, 128, 128, None) != 0
    assert L.fp8_gemm_blockscaled_q1x128(*p, 0, Q.data_ptr(), None, 128, 128, 128, None) != 0
    assert L.fp8_gemm_blockscaled_q1x128(*p, 0, Q.data_ptr(), sQ.data_ptr(), 128, 100, 128, None) != 0
    assert L.fp8_gemm_blockscaled_q1x128(*p, 0, Q.data_ptr() + 1, sQ.data_ptr(), 128, 128, 128,
                                         None) != 0
    assert L.fp8_gemm_blockscaled_q1x128(*p, 0, Q.data_ptr(), sQ.data_ptr(), 128, 128, 128, None) == 0


# ---------------------------------------------------------------------------
# both layouts: 1x128 and the transposed 128x1 copy (M a multiple of 128)
# ---------------------------------------------------------------------------

def _both_vs_oracle(dev, A, sA, B, sB, mode, what):
    args = (A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode)
    C = fb.fp8_gemm_blockscaled(*args)
    Q, sQ, QT, sQT = fb.fp8_gemm_blockscaled_q1x128_q128x1T(*args)
    torch.cuda.synchronize()
    M, N = C.shape
    assert QT.shape == (N, M) and sQT.shape == (M // 128, N)
    ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode)
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    assert ok.all(), f"{what}: BF16 result outside the bound (worst {worst:.3g})"
    qo, so = oracle.quant_act_1x128(bf16_bits(C))
    assert_codes_equal(u8(Q), qo, f"{what}: 1x128 codes")
    assert_scales_equal(sQ.cpu().numpy(), so, f"{what}: 1x128 scales")
    qto, sto = oracle.quant_act_128x1_T(bf16_bits(C))
    assert_codes_equal(u8(QT), qto, f"{what}: 128x1 transposed codes")
    assert_scales_equal(sQT.cpu().numpy(), sto, f"{what}: 128x1 scales")


# these shapes take the 128x128 tiles of 8 waves of 128 rows; the full-size
# layer below takes 256x256
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 256, 384), (384, 640, 256), (1024, 1280, 512),
                                   (640, 384, 1024)])
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_fused_both_layouts_random_codes(dev, M, N, K, mode):
    A, B = _codes((M, K), 5 * M + N + K), _codes((N, K), 17 + M + 2 * N + K)
    sA = _scales((K // 128, M), 3 + M)
    sB = _scales(_sb_shape(mode, N, K), 11 + N)
    _both_vs_oracle(dev, A, sA, B, sB, mode, f"both layouts {M}x{N}x{K} mode {mode}")


def test_fused_both_layouts_zero_and_wide(dev):
    M, N, K = 384, 512, 256
    A, B = _codes((M, K), 31), _codes((N, K), 32)
    A[128:256] = 0                        # a zero 128-row group for every column
    B[200] = 0                            # one zero column
    g = torch.Generator().manual_seed(33)
    sA = torch.pow(2.0, torch.randint(-30, 31, (K // 128, M), generator=g).float())
    sB = torch.pow(2.0, torch.randint(-10, 11, (N // 128, K // 128), generator=g).float())
    _both_vs_oracle(dev, A, sA, B, sB, MODE_BLOCK, "both layouts, zero groups and wide scales")


def test_fused_both_layouts_dense_fprop(dev):
    d = workloads.dense_fprop(device=dev)
    qx, sx = fb.fp8_quant_act_1x128(d["X"])
    qw, sw = fb.fp8_quant_w_128x128(d["W"])
    C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw)
    Q, sQ, QT, sQT = fb.fp8_gemm_blockscaled_q1x128_q128x1T(qx, sx, qw, sw)
    q2, s2 = fb.fp8_quant_act_1x128(C)
    qt2, st2 = fb.fp8_quant_act_128x1_T(C)
    torch.cuda.synchronize()
    assert torch.equal(Q, q2) and torch.equal(sQ.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(QT, qt2) and torch.equal(sQT.view(torch.int32), st2.view(torch.int32))
    # and one 128-row group of columns against the oracle directly
    qto, sto = oracle.quant_act_128x1_T(bf16_bits(C[256:384]))
    assert_codes_equal(u8(QT[:, 256:384]), qto, "dense fprop 128x1 codes, rows 256..383")
    assert_scales_equal(sQT[2:3].cpu().numpy(), sto, "dense fprop 128x1 scales, rows 256..383")


def test_fused_both_layouts_rejects_ragged_m(dev):
    A = torch.zeros((100, 128), dtype=torch.uint8, device=dev)
    sA = torch.ones((1, 100), device=dev)
    B = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    sB = torch.ones((1, 1), device=dev)
    with pytest.raises(fb.Fp8bsError):
        fb.fp8_gemm_blockscaled_q1x128_q128x1T(A, sA, B, sB)
