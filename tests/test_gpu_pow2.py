"""GPU parity of the power-of-two scale variant: the three _pow2 quantizers
bit for bit against the oracle's pow2 rule, and the hardware-scaled GEMM
(E8M0 operand scales applied by the MFMA) within the GEMM acceptance bound;
plus its accuracy next to the FP32-scale path on the dense Fprop layer."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import adversarial_rows, assert_codes_equal, assert_scales_equal, bf16_bits, to_oracle, u8
from oracle.gemm import MODE_BLOCK, MODE_ROW

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _rand(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[0], 1, generator=g) * 3)
    if shape[1] > 8:
        x[:, 3] *= 100
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,K", [(1, 128), (5, 1024), (130, 384), (257, 640)])
def test_pow2_quant_act(dev, dtype, M, K):
    x = _rand((M, K), M + K, dtype)
    q, s = fb.fp8_quant_act_1x128(x.to(dev), pow2=True)
    qo, so = oracle.quant_act_1x128(to_oracle(x), pow2=True)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "pow2 1x128 codes")
    assert_scales_equal(s.cpu().numpy(), so, "pow2 1x128 scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pow2_quant_act_adversarial(dev, dtype):
    x = torch.from_numpy(adversarial_rows(41, 1280, seed=7)).to(dtype)
    q, s = fb.fp8_quant_act_1x128(x.to(dev), pow2=True)
    qo, so = oracle.quant_act_1x128(to_oracle(x), pow2=True)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "pow2 1x128 adversarial codes")
    assert_scales_equal(s.cpu().numpy(), so, "pow2 1x128 adversarial scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,K", [(128, 128), (256, 384)])
def test_pow2_quant_w(dev, dtype, N, K):
    w = _rand((N, K), N * K, dtype)
    q, s, qT, sT = fb.fp8_quant_w_128x128(w.to(dev), transposed=True, pow2=True)
    qo, so = oracle.quant_w_128x128(to_oracle(w), pow2=True)
    torch.cuda.synchronize()
    assert_codes_equal(u8(q), qo, "pow2 128x128 codes")
    assert_scales_equal(s.cpu().numpy(), so, "pow2 128x128 scales")
    assert_codes_equal(u8(qT), qo.T, "pow2 128x128 transposed codes")
    assert_scales_equal(sT.cpu().numpy(), so.T, "pow2 128x128 transposed scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,C", [(128, 64), (256, 63), (384, 130)])
def test_pow2_quant_128x1_T(dev, dtype, M, C):
    x = _rand((M, C), M + C, dtype)
    qT, sT = fb.fp8_quant_act_128x1_T(x.to(dev), pow2=True)
    qo, so = oracle.quant_act_128x1_T(to_oracle(x), pow2=True)
    torch.cuda.synchronize()
    assert_codes_equal(u8(qT), qo, "pow2 128x1 codes")
    assert_scales_equal(sT.cpu().numpy(), so, "pow2 128x1 scales")


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B
    return c


def _pow2_scales(shape, seed, lo=-20, hi=6):
    g = torch.Generator().manual_seed(seed)
    return torch.pow(2.0, torch.randint(lo, hi, shape, generator=g).float())


def _check(C, ref, absref, what):
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        c = oracle.bf16_bits_to_f64(bf16_bits(C))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound (worst {worst:.3g}); "
                             f"first at {i}: got {c[i]!r}, ref {ref[i]!r}")
    return worst


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 256, 384), (255, 512, 1024), (300, 384, 640),
                                   (513, 640, 256), (1024, 1280, 512)])
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_pow2_gemm_random_codes(dev, M, N, K, mode):
    A, B = _codes((M, K), 3 * M + N + K), _codes((N, K), M + 5 * N + K)
    sA = _pow2_scales((K // 128, M), M + 1)
    sB = _pow2_scales((N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N), N + 2)
    C = fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode, pow2=True)
    ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"pow2 gemm {M}x{N}x{K} mode {mode}")


# shapes for which the power-of-two GEMM picks each of its kernels on a
# 256-CU MI355X (its time estimate over 256x256 four-wave tiles and the
# four-deep 128x128 and 64x64 ones); rows of every 16-row band checked
@pytest.mark.parametrize("M,N,K", [(1000, 2048, 512),     # 64x64, four deep (ragged last m-tile)
                                   (2000, 2048, 512),     # 128x128, four deep (ragged last m-tile)
                                   (4096, 4096, 256)])    # 256x256, four waves
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_pow2_gemm_every_tile(dev, M, N, K, mode):
    A, B = _codes((M, K), 7 * M + N + K + mode), _codes((N, K), M + 11 * N + K)
    sA = _pow2_scales((K // 128, M), M + 3)
    sB = _pow2_scales((N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N), N + 4)
    C = fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode, pow2=True)
    rows = np.array(sorted({min(16 * b + (3 * b) % 16, M - 1) for b in range(-(-M // 16))}))
    ref, absref = oracle.gemm_ref_rows(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode, rows=rows)
    torch.cuda.synchronize()
    _check(C[rows], ref, absref, f"pow2 gemm {M}x{N}x{K} mode {mode}")


def test_pow2_gemm_extreme_scales(dev):
    # scales near both ends of the E8M0 range the quantizers produce
    M, N, K = 256, 256, 512
    A, B = _codes((M, K), 1), _codes((N, K), 2)
    sA = _pow2_scales((K // 128, M), 3, lo=-126, hi=-100)
    sB = _pow2_scales((N // 128, K // 128), 4, lo=95, hi=110)
    C = fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), MODE_BLOCK, pow2=True)
    ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), MODE_BLOCK)
    torch.cuda.synchronize()
    _check(C, ref, absref, "pow2 gemm extreme scales")


def test_pow2_backward_pair_sampled(dev):
    d = workloads.backward_pair(device=dev)
    qdy, sdy = fb.fp8_quant_act_1x128(d["dY"], pow2=True)
    _, _, qwT, swT = fb.fp8_quant_w_128x128(d["W"], transposed=True, pow2=True)
    dX = fb.fp8_gemm_blockscaled(qdy, sdy, qwT, swT, fb.SCALE_BLOCK128, pow2=True)
    qdyT, sdyT = fb.fp8_quant_act_128x1_T(d["dY"], pow2=True)
    qxT, sxT = fb.fp8_quant_act_128x1_T(d["X"], pow2=True)
    dW = fb.fp8_gemm_blockscaled(qdyT, sdyT, qxT, sxT, fb.SCALE_ROW, pow2=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 4000, 4095])
    ref, absref = oracle.gemm_ref_rows(u8(qdy), sdy.cpu().numpy(), u8(qwT), swT.cpu().numpy(), MODE_BLOCK, rows=rows)
    _check(dX[rows], ref, absref, "pow2 dgrad sampled")
    rows = np.array([0, 5, 7167])
    ref, absref = oracle.gemm_ref_rows(u8(qdyT), sdyT.cpu().numpy(), u8(qxT), sxT.cpu().numpy(), MODE_ROW, rows=rows)
    _check(dW[rows], ref, absref, "pow2 wgrad sampled")


def test_pow2_accuracy_next_to_fp32_scales(dev):
    # dense Fprop 4096x7168x7168: error of each path against the exact product
    # of the BF16 inputs, on sampled rows, relative to sum |x||w|
    d = workloads.dense_fprop(device=dev)
    rows = np.array([0, 1, 77, 2048, 4095])
    out = {}
    for pow2 in (False, True):
        qx, sx = fb.fp8_quant_act_1x128(d["X"], pow2=pow2)
        qw, sw = fb.fp8_quant_w_128x128(d["W"], pow2=pow2)
        C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw, pow2=pow2)
        torch.cuda.synchronize()
        ref, absref = oracle.gemm_ref_rows(u8(qx), sx.cpu().numpy(), u8(qw), sw.cpu().numpy(), MODE_BLOCK, rows=rows)
        _check(C[rows], ref, absref, f"dense fprop pow2={pow2}")
        out[pow2] = oracle.bf16_bits_to_f64(bf16_bits(C[rows]))
    X = d["X"][rows].double().cpu()
    W = d["W"].double().cpu()
    exact = (X @ W.T).numpy()
    mag = (X.abs() @ W.abs().T).numpy()
    e32 = np.abs(out[False] - exact) / mag
    e2 = np.abs(out[True] - exact) / mag
    print(f"relative error vs exact: fp32 scales median {np.median(e32):.3e} max {e32.max():.3e}; "
          f"pow2 scales median {np.median(e2):.3e} max {e2.max():.3e}")
    assert np.median(e2) <= 1.5 * np.median(e32) and e2.max() <= 2.0 * e32.max()
