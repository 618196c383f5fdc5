"""GPU parity of the three quantizers against the CPU oracle: bit-exact codes
and bit-exact FP32 scales, through the C ABI (via the thin binding)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import adversarial_rows, assert_codes_equal, assert_scales_equal, to_oracle

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _rand(shape, seed, dtype, outliers=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[0], 1, generator=g) * 2)
    if outliers and shape[1] > 8:
        x[:, 3] *= 100
    return x.to(dtype)


def _check_act(x_cpu, dev, what):
    q, s = fb.fp8_quant_act_1x128(x_cpu.to(dev))
    qo, so = oracle.quant_act_1x128(to_oracle(x_cpu))
    torch.cuda.synchronize()
    assert_codes_equal(q.cpu().numpy(), qo, what + " codes")
    assert_scales_equal(s.cpu().numpy(), so, what + " scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (5, 1024), (130, 384), (257, 640), (64, 7168)])
def test_quant_act_1x128_shapes(dev, dtype, M, K):
    _check_act(_rand((M, K), M * 1000 + K, dtype), dev, f"1x128 {dtype} {M}x{K}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_act_1x128_adversarial(dev, dtype):
    x = torch.from_numpy(adversarial_rows(41, 1280, seed=3)).to(dtype)
    _check_act(x, dev, f"1x128 adversarial {dtype}")


def test_quant_act_1x128_tiny_fprop_workload(dev):
    d = workloads.tiny_fprop()
    _check_act(d["X"], dev, "1x128 tiny-fprop X")


def test_quant_act_1x128_dense_fprop_workload(dev):
    d = workloads.dense_fprop(device=dev)
    _check_act(d["X"].cpu(), dev, "1x128 dense-fprop X 4096x7168 bf16")


def _check_w(w_cpu, dev, what):
    q, s, qT, sT = fb.fp8_quant_w_128x128(w_cpu.to(dev), transposed=True)
    q2, s2 = fb.fp8_quant_w_128x128(w_cpu.to(dev))
    qo, so = oracle.quant_w_128x128(to_oracle(w_cpu))
    torch.cuda.synchronize()
    assert_codes_equal(q.cpu().numpy(), qo, what + " codes")
    assert_scales_equal(s.cpu().numpy(), so, what + " scales")
    assert_codes_equal(qT.cpu().numpy(), qo.T, what + " transposed codes")
    assert_scales_equal(sT.cpu().numpy(), so.T, what + " transposed scales")
    assert_codes_equal(q2.cpu().numpy(), qo, what + " codes (no transposed copy)")
    assert_scales_equal(s2.cpu().numpy(), so, what + " scales (no transposed copy)")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (384, 1024)])
def test_quant_w_128x128_shapes(dev, dtype, N, K):
    _check_w(_rand((N, K), N + K, dtype), dev, f"128x128 {dtype} {N}x{K}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_w_128x128_adversarial(dev, dtype):
    # one pattern per 128x128 block: build rows from adversarial groups, then
    # scale whole blocks so their amax patterns differ
    x = adversarial_rows(256, 1280, seed=5)
    x[:128, :128] = 0.0
    x[128:, 128:256] = -0.0
    _check_w(torch.from_numpy(x).to(dtype), dev, f"128x128 adversarial {dtype}")


def test_quant_w_128x128_tiny_fprop_workload(dev):
    _check_w(workloads.tiny_fprop()["W"], dev, "128x128 tiny-fprop W")


def test_quant_w_128x128_dense_weight(dev):
    w = workloads.dense_fprop(device=dev)["W"]
    q, s = fb.fp8_quant_w_128x128(w)
    rows = slice(3 * 128, 5 * 128)                        # two block rows, all 56 block columns
    qo, so = oracle.quant_w_128x128(to_oracle(w[rows]))
    torch.cuda.synchronize()
    assert_codes_equal(q[rows].cpu().numpy(), qo, "128x128 dense W rows 384..639")
    assert_scales_equal(s[3:5].cpu().numpy(), so, "128x128 dense W scales")


def _check_t(x_cpu, dev, what):
    qT, sT = fb.fp8_quant_act_128x1_T(x_cpu.to(dev))
    qo, so = oracle.quant_act_128x1_T(to_oracle(x_cpu))
    torch.cuda.synchronize()
    assert_codes_equal(qT.cpu().numpy(), qo, what + " codes")
    assert_scales_equal(sT.cpu().numpy(), so, what + " scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,C", [(128, 1), (128, 64), (256, 63), (384, 130), (256, 72), (128, 200), (128, 7168)])
def test_quant_act_128x1_T_shapes(dev, dtype, M, C):
    _check_t(_rand((M, C), M + 7 * C, dtype), dev, f"128x1 {dtype} {M}x{C}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("channels", [70, 72])   # the 16-byte-load kernel takes C % 8 == 0
def test_quant_act_128x1_T_adversarial(dev, dtype, channels):
    # groups of the 128x1 quantizer run down columns: transpose adversarial rows
    cols = np.ascontiguousarray(adversarial_rows(channels, 384, seed=9).T)   # [384 tokens][C channels]
    _check_t(torch.from_numpy(cols).to(dtype), dev, f"128x1 adversarial {dtype} C={channels}")


def test_quant_act_128x1_T_backward_workload(dev):
    d = workloads.backward_pair(device=dev)
    for name in ("dY", "X"):
        x = d[name]
        qT, sT = fb.fp8_quant_act_128x1_T(x)
        # sampled: token chunks 0 and 31, all channels
        for tb in (0, 31):
            xs = x[tb * 128:(tb + 1) * 128]
            qo, so = oracle.quant_act_128x1_T(to_oracle(xs))
            torch.cuda.synchronize()
            assert_codes_equal(qT[:, tb * 128:(tb + 1) * 128].cpu().numpy(), qo, f"128x1 {name} chunk {tb}")
            assert_scales_equal(sT[tb:tb + 1].cpu().numpy(), so, f"128x1 {name} scales chunk {tb}")


def _check_dual(x_cpu, dev, what):
    q, s, qT, sT = fb.fp8_quant_act_1x128_128x1_T(x_cpu.to(dev))
    qo, so = oracle.quant_act_1x128(to_oracle(x_cpu))
    qto, sto = oracle.quant_act_128x1_T(to_oracle(x_cpu))
    torch.cuda.synchronize()
    assert_codes_equal(q.cpu().numpy(), qo, what + " 1x128 codes")
    assert_scales_equal(s.cpu().numpy(), so, what + " 1x128 scales")
    assert_codes_equal(qT.cpu().numpy(), qto, what + " 128x1 codes")
    assert_scales_equal(sT.cpu().numpy(), sto, what + " 128x1 scales")


# C % 256 == 0 with BF16 takes the single pass; the other cases the two passes
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,C", [(128, 256), (256, 512), (384, 7168), (128, 384), (256, 128)])
def test_dual_layout_quantizer(dev, dtype, M, C):
    _check_dual(_rand((M, C), 3 * M + C, dtype), dev, f"1x128+128x1 {dtype} {M}x{C}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dual_layout_quantizer_adversarial(dev, dtype):
    # hard 1x128 groups along the rows, then hard 128x1 groups down the columns
    rows = adversarial_rows(256, 512, seed=21)                             # [256 tokens][512 channels]
    cols = np.ascontiguousarray(adversarial_rows(512, 256, seed=22).T)     # [256 tokens][512 channels]
    _check_dual(torch.from_numpy(rows).to(dtype), dev, f"1x128+128x1 adversarial rows {dtype}")
    _check_dual(torch.from_numpy(cols).to(dtype), dev, f"1x128+128x1 adversarial columns {dtype}")


def test_dual_layout_quantizer_backward_workload(dev):
    # full size: identical to the two separate passes (each pinned to the
    # oracle above), and sampled token chunks against the oracle
    d = workloads.backward_pair(device=dev)
    dY = d["dY"]
    q, s, qT, sT = fb.fp8_quant_act_1x128_128x1_T(dY)
    q1, s1 = fb.fp8_quant_act_1x128(dY)
    qt1, st1 = fb.fp8_quant_act_128x1_T(dY)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(qT, qt1), "codes differ from the separate passes"
    assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), "1x128 scales differ from the separate pass"
    assert torch.equal(sT.view(torch.int32), st1.view(torch.int32)), "128x1 scales differ from the separate pass"
    for tb in (0, 17, 31):
        xs = dY[tb * 128:(tb + 1) * 128]
        qo, so = oracle.quant_act_128x1_T(to_oracle(xs))
        assert_codes_equal(qT[:, tb * 128:(tb + 1) * 128].cpu().numpy(), qo, f"dY 128x1 chunk {tb}")
        assert_scales_equal(sT[tb:tb + 1].cpu().numpy(), so, f"dY 128x1 scales chunk {tb}")
        qo, so = oracle.quant_act_1x128(to_oracle(xs))
        assert_codes_equal(q[tb * 128:(tb + 1) * 128].cpu().numpy(), qo, f"dY 1x128 rows of chunk {tb}")
        assert_scales_equal(s[:, tb * 128:(tb + 1) * 128].cpu().numpy(), so, f"dY 1x128 scales of chunk {tb}")


def test_quantizers_are_deterministic(dev):
    x = _rand((512, 1024), 77, torch.bfloat16).to(dev)
    a = fb.fp8_quant_act_1x128(x)
    b = fb.fp8_quant_act_1x128(x)
    c = fb.fp8_quant_act_128x1_T(x)
    d = fb.fp8_quant_act_128x1_T(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


def test_empty_inputs_are_no_ops(dev):
    q, s = fb.fp8_quant_act_1x128(torch.zeros((0, 256), device=dev))
    assert q.shape == (0, 256) and s.shape == (2, 0)
    qT, sT = fb.fp8_quant_act_128x1_T(torch.zeros((128, 0), device=dev))
    assert qT.shape == (0, 128)
