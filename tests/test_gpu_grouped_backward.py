"""GPU parity of the per-expert backward path: the grouped 128x1 transposed
quantizer (codes and scales bit for bit against the oracle, nothing written
past the last group), the per-expert Wgrad GEMM (within the GEMM acceptance
bound), and the grouped Dgrad (the grouped GEMM on the weights' transposed
copies)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import adversarial_rows, assert_codes_equal, assert_scales_equal, bf16_bits, to_oracle, u8

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def _x(M, C, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, C), generator=g)
    x[torch.rand((M, C), generator=g) < 0.01] *= 100.0
    return x.to(dtype)


def _check_grouped_quant(dev, x, counts, what):
    off = _offsets(counts)
    offd = torch.from_numpy(off).to(dev)
    M, C = x.shape
    E = len(counts)
    ld = fb.grouped_ld(M, E)
    # sentinels: nothing past the last group may be written
    qT = torch.full((C, ld), 0xCD, dtype=torch.uint8, device=dev)
    sT = torch.full((ld // 128, C), -7.0, dtype=torch.float32, device=dev)
    xd = x.to(dev)
    rc = fb.lib().fp8_quant_act_128x1_T_grouped(xd.data_ptr(), fb.BF16 if x.dtype == torch.bfloat16 else fb.F32,
                                                M, C, offd.data_ptr(), E, ld, qT.data_ptr(), sT.data_ptr(),
                                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fb.status_string(rc)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act_128x1_T_grouped(to_oracle(x), off)
    G = s_ref.shape[0]
    assert_codes_equal(u8(qT[:, :128 * G]), q_ref, f"{what}: codes")
    assert_scales_equal(sT[:G].cpu().numpy(), s_ref, f"{what}: scales")
    assert torch.all(qT[:, 128 * G:] == 0xCD), f"{what}: codes written past the last group"
    assert torch.all(sT[G:] == -7.0), f"{what}: scales written past the last group"


COUNTS = [
    [5],
    [128],
    [0, 1, 0, 300, 17, 0],
    [127, 128, 129, 255, 256, 257],
    [0, 0, 0],
    [1000, 3, 600, 0, 64],
]


@pytest.mark.parametrize("counts", COUNTS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("C", [128, 384])
def test_grouped_quant_128x1_T(dev, counts, dtype, C):
    x = _x(sum(counts), C, sum(counts) + C, dtype)
    _check_grouped_quant(dev, x, counts, f"grouped 128x1 {counts} C={C} {dtype}")


@pytest.mark.parametrize("counts", COUNTS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("C", [256, 384, 512])
def test_grouped_dual_layout_quantizer(dev, counts, dtype, C):
    # 1x128 over all rows and the grouped 128x1 in one call (one pass for
    # BF16 with C % 256 == 0, the two passes otherwise)
    x = _x(sum(counts), C, 7 * sum(counts) + C, dtype)
    off = _offsets(counts)
    offd = torch.from_numpy(off).to(dev)
    M, E = sum(counts), len(counts)
    ld = fb.grouped_ld(M, E)
    q = torch.full((M, C), 0xCD, dtype=torch.uint8, device=dev)
    s = torch.full((C // 128, M), -7.0, dtype=torch.float32, device=dev)
    qT = torch.full((C, ld), 0xCD, dtype=torch.uint8, device=dev)
    sT = torch.full((ld // 128, C), -7.0, dtype=torch.float32, device=dev)
    xd = x.to(dev)
    rc = fb.lib().fp8_quant_act_1x128_128x1_T_grouped(
        xd.data_ptr(), fb.BF16 if x.dtype == torch.bfloat16 else fb.F32, M, C, offd.data_ptr(), E, ld,
        q.data_ptr(), s.data_ptr(), qT.data_ptr(), sT.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fb.status_string(rc)
    torch.cuda.synchronize()
    what = f"grouped 1x128+128x1 {counts} C={C} {dtype}"
    if M > 0:
        qo, so = oracle.quant_act_1x128(to_oracle(x))
        assert_codes_equal(u8(q), qo, f"{what}: 1x128 codes")
        assert_scales_equal(s.cpu().numpy(), so, f"{what}: 1x128 scales")
    q_ref, s_ref = oracle.quant_act_128x1_T_grouped(to_oracle(x), off)
    G = s_ref.shape[0]
    assert_codes_equal(u8(qT[:, :128 * G]), q_ref, f"{what}: 128x1 codes")
    assert_scales_equal(sT[:G].cpu().numpy(), s_ref, f"{what}: 128x1 scales")
    assert torch.all(qT[:, 128 * G:] == 0xCD), f"{what}: codes written past the last group"
    assert torch.all(sT[G:] == -7.0), f"{what}: scales written past the last group"


def test_grouped_dual_layout_quantizer_moe_workload(dev):
    # the MoE backward's dY_down at full size (65,536 routed rows x 7,168):
    # identical to the two separate passes
    d = workloads.grouped_moe(device=dev, with_weights=False)
    off = torch.from_numpy(d["offsets"]).to(dev)
    x = d["A_up"]
    q, s, qT, sT = fb.fp8_quant_act_1x128_128x1_T_grouped(x, off)
    q1, s1 = fb.fp8_quant_act_1x128(x)
    qt1, st1 = fb.fp8_quant_act_128x1_T_grouped(x, off)
    torch.cuda.synchronize()
    G = int(oracle.padded_group_starts(d["offsets"])[-1])
    assert torch.equal(q, q1), "1x128 codes differ from the separate pass"
    assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), "1x128 scales differ from the separate pass"
    assert torch.equal(qT[:, :128 * G], qt1[:, :128 * G]), "128x1 codes differ from the separate pass"
    assert torch.equal(sT[:G].view(torch.int32), st1[:G].view(torch.int32)), "128x1 scales differ"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_grouped_quant_128x1_T_adversarial(dev, dtype):
    # the hard patterns of the quantizer tests, down the token columns of
    # experts whose groups start at unaligned rows
    cols = np.ascontiguousarray(adversarial_rows(128, 640, seed=11).T)   # [640 tokens][128 channels]
    counts = [3, 256, 125, 256]
    _check_grouped_quant(dev, torch.from_numpy(cols).to(dtype), counts, f"grouped 128x1 adversarial {dtype}")


def _padded_codes(counts, rows, seed):
    """Random codes [rows][128 P_E] with zero codes in every expert's padding."""
    off = _offsets(counts)
    P = oracle.padded_group_starts(off)
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, (rows, 128 * int(P[-1])), generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B
    for e, n in enumerate(counts):
        c[:, 128 * P[e] + n:128 * P[e + 1]] = 0
    return c


def _wgrad_case(dev, counts, N, K, seed):
    off = _offsets(counts)
    E, M = len(counts), int(off[-1])
    G = int(oracle.padded_group_starts(off)[-1])
    ld = fb.grouped_ld(M, E)
    A = torch.zeros((N, ld), dtype=torch.uint8)
    B = torch.zeros((K, ld), dtype=torch.uint8)
    A[:, :128 * G] = _padded_codes(counts, N, seed)
    B[:, :128 * G] = _padded_codes(counts, K, seed + 1)
    g = torch.Generator().manual_seed(seed + 2)
    sA = (1e-3 + torch.rand((ld // 128, N), generator=g)).float()
    sB = (1e-3 + torch.rand((ld // 128, K), generator=g)).float()
    C = fb.fp8_grouped_gemm_wgrad(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), torch.from_numpy(off).to(dev), M)
    torch.cuda.synchronize()
    return A, sA, B, sB, off, C


def _check(C, ref, absref, what):
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        c = oracle.bf16_bits_to_f64(bf16_bits(C))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound (worst {worst:.3g}); "
                             f"first at {i}: got {c[i]!r}, ref {ref[i]!r}")


@pytest.mark.parametrize("counts,N,K", [
    ([5], 128, 128),
    ([0, 1, 0, 300, 17, 0], 256, 384),
    ([127, 128, 129], 384, 256),
    ([0, 0], 128, 256),
    ([700, 2, 260, 0, 1], 512, 640),
])
def test_grouped_wgrad_random_codes(dev, counts, N, K):
    A, sA, B, sB, off, C = _wgrad_case(dev, counts, N, K, sum(counts) + N + K)
    assert C.shape == (len(counts), N, K)
    ref, absref = oracle.grouped_wgrad_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    _check(C, ref, absref, f"grouped wgrad {counts} N={N} K={K}")
    for e, n in enumerate(counts):
        if n == 0:
            assert torch.all(C[e].float() == 0), f"expert {e} without tokens is not zero"


def test_grouped_backward_pipeline_small(dev):
    # BF16 dY and X -> grouped 128x1 quantizers -> per-expert Wgrad, every
    # stage against the oracle
    counts = [130, 0, 77, 256]
    off = _offsets(counts)
    offd = torch.from_numpy(off).to(dev)
    M = sum(counts)
    dY, X = _x(M, 256, 1, torch.bfloat16), _x(M, 384, 2, torch.bfloat16)
    qa, sa = fb.fp8_quant_act_128x1_T_grouped(dY.to(dev), offd)
    qb, sb = fb.fp8_quant_act_128x1_T_grouped(X.to(dev), offd)
    dW = fb.fp8_grouped_gemm_wgrad(qa, sa, qb, sb, offd, M)
    torch.cuda.synchronize()
    qa_ref, sa_ref = oracle.quant_act_128x1_T_grouped(to_oracle(dY), off)
    qb_ref, sb_ref = oracle.quant_act_128x1_T_grouped(to_oracle(X), off)
    G = sa_ref.shape[0]
    assert_codes_equal(u8(qa[:, :128 * G]), qa_ref, "dY codes")
    assert_codes_equal(u8(qb[:, :128 * G]), qb_ref, "X codes")
    ref, absref = oracle.grouped_wgrad_ref(qa_ref, sa_ref, qb_ref, sb_ref, off)
    _check(dW, ref, absref, "grouped backward pipeline")


def test_grouped_wgrad_rejects_bad_arguments(dev):
    L = fb.lib()
    off = torch.tensor([0, 100, 300], dtype=torch.int32, device=dev)
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    p = buf.data_ptr()                        # x: 300 x 128 BF16 = 75 KB
    q, sc = p + (1 << 18), p + (1 << 19)      # qT: 128 x 640 B, sT: 5 x 128 floats
    s = torch.cuda.current_stream().cuda_stream
    ld = fb.grouped_ld(300, 2)
    assert ld == 640
    assert L.fp8_quant_act_128x1_T_grouped(p, 1, 300, 128, off.data_ptr(), 2, ld, q, sc, s) == 0
    assert L.fp8_quant_act_128x1_T_grouped(p, 1, 300, 128, off.data_ptr(), 2, ld - 128, q, sc, s) != 0  # ld small
    assert L.fp8_quant_act_128x1_T_grouped(p, 1, 300, 100, off.data_ptr(), 2, ld, q, sc, s) != 0       # C % 128
    assert L.fp8_quant_act_128x1_T_grouped(p, 1, 300, 128, off.data_ptr(), 0, ld, q, sc, s) != 0       # E = 0
    assert L.fp8_quant_act_128x1_T_grouped(p, 1, 300, 128, None, 2, ld, q, sc, s) != 0
    assert L.fp8_quant_act_128x1_T_grouped(p + 1, 1, 300, 128, off.data_ptr(), 2, ld, q, sc, s) != 0
    assert L.fp8_grouped_gemm_wgrad(p, p, p, p, p, off.data_ptr(), 2, 300, 128, 128, ld - 128, s) != 0
    assert L.fp8_grouped_gemm_wgrad(p, p, p, p, p, off.data_ptr(), 2, 300, 100, 128, ld, s) != 0
    assert L.fp8_grouped_gemm_wgrad(p, p, p, p, None, off.data_ptr(), 2, 300, 128, 128, ld, s) != 0
    torch.cuda.synchronize()


def test_grouped_moe_backward_workload_sampled(dev):
    d = workloads.grouped_moe_backward(device=dev)
    off = d["offsets"]
    offd = torch.from_numpy(off).to(dev)
    M, E = int(off[-1]), len(d["counts"])
    P = oracle.padded_group_starts(off)
    nz = [e for e in range(E) if d["counts"][e] > 0]
    experts = sorted({nz[0], nz[-1], int(np.argmax(d["counts"])), int(np.argmin(np.where(d["counts"] > 0,
                                                                                       d["counts"], 1 << 30)))})
    for dy_key, x_key, w_key in (("dY_up", "A_up", "W_up"), ("dY_dn", "A_dn", "W_dn")):
        dY, X, W = d[dy_key], d[x_key], d[w_key]
        N, K = dY.shape[1], X.shape[1]
        # Wgrad: dW_e = dY_e^T X_e
        qa, sa = fb.fp8_quant_act_128x1_T_grouped(dY, offd)
        qb, sb = fb.fp8_quant_act_128x1_T_grouped(X, offd)
        dW = fb.fp8_grouped_gemm_wgrad(qa, sa, qb, sb, offd, M)
        # Dgrad: dX = dY_e W_e per expert, with the weights' transposed copies
        qdy, sdy = fb.fp8_quant_act_1x128(dY)
        qwT = torch.empty((E, K, N), dtype=torch.uint8, device=dev)
        swT = torch.empty((E, K // 128, N // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            _, _, qwT[e], swT[e] = fb.fp8_quant_w_128x128(W[e], transposed=True)
        dX = fb.fp8_grouped_gemm_blockscaled(qdy, sdy, qwT, swT, offd)
        torch.cuda.synchronize()
        rows = np.array([0, 1, 77, N - 1])
        cols = np.arange(0, K, 97)
        for e in experts:
            c = slice(128 * int(P[e]), 128 * int(P[e + 1]))
            g = slice(int(P[e]), int(P[e + 1]))
            # the sampled rows of the expert's quantized operands against the oracle quantizer
            xe = to_oracle(dY[off[e]:off[e + 1]])
            q_ref, s_ref = oracle.quant_act_128x1_T_grouped(xe, [0, len(xe)])
            assert_codes_equal(u8(qa[rows][:, c]), q_ref[rows], f"{dy_key} codes, expert {e}")
            assert_scales_equal(sa[g][:, rows].cpu().numpy(), s_ref[:, rows], f"{dy_key} scales, expert {e}")
            ref, absref = oracle.gemm_ref_rows(u8(qa[:, c]), sa[g].cpu().numpy(), u8(qb[:, c]),
                                               sb[g].cpu().numpy(), 1, rows=rows, cols=cols)
            _check(dW[e][rows][:, cols], ref, absref, f"{dy_key} wgrad expert {e}, sampled")
        # Dgrad: first and last row of the sampled experts
        drows = np.unique(np.concatenate([[off[e], off[e + 1] - 1] for e in experts]))
        ref, absref = oracle.grouped_gemm_ref(u8(qdy[drows]), sdy[:, drows].cpu().numpy(), u8(qwT),
                                              swT.cpu().numpy(), _compact(off, drows), cols=cols)
        _check(dX[drows][:, cols], ref, absref, f"{dy_key} grouped dgrad, sampled")
        del qa, sa, qb, sb, dW, qdy, sdy, qwT, swT, dX


def _compact(off, rows):
    expert = np.searchsorted(off, rows, side="right") - 1
    counts = np.bincount(expert, minlength=len(off) - 1)
    out = np.zeros(len(off), np.int32)
    out[1:] = np.cumsum(counts)
    return out
