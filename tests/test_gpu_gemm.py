"""GPU parity of the block-scaled GEMM (dense, both scale modes) and its
grouped per-expert form against the CPU oracle, within the acceptance bound
|C - ref| <= 4e-3 * sum_k |a_k b_k| + ulp_bf16(ref)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import bf16_bits, to_oracle, u8
from oracle.gemm import MODE_BLOCK, MODE_ROW

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3B
    return c


def _scales(shape, seed, lo=1e-3, hi=1.0):
    g = torch.Generator().manual_seed(seed)
    return (lo + (hi - lo) * torch.rand(shape, generator=g)).to(torch.float32)


def _check(C, ref, absref, what):
    ok, worst = oracle.check_gemm(bf16_bits(C), ref, absref)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        c = oracle.bf16_bits_to_f64(bf16_bits(C))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound "
                             f"(worst {worst:.3g}); first at {i}: got {c[i]!r}, ref {ref[i]!r}, "
                             f"absref {absref[i]!r}")
    return worst


SHAPES = [(1, 128, 128), (16, 128, 256), (17, 256, 384), (256, 256, 128), (255, 512, 1024),
          (300, 384, 640), (513, 640, 256), (1024, 1280, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_gemm_random_codes(dev, M, N, K, mode):
    A, B = _codes((M, K), M + 3 * N + 7 * K), _codes((N, K), 11 + M + N + K)
    sA = _scales((K // 128, M), 5 + M)
    sB = _scales((N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N), 9 + N)
    # NaN-filled output: an element the kernel does not write fails the bound
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode, out=C)
    ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"gemm {M}x{N}x{K} mode {mode}")


def test_gemm_exact_small_integers(dev):
    # codes of 0 and +-1 with unit scales: every partial and the sum are small
    # integers (|C| <= 256), exact in FP32 and in BF16, so the result must be exact
    g = torch.Generator().manual_seed(3)
    vals = torch.tensor([0x00, 0x38, 0xB8], dtype=torch.uint8)  # 0, 1, -1
    A = vals[torch.randint(0, 3, (64, 256), generator=g)]
    B = vals[torch.randint(0, 3, (128, 256), generator=g)]
    sA = torch.ones((2, 64)); sB = torch.ones((1, 2))
    C = fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev))
    ref, _ = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy())
    assert np.all(np.abs(ref) <= 256)        # exact in BF16 (8 significant bits)
    assert np.array_equal(C.float().cpu().numpy().astype(np.float64), ref)


def test_gemm_tiny_fprop_end_to_end(dev):
    d = workloads.tiny_fprop(device=dev)
    qx, sx = fb.fp8_quant_act_1x128(d["X"])
    qw, sw = fb.fp8_quant_w_128x128(d["W"])
    C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw)
    ref, absref = oracle.gemm_ref(u8(qx), sx.cpu().numpy(), u8(qw), sw.cpu().numpy())
    torch.cuda.synchronize()
    _check(C, ref, absref, "tiny fprop 256x512x1024")
    # and the quantized operands themselves match the oracle's
    qxo, sxo = oracle.quant_act_1x128(to_oracle(d["X"]))
    assert np.array_equal(u8(qx), qxo)


SAMPLE_ROWS = [0, 1, 127, 128, 255, 256, 2047, 3071, 4000, 4095]


def test_gemm_dense_fprop_sampled(dev):
    d = workloads.dense_fprop(device=dev)
    qx, sx = fb.fp8_quant_act_1x128(d["X"])
    qw, sw = fb.fp8_quant_w_128x128(d["W"])
    C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw)
    torch.cuda.synchronize()
    ref, absref = oracle.gemm_ref_rows(u8(qx), sx.cpu().numpy(), u8(qw), sw.cpu().numpy(), MODE_BLOCK,
                                       rows=np.array(SAMPLE_ROWS))
    _check(C[SAMPLE_ROWS], ref, absref, "dense fprop 4096x7168x7168, sampled rows")


def test_gemm_backward_pair_sampled(dev):
    d = workloads.backward_pair(device=dev)
    # Dgrad: dX = dY . W with W's transposed 128x128 copy, block mode
    qdy, sdy = fb.fp8_quant_act_1x128(d["dY"])
    qw, sw, qwT, swT = fb.fp8_quant_w_128x128(d["W"], transposed=True)
    dX = fb.fp8_gemm_blockscaled(qdy, sdy, qwT, swT, fb.SCALE_BLOCK128)
    # Wgrad: dW = dY^T . X over tokens, both operands 128x1-quantized, row mode
    qdyT, sdyT = fb.fp8_quant_act_128x1_T(d["dY"])
    qxT, sxT = fb.fp8_quant_act_128x1_T(d["X"])
    dW = fb.fp8_gemm_blockscaled(qdyT, sdyT, qxT, sxT, fb.SCALE_ROW)
    torch.cuda.synchronize()
    ref, absref = oracle.gemm_ref_rows(u8(qdy), sdy.cpu().numpy(), u8(qwT), swT.cpu().numpy(), MODE_BLOCK,
                                       rows=np.array(SAMPLE_ROWS))
    _check(dX[SAMPLE_ROWS], ref, absref, "dgrad 4096x7168x7168, sampled rows")
    rows = np.array([0, 5, 1000, 4095, 7100, 7167])
    ref, absref = oracle.gemm_ref_rows(u8(qdyT), sdyT.cpu().numpy(), u8(qxT), sxT.cpu().numpy(), MODE_ROW,
                                       rows=rows)
    _check(dW[rows], ref, absref, "wgrad 7168x7168x4096, sampled rows")


def _grouped_case(dev, counts, N, K, seed):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M, E = int(off[-1]), len(counts)
    A = _codes((M, K), seed)
    sA = _scales((K // 128, M), seed + 1)
    B = _codes((E, N, K), seed + 2)
    sB = _scales((E, N // 128, K // 128), seed + 3)
    # NaN-filled output: a row the kernel does not write fails the bound
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), torch.from_numpy(off).to(dev),
                                    out=C)
    return A, sA, B, sB, off, C


@pytest.mark.parametrize("counts,N,K", [
    ([5], 128, 128),
    ([0, 1, 0, 300, 17, 0], 256, 256),
    ([256, 255, 257, 1], 384, 384),
    ([17, 0, 130, 64, 2, 33], 640, 896),
    ([600, 1, 0, 1], 256, 512),                                      # one expert past a 256-row pass
    ([int(c) for c in np.random.default_rng(5).integers(0, 9, 200) * (np.arange(200) % 3 != 0)], 384, 256),
    ([int(c) for c in np.random.default_rng(6).integers(0, 5, 300)], 128, 256),   # > 256 experts: index order
    ([1000, 3, 600], 512, 1024),
])
def test_grouped_gemm_random(dev, counts, N, K):
    A, sA, B, sB, off, C = _grouped_case(dev, counts, N, K, sum(counts) + N)
    ref, absref = oracle.grouped_gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"grouped {counts} N={N} K={K}")


def test_grouped_decode_every_subtile_count(dev):
    # the weight-streaming kernel is compiled once per count of 16-row
    # activation subtiles (1 .. 16): give it every count, with the rows
    # filling the last subtile and with one row in it (mean <= 256 rows per
    # expert, so every expert takes that kernel)
    full = [16 * k for k in range(1, 17)]
    ragged = [16 * k - 15 for k in range(1, 17)]
    counts = [c for pair in zip(full, ragged[::-1]) for c in pair]
    assert sum(counts) <= 256 * len(counts)
    A, sA, B, sB, off, C = _grouped_case(dev, counts, 256, 256, 4242)
    ref, absref = oracle.grouped_gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    torch.cuda.synchronize()
    _check(C, ref, absref, "decode kernel, every subtile count")


def test_grouped_gemm_decode_workload(dev):
    d = workloads.decode_grouped(device=dev)
    off = d["offsets"]
    E, N, K = d["W"].shape
    qa, sa = fb.fp8_quant_act_1x128(d["A"])
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        qw[e], sw[e] = fb.fp8_quant_w_128x128(d["W"][e])
    C = torch.full((int(off[-1]), N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(qa, sa, qw, sw, torch.from_numpy(off).to(dev), out=C)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any(), "rows left unwritten"
    # first and last row of every expert
    rows = np.unique(np.concatenate([off[:-1], off[1:] - 1]))
    ref, absref = oracle.grouped_gemm_ref(u8(qa), sa.cpu().numpy(), u8(qw), sw.cpu().numpy(), off, rows=rows)
    _check(C[rows], ref, absref, "decode grouped 32 experts, sampled rows")


def test_grouped_gemm_moe_workload_sampled(dev):
    d = workloads.grouped_moe(device=dev)
    off = d["offsets"]
    offd = torch.from_numpy(off).to(dev)
    for a_key, w_key in (("A_up", "W_up"), ("A_dn", "W_dn")):
        Wt = d[w_key]
        E, N, K = Wt.shape
        qa, sa = fb.fp8_quant_act_1x128(d[a_key])
        qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            qw[e], sw[e] = fb.fp8_quant_w_128x128(Wt[e])
        C = fb.fp8_grouped_gemm_blockscaled(qa, sa, qw, sw, offd)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([off[:-1][np.diff(off) > 0], off[1:][np.diff(off) > 0] - 1]))
        cols = np.arange(0, N, 37)
        # only the needed expert weights go to the host
        ref, absref = oracle.grouped_gemm_ref(u8(qa[rows]), sa[:, rows].cpu().numpy(), u8(qw), sw.cpu().numpy(),
                                              _compact_offsets(off, rows), cols=cols)
        _check(C[rows][:, cols], ref, absref, f"moe {a_key} grouped, sampled rows/cols")


def _compact_offsets(off, rows):
    """Offsets of the expert groups after keeping only ``rows`` (sorted)."""
    expert = np.searchsorted(off, rows, side="right") - 1
    counts = np.bincount(expert, minlength=len(off) - 1)
    out = np.zeros(len(off), np.int32)
    out[1:] = np.cumsum(counts)
    return out


def test_gemm_deterministic(dev):
    A, B = _codes((512, 1024), 1).to(dev), _codes((768, 1024), 2).to(dev)
    sA, sB = _scales((8, 512), 3).to(dev), _scales((6, 8), 4).to(dev)
    c1 = fb.fp8_gemm_blockscaled(A, sA, B, sB)
    c2 = fb.fp8_gemm_blockscaled(A, sA, B, sB)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_gemm_empty_m_is_no_op(dev):
    C = fb.fp8_gemm_blockscaled(torch.zeros((0, 128), dtype=torch.uint8, device=dev),
                                torch.zeros((1, 0), device=dev),
                                torch.zeros((128, 128), dtype=torch.uint8, device=dev),
                                torch.ones((1, 1), device=dev))
    assert C.shape == (0, 128)
