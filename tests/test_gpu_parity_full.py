"""GPU parity at full size and on every tile shape the dense GEMM can pick.

* Every output tile the host can choose for fp8_gemm_blockscaled is run at a
  shape that picks it (confirmed through fp8_gemm_blockscaled_tile), in both
  scale modes, and the whole NaN-prefilled output is compared with the oracle;
  so is the region a tail launch of 64x64 subtiles computes.
* The dense Fprop, Dgrad and Wgrad layers at their real sizes are compared on
  one full output row per m-tile, the row's offset inside its tile moving
  from tile to tile, so every wave row and both halves of every tile are seen.
* The grouped GEMM's tile kernel (chosen when the experts average more than
  256 rows) on ragged experts that include empty ones, with and without a
  last partial round left to its 64x64-subtile tail kernel, and skewed
  batches whose few large experts go to the tile kernel while the rest take
  the weight-streaming kernel.
* The MoE activation and expert-weight quantizers at their full sizes
  (65,536 x 7,168 and 65,536 x 2,048 activations, 32 x 4,096 x 7,168 and
  32 x 7,168 x 2,048 weights), bit for bit against the oracle.

Acceptance bound for the GEMMs: |C - ref| <= 4e-3 * sum_k |a_k b_k| + ulp_bf16(ref).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (assert_codes_equal, assert_scales_equal, bf16_bits, oracle_quant_act_1x128_big,
                     oracle_quant_w_128x128_big, to_oracle, u8)
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
                             f"(worst {worst:.3g}); first at {i}: got {c[i]!r}, ref {ref[i]!r}")
    return worst


# shapes that pick each kernel (rows, columns, ring depth, tail tiles) on a
# 256-CU MI355X; the test asserts the pick
TILE_CASES = [((4096, 4096, 256), (256, 256, 2, 0)),
              ((4096, 7168, 256), (256, 224, 3, 0)),
              ((7168, 2048, 256), (224, 256, 3, 0)),
              ((7168, 4096, 128), (224, 256, 3, 0)),
              ((777, 5120, 128), (128, 256, 2, 0)),      # ragged last m-tile (9 rows)
              ((3700, 2176, 128), (128, 128, 2, 0)),     # ragged last m-tile (116 rows)
              ((1700, 2048, 128), (128, 128, 4, 0)),     # ragged last m-tile (36 rows)
              ((1300, 3072, 128), (64, 64, 2, 0)),       # ragged last m-tile (20 rows)
              ((300, 640, 256), (64, 64, 4, 0)),         # ragged last m-tile (44 rows)
              ((1, 128, 128), (64, 64, 4, 0))]           # one row
# (the three-deep 64x64 kernel computes the tails: test_gemm_tail_launch)


def test_tile_cases_cover_every_tile(dev):
    picked = {fb.fp8_gemm_blockscaled_tile(M, N, K, mode) for (M, N, K), _ in TILE_CASES
              for mode in (MODE_BLOCK, MODE_ROW)}
    assert picked == {t for _, t in TILE_CASES}


@pytest.mark.parametrize("shape,tile", TILE_CASES)
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_gemm_every_tile_full_output(dev, shape, tile, mode):
    M, N, K = shape
    assert fb.fp8_gemm_blockscaled_tile(M, N, K, mode) == tile, "the shape no longer picks this tile"
    A, B = _codes((M, K), M + N + K + mode), _codes((N, K), 3 * N + K + mode)
    sA = _scales((K // 128, M), 17 + M)
    sB = _scales((N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N), 19 + N)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode, out=C)
    ref, absref = oracle.gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), mode)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"gemm {M}x{N}x{K} tile {tile} mode {mode}")


@pytest.mark.parametrize("shape", [(4352, 4096, 2048), (4252, 3968, 2048)])
@pytest.mark.parametrize("mode", [MODE_BLOCK, MODE_ROW])
def test_gemm_tail_launch(dev, shape, mode):
    # 17 x 16 tiles of 256x256: one round of 256 and 16 left to the tail
    # launch as 64x64 subtiles. The tile order takes 4 m-tiles at a time, so
    # the last 16 tiles are the 16 n-tiles of the 17th m-tile: every row from
    # 4096 on is checked in full (the second shape has a ragged last m-tile
    # and a last n-tile of 128 columns), with one row of every other m-tile.
    M, N, K = shape
    assert fb.fp8_gemm_blockscaled_tile(M, N, K, mode) == (256, 256, 2, 16)
    A, B = _codes((M, K), M + N + mode), _codes((N, K), 5 * N + mode)
    sA = _scales((K // 128, M), 23 + M)
    sB = _scales((N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N), 29 + N)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), mode, out=C)
    rows = np.array(sorted(set(range(4096, M)) | {t * 256 + (37 * t) % 256 for t in range(16)}))
    ref, absref = oracle.gemm_ref_rows(A[rows].numpy(), sA[:, rows].numpy(), B.numpy(), sB.numpy(), mode)
    torch.cuda.synchronize()
    _check(C[rows], ref, absref, f"gemm {M}x{N}x{K} with a tail, mode {mode}")


def _rows_per_tile(M, N, K, mode):
    """One row per m-tile, at offset 16*(t mod BM/16) + (7t mod 16) inside tile t."""
    bm = fb.fp8_gemm_blockscaled_tile(M, N, K, mode)[0]
    rows = [t * bm + (16 * (t % (bm // 16)) + (7 * t) % 16) % bm for t in range(-(-M // bm))]
    return np.array(sorted({min(r, M - 1) for r in rows} | {M - 1}))


def test_dense_fprop_full_size_rows_per_tile(dev):
    d = workloads.dense_fprop(device=dev)
    qx, sx = fb.fp8_quant_act_1x128(d["X"])
    qw, sw = fb.fp8_quant_w_128x128(d["W"])
    C = torch.full((qx.shape[0], qw.shape[0]), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(qx, sx, qw, sw, out=C)
    torch.cuda.synchronize()
    M, K = qx.shape
    N = qw.shape[0]
    rows = _rows_per_tile(M, N, K, MODE_BLOCK)
    ref, absref = oracle.gemm_ref_rows(u8(qx[rows]), sx[:, rows].cpu().numpy(), u8(qw), sw.cpu().numpy(),
                                       MODE_BLOCK)
    _check(C[rows], ref, absref, f"dense fprop {M}x{N}x{K}, rows {rows.tolist()}")


def test_backward_pair_full_size_rows_per_tile(dev):
    d = workloads.backward_pair(device=dev)
    qdy, sdy = fb.fp8_quant_act_1x128(d["dY"])
    _, _, qwT, swT = fb.fp8_quant_w_128x128(d["W"], transposed=True)
    qdyT, sdyT = fb.fp8_quant_act_128x1_T(d["dY"])
    qxT, sxT = fb.fp8_quant_act_128x1_T(d["X"])
    M, N = qdy.shape
    K = qwT.shape[0]
    dX = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=dev)
    dW = torch.full((N, K), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(qdy, sdy, qwT, swT, fb.SCALE_BLOCK128, out=dX)
    fb.fp8_gemm_blockscaled(qdyT, sdyT, qxT, sxT, fb.SCALE_ROW, out=dW)
    torch.cuda.synchronize()
    rows = _rows_per_tile(M, K, N, MODE_BLOCK)
    ref, absref = oracle.gemm_ref_rows(u8(qdy[rows]), sdy[:, rows].cpu().numpy(), u8(qwT), swT.cpu().numpy(),
                                       MODE_BLOCK)
    _check(dX[rows], ref, absref, f"dgrad {M}x{K}x{N}, rows {rows.tolist()}")
    rows = _rows_per_tile(N, K, M, MODE_ROW)
    ref, absref = oracle.gemm_ref_rows(u8(qdyT[rows]), sdyT[:, rows].cpu().numpy(), u8(qxT), sxT.cpu().numpy(),
                                       MODE_ROW)
    _check(dW[rows], ref, absref, f"wgrad {N}x{K}x{M}, rows {rows.tolist()}")


@pytest.mark.parametrize("counts,N,K", [
    ([0, 900, 0, 250], 512, 512),                               # empty first and inner experts
    ([300, 0, 0, 0, 1200, 17, 0, 540], 384, 256),               # M_total = 2057 > 256 * 8
    ([0, 0, 2100, 0], 256, 384),                                 # one expert holds every row
])
def test_grouped_tile_kernel_with_empty_experts(dev, counts, N, K):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M, E = int(off[-1]), len(counts)
    assert M > 256 * E, "the case must take the grouped tile kernel"
    seed = M + N + K
    A, sA = _codes((M, K), seed), _scales((K // 128, M), seed + 1)
    B, sB = _codes((E, N, K), seed + 2), _scales((E, N // 128, K // 128), seed + 3)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), torch.from_numpy(off).to(dev),
                                    out=C)
    ref, absref = oracle.grouped_gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"grouped tile kernel {counts} N={N} K={K}")


def test_moe_activation_quantizers_full_size(dev):
    d = workloads.grouped_moe(device=dev)
    for key in ("A_up", "A_dn"):
        X = d.pop(key)
        q, s = fb.fp8_quant_act_1x128(X)
        torch.cuda.synchronize()
        qo, so = oracle_quant_act_1x128_big(to_oracle(X))
        assert_codes_equal(u8(q), qo, f"{key} {tuple(X.shape)} codes")
        assert_scales_equal(s.cpu().numpy(), so, f"{key} {tuple(X.shape)} scales")
        del X, q, s


def test_moe_expert_weight_quantizers_full_size(dev):
    d = workloads.grouped_moe(device=dev)
    for key in ("W_up", "W_dn"):
        W = d.pop(key)
        for e in range(W.shape[0]):
            q, s = fb.fp8_quant_w_128x128(W[e])
            torch.cuda.synchronize()
            qo, so = oracle_quant_w_128x128_big(to_oracle(W[e]))
            assert_codes_equal(u8(q), qo, f"{key}[{e}] codes")
            assert_scales_equal(s.cpu().numpy(), so, f"{key}[{e}] scales")
        del W


def _grouped_route(counts, N, cus):
    """(tiles of the grouped tile kernel, tiles left to its tail kernel): a
    last round of 256x256 tiles that fits one round of 64x64 subtiles, three
    per CU, goes to the tail."""
    tiles = sum(-(-c // 256) for c in counts) * -(-N // 256)
    rem = tiles % cus
    tail = rem if rem * 16 <= 3 * cus else 0
    return tiles - tail, tail


@pytest.mark.parametrize("counts,N,K,route", [
    ([7580] * 9 + [0] + [7600], 256, 128, (256, 44)),       # one full round, 44 tiles left to the tail
    ([0, 900, 0, 250], 512, 256, (0, 10)),                  # fewer tiles than a quarter of the CUs: all tail
    ([5000, 5000, 0, 1], 1280, 128, (205, 0)),             # a partial round of 205 tiles: no tail
    ([16367, 16384, 16384, 16379], 512, 128, (512, 0)),     # exactly two rounds
    ([38909, 38912], 256, 128, (256, 48)),                  # the largest tail: 768 subtiles, 3 per CU
    ([38909, 38913], 256, 128, (305, 0)),                   # one tile more: no tail
])
def test_grouped_tile_kernel_and_its_tail(dev, counts, N, K, route):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M, E = int(off[-1]), len(counts)
    assert M > 256 * E, "the case must take the grouped tile kernel"
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if cus == 256:
        assert _grouped_route(counts, N, cus) == route
    seed = 5 * M + N
    A, sA = _codes((M, K), seed), _scales((K // 128, M), seed + 1)
    B, sB = _codes((E, N, K), seed + 2), _scales((E, N // 128, K // 128), seed + 3)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), torch.from_numpy(off).to(dev),
                                    out=C)
    ref, absref = oracle.grouped_gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"grouped {counts[:4]}... N={N} K={K} route {route}")


@pytest.mark.parametrize("counts,N,K", [
    ([3000] + [int(c) for c in np.random.default_rng(9).integers(1, 21, 31)], 512, 768),   # one big among tiny
    ([5, 600, 3, 0, 300, 1], 384, 512),                         # two experts past one 256-row pass
    ([257, 0, 256, 1], 256, 256),                               # at the 256-row boundary
])
def test_grouped_skewed_experts_take_both_kernels(dev, counts, N, K):
    # few rows per expert on average, so the weight-streaming kernel runs, but
    # the experts with more than 256 rows go to the tile kernel
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M, E = int(off[-1]), len(counts)
    assert M < 256 * E and max(counts) > 256
    seed = 3 * M + N
    A, sA = _codes((M, K), seed), _scales((K // 128, M), seed + 1)
    B, sB = _codes((E, N, K), seed + 2), _scales((E, N // 128, K // 128), seed + 3)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(A.to(dev), sA.to(dev), B.to(dev), sB.to(dev), torch.from_numpy(off).to(dev),
                                    out=C)
    ref, absref = oracle.grouped_gemm_ref(A.numpy(), sA.numpy(), B.numpy(), sB.numpy(), off)
    torch.cuda.synchronize()
    _check(C, ref, absref, f"grouped skewed {counts[:4]}... N={N} K={K}")
