"""Randomized GPU parity: seeded random shapes, modes, dtypes and value ranges
against the oracle, beyond the hand-picked cases of the other files.

* Dense GEMM: M in 1..1199, N and K multiples of 128 up to 1,536, both scale
  modes, codes over the whole E4M3 range, scales spread over 2^-8 .. 2^8;
  the whole NaN-prefilled output is checked. Larger shapes whose last round
  of 256x256 tiles goes to the tail launch, checked on rows spread over the
  tail's tiles and over every other m-tile.
* Grouped GEMM: 1..16 experts whose row counts mix empty, small (<= 32),
  medium and past-one-pass (> 256) experts, so both the weight-streaming and
  the tile kernel run, alone and together; the whole output is checked.
  Larger batches for the tile kernel with and without the tail launch of its
  last partial round, checked on the experts holding the last tiles in full.
* Quantizers: 1x128 (any M, F32 or BF16), 128x128 (with and without the
  transposed copy) and 128x1 transposed (any C) on values whose magnitude
  varies per column and per row, with outliers, bit for bit.
* The fused quantizing epilogues (1x128, and both layouts), the power-of-two
  quantizers and the MFMA-scaled GEMM on their outputs, the grouped 128x1
  quantizers and the per-expert Wgrad on their outputs, and the MoE dispatch
  payload (routing, codes, scales) and the combine.

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


def _tail_m_tiles(tiles_m, tiles_n, tail, group_m=4):
    """m-tiles holding the dense GEMM's last `tail` tiles: its tile order takes
    group_m m-tiles at a time, all n-tiles of a group column by column."""
    out = set()
    for pid in range(tiles_m * tiles_n - tail, tiles_m * tiles_n):
        g, i = divmod(pid, group_m * tiles_n)
        gm = min(tiles_m - g * group_m, group_m)
        out.add(g * group_m + i % gm)
    return sorted(out)


@pytest.mark.parametrize("seed", range(8))
def test_random_dense_tail(dev, seed):
    # shapes whose 256x256 tiles leave 1..48 past whole rounds, with a K that
    # makes the tail launch worth it; every 64-row band of the m-tiles the
    # tail touches is checked on 16 rows, the other m-tiles on one row each
    rng = np.random.default_rng(7500 + seed)
    for _ in range(100):
        tn = int(rng.integers(4, 17))
        tm = -(-(256 * int(rng.integers(1, 3)) + int(rng.integers(1, 49))) // tn)
        M = 256 * tm - int(rng.integers(0, 200))
        N = 256 * tn - 128 * int(rng.integers(0, 2))
        K = 128 * int(rng.integers(12, 17))
        mode = int(rng.integers(0, 2))
        bm, bn, _, tail = fb.fp8_gemm_blockscaled_tile(M, N, K, mode)
        if tail:
            break
    assert tail and (bm, bn) == (256, 256), "no shape with a tail drawn"
    A, B = _codes(rng, (M, K)), _codes(rng, (N, K))
    sA = _scales(rng, (K // 128, M))
    sB = _scales(rng, (N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N))
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_gemm_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(sA).to(dev), torch.from_numpy(B).to(dev),
                            torch.from_numpy(sB).to(dev), mode, out=C)
    rows = {256 * t + int(rng.integers(0, 256)) for t in range(tm)}
    for t in _tail_m_tiles(tm, -(-N // 256), tail):
        for band in range(4):
            rows |= {256 * t + 64 * band + int(r) for r in rng.integers(0, 64, 16)}
    rows = np.array(sorted(r for r in rows if r < M))
    ref, absref = oracle.gemm_ref_rows(A[rows], sA[:, rows], B, sB, mode)
    torch.cuda.synchronize()
    _check(C[rows], ref, absref, f"seed {seed}: gemm {M}x{N}x{K} mode {mode}, tail {tail}")


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


@pytest.mark.parametrize("seed", range(8))
def test_random_grouped_tile_and_tail(dev, seed):
    # experts averaging more than 256 rows (the tile kernel) in batches whose
    # 256x256 tiles leave 1..48 past whole rounds of 256 CUs (the tail launch
    # takes those as 64x64 subtiles; 6 of the 8 seeds) or more (no tail):
    # every row of the experts that hold the last tiles, every 16th elsewhere
    rng = np.random.default_rng(8500 + seed)
    want_tail = seed % 4 != 3
    for _ in range(1000):
        E = int(rng.integers(4, 25))
        tn = int(rng.integers(1, 5))
        mt = rng.integers(0, 9, E)
        mt[rng.random(E) < 0.15] = 0
        tiles = int(mt.sum()) * tn
        rem = tiles % 256
        if tiles > 256 and ((1 <= rem <= 48) if want_tail else rem > 48):
            counts = np.where(mt > 0, 256 * (mt - 1) + rng.integers(1, 257, E), 0)
            if counts.sum() > 256 * E:
                break
    else:
        raise AssertionError("no batch drawn")
    N, K = 256 * tn, 128 * int(rng.integers(1, 5))
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M = int(off[-1])
    A, B = _codes(rng, (M, K)), _codes(rng, (E, N, K))
    sA, sB = _scales(rng, (K // 128, M)), _scales(rng, (E, N // 128, K // 128))
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    fb.fp8_grouped_gemm_blockscaled(torch.from_numpy(A).to(dev), torch.from_numpy(sA).to(dev),
                                    torch.from_numpy(B).to(dev), torch.from_numpy(sB).to(dev),
                                    torch.from_numpy(off).to(dev), out=C)
    # the experts holding the last 48 tiles (tiles are numbered expert-major)
    last, acc = set(), 0
    for e in range(E - 1, -1, -1):
        if acc >= 48:
            break
        if mt[e]:
            last.add(e)
            acc += int(mt[e]) * tn
    rows = set(range(0, M, 16))
    for e in last:
        rows |= set(range(int(off[e]), int(off[e + 1])))
    rows = np.array(sorted(rows))
    ref, absref = oracle.grouped_gemm_ref(A, sA, B, sB, off, rows=rows)
    torch.cuda.synchronize()
    _check(C[rows], ref, absref, f"seed {seed}: grouped {E} experts, {tiles} tiles (past rounds: {tiles % 256}), "
                                 f"N={N} K={K}")


def _values(rng, shape, dtype):
    """Normals scaled per column (2^-20 .. 2^20) and per row (2^-6 .. 2^6), with
    a few outliers x1000 and some exact zeros."""
    x = rng.standard_normal(shape) * np.exp2(rng.uniform(-20, 20, (1, shape[1])))
    x *= np.exp2(rng.uniform(-6, 6, (shape[0], 1)))
    if x.size:
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


# ---------------------------------------------------------------------------
# the other entry points: fused quantizing epilogues, power-of-two path,
# grouped backward, dispatch and combine
# ---------------------------------------------------------------------------

def _to(dev, *arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrays]


@pytest.mark.parametrize("seed", range(24))
def test_random_fused_epilogues(dev, seed):
    # 1x128 epilogue for any M; both layouts when M is a multiple of 128. The
    # fused codes and scales are the oracle's quantization of the GEMM's BF16 result.
    rng = np.random.default_rng(9300 + seed)
    both = seed % 2 == 1
    M = 128 * int(rng.integers(1, 7)) if both else int(rng.integers(1, 800))
    N, K = 128 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 9))
    mode = int(rng.integers(0, 2))
    A, B = _codes(rng, (M, K)), _codes(rng, (N, K))
    sA = _scales(rng, (K // 128, M))
    sB = _scales(rng, (N // 128, K // 128) if mode == MODE_BLOCK else (K // 128, N))
    args = (*_to(dev, A, sA, B, sB), mode)
    C = fb.fp8_gemm_blockscaled(*args)
    out = fb.fp8_gemm_blockscaled_q1x128_q128x1T(*args) if both else fb.fp8_gemm_blockscaled_q1x128(*args)
    torch.cuda.synchronize()
    what = f"seed {seed}: fused {'both' if both else '1x128'} {M}x{N}x{K} mode {mode}"
    ref, absref = oracle.gemm_ref(A, sA, B, sB, mode)
    _check(C, ref, absref, what + " BF16 result")
    qo, so = oracle.quant_act_1x128(bf16_bits(C))
    assert_codes_equal(u8(out[0]), qo, what + " 1x128 codes")
    assert_scales_equal(out[1].cpu().numpy(), so, what + " 1x128 scales")
    if both:
        qto, sto = oracle.quant_act_128x1_T(bf16_bits(C))
        assert_codes_equal(u8(out[2]), qto, what + " 128x1 codes")
        assert_scales_equal(out[3].cpu().numpy(), sto, what + " 128x1 scales")


@pytest.mark.parametrize("seed", range(24))
def test_random_pow2_path(dev, seed):
    # power-of-two quantizers bit for bit, then the MFMA-scaled GEMM on their outputs
    rng = np.random.default_rng(9400 + seed)
    M, N, K = int(rng.integers(1, 700)), 128 * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 9))
    dtype = ("bf16", "f32")[seed % 2]
    X, W = _values(rng, (M, K), dtype), _values(rng, (N, K), dtype)
    qx, sx = fb.fp8_quant_act_1x128(X.to(dev), pow2=True)
    qw, sw = fb.fp8_quant_w_128x128(W.to(dev), pow2=True)
    C = fb.fp8_gemm_blockscaled(qx, sx, qw, sw, MODE_BLOCK, pow2=True)
    torch.cuda.synchronize()
    what = f"seed {seed}: pow2 {M}x{N}x{K} {dtype}"
    qxo, sxo = oracle.quant_act_1x128(to_oracle(X), pow2=True)
    qwo, swo = oracle.quant_w_128x128(to_oracle(W), pow2=True)
    assert_codes_equal(u8(qx), qxo, what + " activation codes")
    assert_scales_equal(sx.cpu().numpy(), sxo, what + " activation scales")
    assert_codes_equal(u8(qw), qwo, what + " weight codes")
    assert_scales_equal(sw.cpu().numpy(), swo, what + " weight scales")
    ref, absref = oracle.gemm_ref(qxo, sxo, qwo, swo, MODE_BLOCK)
    _check(C, ref, absref, what + " GEMM")


@pytest.mark.parametrize("seed", range(16))
def test_random_grouped_backward(dev, seed):
    # BF16/F32 dY and X over ragged experts -> grouped 128x1 quantizers
    # (bit for bit) -> per-expert Wgrad on their outputs (within the bound)
    rng = np.random.default_rng(9500 + seed)
    counts = _expert_counts(rng)
    E = len(counts)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    M = int(off[-1])
    N, K = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 5))
    dtype = ("bf16", "f32")[seed % 2]
    dY, X = _values(rng, (M, N), dtype), _values(rng, (M, K), dtype)
    offd = torch.from_numpy(off).to(dev)
    qa, sa = fb.fp8_quant_act_128x1_T_grouped(dY.to(dev), offd)
    qb, sb = fb.fp8_quant_act_128x1_T_grouped(X.to(dev), offd)
    dW = fb.fp8_grouped_gemm_wgrad(qa, sa, qb, sb, offd, M)
    torch.cuda.synchronize()
    what = f"seed {seed}: grouped backward counts {counts.tolist()} N={N} K={K} {dtype}"
    qao, sao = oracle.quant_act_128x1_T_grouped(to_oracle(dY), off)
    qbo, sbo = oracle.quant_act_128x1_T_grouped(to_oracle(X), off)
    G = sao.shape[0]
    assert_codes_equal(u8(qa[:, :128 * G]), qao, what + " dY codes")
    assert_scales_equal(sa[:G].cpu().numpy(), sao, what + " dY scales")
    assert_codes_equal(u8(qb[:, :128 * G]), qbo, what + " X codes")
    assert_scales_equal(sb[:G].cpu().numpy(), sbo, what + " X scales")
    ref, absref = oracle.grouped_wgrad_ref(u8(qa), sa.cpu().numpy(), u8(qb), sb.cpu().numpy(), off)
    _check(dW, ref, absref, what + " Wgrad")


@pytest.mark.parametrize("seed", range(16))
def test_random_dispatch_and_combine(dev, seed):
    rng = np.random.default_rng(9600 + seed)
    T, K = int(rng.integers(1, 1500)), 128 * int(rng.integers(1, 9))
    E = int(rng.integers(1, 300))
    topk = int(rng.integers(1, min(E, 8) + 1))
    p = rng.dirichlet(np.full(E, 0.3)) + 1e-3
    p /= p.sum()
    ids = np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    dtype = ("bf16", "f32")[seed % 2]
    x = _values(rng, (T, K), dtype)
    q, s, off, pos, src = fb.fp8_moe_dispatch(x.to(dev), torch.from_numpy(ids).to(dev), E)
    torch.cuda.synchronize()
    what = f"seed {seed}: dispatch T={T} K={K} E={E} topk={topk} {dtype}"
    qo, so, offo, poso, srco = oracle.dispatch_quant(to_oracle(x), ids, E)
    assert np.array_equal(off.cpu().numpy(), offo), what + " offsets"
    assert np.array_equal(pos.cpu().numpy(), poso), what + " pos"
    assert np.array_equal(src.cpu().numpy(), srco), what + " src_row"
    assert_codes_equal(u8(q), qo, what + " codes")
    assert_scales_equal(s.cpu().numpy(), so, what + " scales")
    # combine expert outputs Y (BF16, in the dispatched row order) with random weights
    N = 128 * int(rng.integers(1, 9))
    Y = torch.from_numpy(rng.standard_normal((T * topk, N)).astype(np.float32) * 3).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((T, topk)).astype(np.float32))
    out = fb.fp8_moe_combine(Y.to(dev), pos, w.to(dev))
    torch.cuda.synchronize()
    ref, absref = oracle.combine_ref(oracle.bf16_bits_to_f64(bf16_bits(Y)), poso, w.numpy().astype(np.float64))
    ok, worst = oracle.check_combine(bf16_bits(out), ref, absref, topk)
    assert ok.all(), f"{what} combine: {int((~ok).sum())} outside the bound (worst {worst:.3g})"
