"""GPU parity of the MoE dispatch payload (routing bit for bit, FP8 codes and
scales bit for bit) and of the BF16 combine (within its FP32-sum bound)
against the oracle, plus the chain dispatch -> grouped GEMM -> combine."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_codes_equal, assert_scales_equal, bf16_bits, to_oracle, u8

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _ids(T, topk, E, seed, distinct=True):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.5))
    if distinct and topk <= E:
        return np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    return rng.choice(E, (T, topk), p=p).astype(np.int32)


def _x(T, K, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, K), generator=g)
    x[torch.rand((T, K), generator=g) < 0.01] *= 100.0
    if T > 3:
        x[3] = 0.0
    return x.to(dtype)


def _check_dispatch(dev, x, ids, E, what):
    q, s, off, pos, src = fb.fp8_moe_dispatch(x.to(dev), torch.from_numpy(ids).to(dev), E)
    torch.cuda.synchronize()
    qo, so, offo, poso, srco = oracle.dispatch_quant(to_oracle(x), ids, E)
    assert np.array_equal(off.cpu().numpy(), offo), f"{what}: offsets"
    assert np.array_equal(pos.cpu().numpy(), poso), f"{what}: pos"
    assert np.array_equal(src.cpu().numpy(), srco), f"{what}: src_row"
    assert_codes_equal(u8(q), qo, f"{what}: codes")
    assert_scales_equal(s.cpu().numpy(), so, f"{what}: scales")
    return q, s, off, pos, src


@pytest.mark.parametrize("T,K,topk,E", [
    (1, 128, 1, 1), (37, 256, 4, 8), (200, 384, 8, 32), (1000, 128, 8, 256), (1500, 128, 2, 1024),
    (2049, 256, 6, 9), (2200, 128, 8, 1024),
])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dispatch_random(dev, T, K, topk, E, dtype):
    _check_dispatch(dev, _x(T, K, T + K, dtype), _ids(T, topk, E, T * E), E, f"dispatch T={T} K={K} topk={topk} E={E}")


def test_dispatch_repeated_experts_in_a_token(dev):
    # the stable order holds also when a token picks an expert twice
    ids = _ids(300, 6, 4, 1, distinct=False)
    _check_dispatch(dev, _x(300, 128, 5, torch.bfloat16), ids, 4, "dispatch with repeats")


def test_dispatch_no_tokens_and_no_columns(dev):
    q, s, off, pos, src = fb.fp8_moe_dispatch(torch.zeros((0, 128), dtype=torch.bfloat16, device=dev),
                                              torch.zeros((0, 4), dtype=torch.int32, device=dev), 5)
    torch.cuda.synchronize()
    assert q.shape == (0, 128) and torch.all(off == 0)
    ids = _ids(20, 3, 5, 2)
    q, s, off, pos, src = fb.fp8_moe_dispatch(torch.zeros((20, 0), dtype=torch.bfloat16, device=dev),
                                              torch.from_numpy(ids).to(dev), 5)
    offo, poso, srco = oracle.route(ids, 5)
    assert np.array_equal(off.cpu().numpy(), offo) and np.array_equal(pos.cpu().numpy(), poso)


@pytest.mark.parametrize("T,topk,N", [(1, 1, 8), (100, 8, 256), (333, 3, 7168), (64, 2, 1000)])
def test_combine_random(dev, T, topk, N):
    g = torch.Generator().manual_seed(T + N)
    Y = (torch.randn((T * topk, N), generator=g) * 3).to(torch.bfloat16)
    pos = torch.randperm(T * topk, generator=g).to(torch.int32).reshape(T, topk)
    w = torch.rand((T, topk), generator=g)
    out = fb.fp8_moe_combine(Y.to(dev), pos.to(dev), w.to(dev))
    torch.cuda.synchronize()
    ref, absref = oracle.combine_ref(oracle.bf16_bits_to_f64(bf16_bits(Y)), pos.numpy(), w.numpy().astype(np.float64))
    ok, worst = oracle.check_combine(bf16_bits(out), ref, absref, topk)
    assert ok.all(), f"combine T={T} topk={topk} N={N}: {int((~ok).sum())} outside the bound (worst {worst:.3g})"


def test_dispatch_gemm_combine_chain(dev):
    # x -> FP8 payload -> per-expert GEMM -> weighted combine, each stage
    # against the oracle on the previous stage's GPU output
    T, K, N, topk, E = 300, 256, 384, 4, 6
    x = _x(T, K, 9, torch.bfloat16)
    ids = _ids(T, topk, E, 10)
    q, s, off, pos, src = _check_dispatch(dev, x, ids, E, "chain dispatch")
    g = torch.Generator().manual_seed(11)
    W = (torch.randn((E, N, K), generator=g) * 0.05).to(torch.bfloat16).to(dev)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        qw[e], sw[e] = fb.fp8_quant_w_128x128(W[e])
    Y = fb.fp8_grouped_gemm_blockscaled(q, s, qw, sw, off)
    w = torch.rand((T, topk), generator=g)
    out = fb.fp8_moe_combine(Y, pos, w.to(dev))
    torch.cuda.synchronize()
    ref, absref = oracle.grouped_gemm_ref(u8(q), s.cpu().numpy(), u8(qw), sw.cpu().numpy(), off.cpu().numpy())
    ok, worst = oracle.check_gemm(bf16_bits(Y), ref, absref)
    assert ok.all(), f"chain grouped GEMM outside the bound (worst {worst:.3g})"
    cref, cabs = oracle.combine_ref(oracle.bf16_bits_to_f64(bf16_bits(Y)), pos.cpu().numpy(),
                                    w.numpy().astype(np.float64))
    ok, worst = oracle.check_combine(bf16_bits(out), cref, cabs, topk)
    assert ok.all(), f"chain combine outside the bound (worst {worst:.3g})"


def test_dispatch_combine_workload(dev):
    # 8192 tokens x top-8 of 32 experts (Dirichlet(0.5) popularity), K = 7168
    d = workloads.moe_dispatch(device=dev)
    ids, E = d["ids"], 32
    q, s, off, pos, src = fb.fp8_moe_dispatch(d["X"], torch.from_numpy(ids).to(dev), E)
    out = fb.fp8_moe_combine(d["Y"], pos, torch.from_numpy(d["w"]).to(dev))
    torch.cuda.synchronize()
    offo, poso, srco = oracle.route(ids, E)
    assert np.array_equal(off.cpu().numpy(), offo)
    assert np.array_equal(pos.cpu().numpy(), poso)
    assert np.array_equal(src.cpu().numpy(), srco)
    # payload rows of a sample of tokens, all their copies
    toks = np.array([0, 1, 3, 4095, 8190, 8191])
    qt, st = oracle.quant_act_1x128(to_oracle(d["X"][toks]))
    for i, t in enumerate(toks):
        rows = poso[t]
        for r in rows:
            assert_codes_equal(u8(q[int(r)]), qt[i], f"payload row {r} (token {t})")
            assert_scales_equal(s[:, int(r)].cpu().numpy(), st[:, i], f"payload scales row {r} (token {t})")
    # combine of the sampled tokens
    Ys = oracle.bf16_bits_to_f64(bf16_bits(d["Y"][torch.from_numpy(poso[toks].reshape(-1)).to(dev)]))
    ref, absref = oracle.combine_ref(Ys, np.arange(len(toks) * 8).reshape(len(toks), 8),
                                     d["w"][toks].astype(np.float64))
    ok, worst = oracle.check_combine(bf16_bits(out[torch.from_numpy(toks).to(dev)]), ref, absref, 8)
    assert ok.all(), f"combine workload outside the bound (worst {worst:.3g})"


def test_dispatch_rejects_bad_arguments(dev):
    L = fb.lib()
    s = torch.cuda.current_stream().cuda_stream
    buf = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    p = buf.data_ptr()
    assert L.fp8_moe_dispatch_workspace_bytes(10, 8, 0) < 0
    assert L.fp8_moe_dispatch_workspace_bytes(10, 65, 4) < 0
    assert L.fp8_moe_dispatch_workspace_bytes(10, 8, 1025) < 0
    assert L.fp8_moe_dispatch(p, 1, 10, 100, p, 2, 4, p, p, p, p, p, p, s) != 0      # K % 128
    assert L.fp8_moe_dispatch(p, 1, 10, 128, p, 0, 4, p, p, p, p, p, p, s) != 0      # topk 0
    assert L.fp8_moe_dispatch(p, 7, 10, 128, p, 2, 4, p, p, p, p, p, p, s) != 0      # dtype
    assert L.fp8_moe_dispatch(p, 1, 10, 128, p, 2, 4, p, p, None, p, p, p, s) != 0   # offsets
    assert L.fp8_moe_dispatch(p, 1, 10, 128, p, 2, 4, p, p, p, p, p, None, s) != 0   # workspace
    assert L.fp8_moe_combine(p, p, p, 10, 2, 12, p, s) != 0                          # N % 8
    assert L.fp8_moe_combine(p + 2, p, p, 10, 2, 16, p, s) != 0                      # alignment
    torch.cuda.synchronize()
