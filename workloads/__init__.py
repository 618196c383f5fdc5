"""Seeded synthetic inputs for the FP8 block-scaled GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no GEMM). Both the HIP path and the CPU
oracle consume what it returns.

Recipe (every draw comes from one torch.Generator seeded with ``seed`` on
the target device, in the order listed; the MoE routing draw uses
numpy.random.default_rng(seed) on the host). "N(0, sigma)" means standard
deviation sigma. Values are drawn in float32 and, where the workload says
BF16, cast to bfloat16 by torch (round to nearest even).

  tiny_fprop      X[256][1024] f32 N(0,1), 4 random columns x100;
                  W[512][1024] f32 N(0,0.02)
  dense_fprop     X[4096][7168] bf16 N(0,1), 1% (72) random columns x50;
                  W[7168][7168] bf16 N(0,0.006)
  moe_topk        8192 tokens, p ~ Dirichlet(0.5 * 1_32), each token picks 8
                  distinct experts without replacement with probabilities p
                  (numpy rng(seed)); weights = p of the picks, renormalised
  moe_routing     moe_topk's picks grouped by expert -> per-expert counts and
                  offsets
  moe_dispatch    moe_topk's picks and weights; X[8192][7168] bf16 N(0,1);
                  Y[65536][7168] bf16 N(0,1) (the experts' outputs)
  grouped_moe     A_up[sum][7168], A_dn[sum][2048] bf16 N(0,1);
                  W_up[32][4096][7168], W_dn[32][7168][2048] bf16 N(0,0.01)
  decode_grouped  32 experts, M_e uniform in 1..256 (numpy rng(seed));
                  A[sum][7168] bf16 N(0,1); W[32][4096][7168] bf16 N(0,0.01)
  grouped_moe_backward
                  grouped_moe's routing, activations and weights (same seed),
                  then dY_up[sum][4096] and dY_dn[sum][7168] bf16 N(0,1e-3),
                  each with 1% of its rows (random) x100
  backward_pair   dY[4096][7168] bf16 N(0,1e-3) with 1% (41) random rows x100;
                  X[4096][7168] bf16 N(0,1) with 4 random columns x100;
                  W as dense_fprop's weight (same draw with the same seed)

The per-workload functions accept smaller shapes so the same recipe can be
used at test sizes.
"""

import numpy as np
import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, g, device, dtype=torch.float32):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype) if dtype != torch.float32 else t


def _pick(n, k, g, device):
    return torch.randperm(n, generator=g, device=device)[:k]


def tiny_fprop(device="cpu", seed=0, M=256, N=512, K=1024, n_outlier_cols=4):
    g = _gen(device, seed)
    X = _randn((M, K), 1.0, g, device)
    cols = _pick(K, n_outlier_cols, g, device)
    X[:, cols] *= 100.0
    W = _randn((N, K), 0.02, g, device)
    return {"X": X, "W": W}


def dense_fprop(device="cpu", seed=0, M=4096, N=7168, K=7168, outlier_frac=0.01,
                outlier_mult=50.0):
    g = _gen(device, seed)
    X = _randn((M, K), 1.0, g, device)
    cols = _pick(K, int(round(outlier_frac * K)), g, device)
    X[:, cols] *= outlier_mult
    X = X.to(torch.bfloat16)
    W = _randn((N, K), 0.006, g, device, torch.bfloat16)
    return {"X": X, "W": W}


def moe_topk(seed=0, tokens=8192, experts=32, topk=8, alpha=0.5):
    """Expert ids [tokens][topk] (int32) and routing weights [tokens][topk]
    (float32, the draw's probabilities renormalised over each token's experts)."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(experts, alpha))
    ids = np.empty((tokens, topk), np.int32)
    for t in range(tokens):
        ids[t] = rng.choice(experts, topk, replace=False, p=p)
    w = p[ids]
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def moe_routing(seed=0, tokens=8192, experts=32, topk=8, alpha=0.5):
    """Per-expert row counts and int32 offsets[E+1] of the expert-sorted rows."""
    ids, _ = moe_topk(seed, tokens, experts, topk, alpha)
    counts = np.bincount(ids.reshape(-1), minlength=experts).astype(np.int64)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def moe_dispatch(device="cpu", seed=0, tokens=8192, experts=32, topk=8, alpha=0.5, d_model=7168):
    """Token activations, their routing and the experts' outputs to combine."""
    ids, w = moe_topk(seed, tokens, experts, topk, alpha)
    g = _gen(device, seed + 3)
    X = _randn((tokens, d_model), 1.0, g, device, torch.bfloat16)
    Y = _randn((tokens * topk, d_model), 1.0, g, device, torch.bfloat16)
    return {"ids": ids, "w": w, "X": X, "Y": Y}


def grouped_moe(device="cpu", seed=0, tokens=8192, experts=32, topk=8, alpha=0.5,
                d_model=7168, d_ff2=4096, d_ff=2048, with_weights=True):
    counts, offsets = moe_routing(seed, tokens, experts, topk, alpha)
    total = int(offsets[-1])
    g = _gen(device, seed)
    out = {"counts": counts, "offsets": offsets}
    out["A_up"] = _randn((total, d_model), 1.0, g, device, torch.bfloat16)
    out["A_dn"] = _randn((total, d_ff), 1.0, g, device, torch.bfloat16)
    if with_weights:
        out["W_up"] = _randn((experts, d_ff2, d_model), 0.01, g, device, torch.bfloat16)
        out["W_dn"] = _randn((experts, d_model, d_ff), 0.01, g, device, torch.bfloat16)
    return out


def grouped_moe_backward(device="cpu", seed=0, tokens=8192, experts=32, topk=8, alpha=0.5,
                         d_model=7168, d_ff2=4096, d_ff=2048, outlier_row_frac=0.01):
    """grouped_moe's inputs plus the output gradients of the up and down GEMMs."""
    out = grouped_moe(device, seed, tokens, experts, topk, alpha, d_model, d_ff2, d_ff)
    total = int(out["offsets"][-1])
    g = _gen(device, seed + 2)
    for key, width in (("dY_up", d_ff2), ("dY_dn", d_model)):
        dY = _randn((total, width), 1e-3, g, device)
        rows = _pick(total, int(round(outlier_row_frac * total)), g, device)
        dY[rows, :] *= 100.0
        out[key] = dY.to(torch.bfloat16)
    return out


def decode_counts(seed=0, experts=32, max_tokens=256):
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, max_tokens + 1, experts).astype(np.int64)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def decode_grouped(device="cpu", seed=0, experts=32, N=4096, K=7168, max_tokens=256):
    counts, offsets = decode_counts(seed, experts, max_tokens)
    total = int(offsets[-1])
    g = _gen(device, seed)
    A = _randn((total, K), 1.0, g, device, torch.bfloat16)
    W = _randn((experts, N, K), 0.01, g, device, torch.bfloat16)
    return {"counts": counts, "offsets": offsets, "A": A, "W": W}


def backward_pair(device="cpu", seed=0, M=4096, N=7168, K=7168, outlier_row_frac=0.01,
                  n_outlier_cols=4):
    """dY[M][N] (gradient of the Fprop output), X[M][K], W[N][K]."""
    g = _gen(device, seed + 1)
    dY = _randn((M, N), 1e-3, g, device)
    rows = _pick(M, int(round(outlier_row_frac * M)), g, device)
    dY[rows, :] *= 100.0
    dY = dY.to(torch.bfloat16)
    X = _randn((M, K), 1.0, g, device)
    cols = _pick(K, n_outlier_cols, g, device)
    X[:, cols] *= 100.0
    X = X.to(torch.bfloat16)
    W = dense_fprop(device, seed, M=M, N=N, K=K)["W"]
    return {"dY": dY, "X": X, "W": W}


def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def ceil_div(a, b):
    return -(-a // b)


__all__ = ["tiny_fprop", "dense_fprop", "moe_topk", "moe_routing", "moe_dispatch", "grouped_moe", "grouped_moe_backward", "decode_counts",
           "decode_grouped", "backward_pair", "gemm_flops", "ceil_div"]
