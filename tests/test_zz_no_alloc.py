"""The no-allocation MoE dispatch (fp8_moe_dispatch_noalloc, routing workspace
in the library's own device array) against fp8_moe_dispatch with a caller
workspace, through the C ABI: routing and payload are integer and byte work,
so every output must be identical, on two calls in a row, the second smaller
(the scratch array keeps the first call's contents)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _case(dev, T, K, topk, E, seed, dtype):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.5))
    ids = np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn((T, K), generator=g, device=dev).to(dtype)
    ids_d = torch.from_numpy(ids).to(dev)
    ref = fb.fp8_moe_dispatch(x, ids_d, E)
    P = T * topk
    # outputs prefilled with a pattern the kernels never produce everywhere
    out = (torch.full((P, K), 0x7F, dtype=torch.uint8, device=dev),
           torch.full((K // 128, P), float("nan"), device=dev),
           torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
           torch.full((T, topk), -7, dtype=torch.int32, device=dev),
           torch.full((P,), -7, dtype=torch.int32, device=dev))
    got = fb.fp8_moe_dispatch_noalloc(x, ids_d, E, *out)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "s", "offsets", "pos", "src_row"), got, ref):
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"T={T} K={K} topk={topk} E={E}: {name} differs from fp8_moe_dispatch"


def test_noalloc_dispatch_matches_dispatch_on_two_calls(dev):
    _case(dev, 8192, 7168, 8, 32, 0, torch.bfloat16)       # the 8192-token top-8 workload
    _case(dev, 1000, 1024, 6, 64, 1, torch.float32)        # then a smaller one, other E, topk, dtype


def test_noalloc_dispatch_rejects_oversized_workspace(dev):
    T, topk, E, K = 257 * 128, 8, 1024, 128                 # 4 * 1024 * 257 bytes > 1 MiB
    x = torch.zeros((T, K), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((T, topk), dtype=torch.int32, device=dev)
    out = (torch.empty((T * topk, K), dtype=torch.uint8, device=dev), torch.empty((1, T * topk), device=dev),
           torch.empty((E + 1,), dtype=torch.int32, device=dev), torch.empty((T, topk), dtype=torch.int32, device=dev),
           torch.empty((T * topk,), dtype=torch.int32, device=dev))
    with pytest.raises(fb.Fp8bsError) as ei:
        fb.fp8_moe_dispatch_noalloc(x, ids, E, *out)
    assert ei.value.status == -8
