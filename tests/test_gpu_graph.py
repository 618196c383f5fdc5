"""HIP graph capture of the path. The C-ABI entry points allocate nothing and
make no memset or synchronizing calls, so a step captured into a graph must
replay to the same bytes as eager calls on the same inputs. Each graph is
replayed several times with its inputs changed in place, its outputs cleared
and other eager work and synchronizations between replays, and every replay
is compared with an eager run."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _capture(fn):
    """fn(stream) launched once on a side stream (warm-up), then captured."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream().cuda_stream)
    return g


def test_graph_fprop_step(dev):
    # quantize X 1x128 and W 128x128, then the block-scaled GEMM; ragged M
    M, N, K = 1000, 768, 1024
    L = fb.lib()
    g = torch.Generator(device=dev).manual_seed(0)
    inputs = [((torch.randn(M, K, device=dev, generator=g) * (i + 1)).to(torch.bfloat16),
               (torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)) for i in range(3)]

    def buffers():
        return {"qx": torch.empty((M, K), dtype=torch.uint8, device=dev),
                "sx": torch.empty((K // 128, M), dtype=torch.float32, device=dev),
                "qw": torch.empty((N, K), dtype=torch.uint8, device=dev),
                "sw": torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
                "C": torch.empty((M, N), dtype=torch.bfloat16, device=dev)}

    def step(X, W, b, stream):
        assert L.fp8_quant_act_1x128(X.data_ptr(), fb.BF16, M, K, b["qx"].data_ptr(), b["sx"].data_ptr(), stream) == 0
        assert L.fp8_quant_w_128x128(W.data_ptr(), fb.BF16, N, K, b["qw"].data_ptr(), b["sw"].data_ptr(),
                                     None, None, stream) == 0
        assert L.fp8_gemm_blockscaled(b["qx"].data_ptr(), b["sx"].data_ptr(), b["qw"].data_ptr(), b["sw"].data_ptr(),
                                      fb.SCALE_BLOCK128, b["C"].data_ptr(), M, N, K, stream) == 0

    refs = []
    eager = buffers()
    for X, W in inputs:
        step(X, W, eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        refs.append({k: v.clone() for k, v in eager.items()})

    Xs, Ws = inputs[0][0].clone(), inputs[0][1].clone()
    b = buffers()
    graph = _capture(lambda stream: step(Xs, Ws, b, stream))
    for rep in range(6):
        i = (rep * 2) % 3
        Xs.copy_(inputs[i][0])
        Ws.copy_(inputs[i][1])
        for v in b.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in b:
            assert _same(b[k], refs[i][k]), f"replay {rep}: {k} differs from the eager result"
        # eager work between replays, on other buffers
        X, W = inputs[(i + 1) % 3]
        step(X, W, eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert _same(eager["C"], refs[(i + 1) % 3]["C"])


def test_graph_moe_dispatch_gemm_combine(dev):
    # route + FP8 payload, per-expert GEMM, BF16 combine; the routing
    # workspace is a caller buffer, the expert offsets stay on the device
    T, K, N, topk, E = 300, 256, 384, 4, 6
    L = fb.lib()
    rng = np.random.default_rng(3)
    g = torch.Generator(device=dev).manual_seed(1)
    inputs = []
    for i in range(3):
        p = rng.dirichlet(np.full(E, 0.5))
        ids = np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        x = torch.randn(T, K, device=dev, generator=g).to(torch.bfloat16)
        w = torch.rand(T, topk, device=dev, generator=g)
        inputs.append((x, torch.from_numpy(ids).to(dev), w))
    Wt = (torch.randn(E, N, K, device=dev, generator=g) * 0.05).to(torch.bfloat16)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
    for e in range(E):
        qw[e], sw[e] = fb.fp8_quant_w_128x128(Wt[e])
    ws_bytes = L.fp8_moe_dispatch_workspace_bytes(T, topk, E)
    assert ws_bytes >= 0

    def buffers():
        P = T * topk
        return {"ws": torch.empty(max(ws_bytes // 4, 1), dtype=torch.int32, device=dev),
                "q": torch.empty((P, K), dtype=torch.uint8, device=dev),
                "s": torch.empty((K // 128, P), dtype=torch.float32, device=dev),
                "off": torch.empty(E + 1, dtype=torch.int32, device=dev),
                "pos": torch.empty((T, topk), dtype=torch.int32, device=dev),
                "src": torch.empty(P, dtype=torch.int32, device=dev),
                "Y": torch.empty((P, N), dtype=torch.bfloat16, device=dev),
                "out": torch.empty((T, N), dtype=torch.bfloat16, device=dev)}

    def step(x, ids, w, b, stream):
        assert L.fp8_moe_dispatch(x.data_ptr(), fb.BF16, T, K, ids.data_ptr(), topk, E, b["q"].data_ptr(),
                                  b["s"].data_ptr(), b["off"].data_ptr(), b["pos"].data_ptr(), b["src"].data_ptr(),
                                  b["ws"].data_ptr(), stream) == 0
        assert L.fp8_grouped_gemm_blockscaled(b["q"].data_ptr(), b["s"].data_ptr(), qw.data_ptr(), sw.data_ptr(),
                                              b["Y"].data_ptr(), b["off"].data_ptr(), E, T * topk, N, K, stream) == 0
        assert L.fp8_moe_combine(b["Y"].data_ptr(), b["pos"].data_ptr(), w.data_ptr(), T, topk, N,
                                 b["out"].data_ptr(), stream) == 0

    refs = []
    eager = buffers()
    for x, ids, w in inputs:
        step(x, ids, w, eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        refs.append({k: v.clone() for k, v in eager.items() if k != "ws"})

    xs, idss, wss = (t.clone() for t in inputs[0])
    b = buffers()
    graph = _capture(lambda stream: step(xs, idss, wss, b, stream))
    for rep in range(6):
        i = (rep * 2) % 3
        xs.copy_(inputs[i][0])
        idss.copy_(inputs[i][1])
        wss.copy_(inputs[i][2])
        for k, v in b.items():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in refs[i]:
            assert _same(b[k], refs[i][k]), f"replay {rep}: {k} differs from the eager result"
        x, ids, w = inputs[(i + 1) % 3]
        step(x, ids, w, eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert _same(eager["out"], refs[(i + 1) % 3]["out"])


def test_graph_grouped_gemm_tile_and_tail_routes(dev):
    # the grouped GEMM's tile kernel and its tail launch decide on the device,
    # from the offsets, which tiles the tail takes: one captured graph must
    # follow offsets that change between replays (on 256 CUs: a round of 256
    # tiles and a tail of 32, for two expert splits; a round and a tail of 8;
    # no tail, with 80 tiles past the round left to the tile kernel)
    E, M, N, K = 4, 2800, 6144, 256
    routes = [[700, 700, 700, 700], [2800, 0, 0, 0], [1, 1, 1, 2797], [900, 900, 500, 500]]
    g = torch.Generator(device=dev).manual_seed(5)
    A = torch.randint(0, 256, (M, K), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3B
    B = torch.randint(0, 256, (E, N, K), generator=g, device=dev, dtype=torch.int32).to(torch.uint8)
    B[(B & 0x7F) == 0x7F] = 0x3B
    sA = 1e-2 + torch.rand((K // 128, M), generator=g, device=dev)
    sB = 1e-2 + torch.rand((E, N // 128, K // 128), generator=g, device=dev)
    offs = [torch.from_numpy(np.concatenate([[0], np.cumsum(c)]).astype(np.int32)).to(dev) for c in routes]
    L = fb.lib()

    def gemm(off, C, stream):
        assert L.fp8_grouped_gemm_blockscaled(A.data_ptr(), sA.data_ptr(), B.data_ptr(), sB.data_ptr(), C.data_ptr(),
                                              off.data_ptr(), E, M, N, K, stream) == 0

    refs = []
    for off in offs:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gemm(off, C, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        refs.append(C)
    off_g = offs[0].clone()
    C_g = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    graph = _capture(lambda stream: gemm(off_g, C_g, stream))
    for rep in range(8):
        i = (3 * rep + 1) % len(routes)
        off_g.copy_(offs[i])
        C_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(C_g, refs[i]), f"replay {rep}: route {routes[i]} differs from the eager result"
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gemm(offs[(i + 1) % len(routes)], C, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert _same(C, refs[(i + 1) % len(routes)])
