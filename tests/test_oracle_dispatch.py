"""Pins for the oracle's MoE dispatch payload and combine.

Checked against: an explicit loop that hands out rows expert by expert,
token by token, slot by slot (the stable order); torch's own 1x128 group
quantization of each row's source token (float32 division and the
float8_e4m3fn cast after clamping); and for the combine a per-element Python
loop plus an exactly representable case checked with rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import check_combine, combine_ref, dispatch_quant, route


def _ids(T, topk, E, seed):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.5))
    return np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int64)


def _route_by_loop(ids, E):
    T, topk = ids.shape
    pos = -np.ones((T, topk), np.int64)
    src, offsets, row = [], [0], 0
    for e in range(E):
        for t in range(T):
            for j in range(topk):
                if ids[t, j] == e:
                    pos[t, j] = row
                    src.append(t)
                    row += 1
        offsets.append(row)
    return np.array(offsets), pos, np.array(src, np.int64)


@pytest.mark.parametrize("T,topk,E", [(1, 1, 1), (37, 4, 8), (200, 8, 32), (64, 2, 3)])
def test_route_matches_the_explicit_stable_loop(T, topk, E):
    ids = _ids(T, topk, E, T + E)
    off, pos, src = route(ids, E)
    off2, pos2, src2 = _route_by_loop(ids, E)
    assert np.array_equal(off, off2) and np.array_equal(pos, pos2) and np.array_equal(src, src2)


def test_route_with_repeated_experts_in_a_token():
    ids = np.array([[2, 2, 0], [0, 2, 2]])
    off, pos, src = route(ids, 3)
    assert list(off) == [0, 2, 2, 6]
    assert pos.tolist() == [[2, 3, 0], [1, 4, 5]]
    assert src.tolist() == [0, 1, 0, 0, 1, 1]
    with pytest.raises(ValueError):
        route(np.array([[3]]), 3)


def test_dispatch_payload_is_each_tokens_group_quantization():
    T, K, topk, E = 50, 384, 4, 6
    rng = np.random.default_rng(1)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[rng.random((T, K)) < 0.02] *= 80.0
    x[7] = 0.0                                        # a zero token: scale 1, codes 0
    ids = _ids(T, topk, E, 2)
    q, s, off, pos, src = dispatch_quant(x, ids, E)
    assert q.shape == (T * topk, K) and s.shape == (K // 128, T * topk)
    g = torch.from_numpy(x).reshape(T, K // 128, 128)
    amax = g.abs().amax(dim=2)
    st = amax / torch.tensor(448.0)
    st = torch.where(st == 0, torch.ones_like(st), st)
    codes = (g / st[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(T, K)
    for r in range(T * topk):
        t = src[r]
        assert np.array_equal(q[r], codes[t].numpy())
        assert np.array_equal(s[:, r].view(np.uint32), st[t].numpy().view(np.uint32))
    for t in range(T):
        for j in range(topk):
            assert src[pos[t, j]] == t and off[ids[t, j]] <= pos[t, j] < off[ids[t, j] + 1]


def test_combine_matches_a_per_element_loop():
    rng = np.random.default_rng(3)
    T, topk, N = 9, 3, 16
    Y = rng.standard_normal((T * topk, N))
    pos = rng.permutation(T * topk).reshape(T, topk)
    w = rng.random((T, topk))
    ref, absref = combine_ref(Y, pos, w)
    for t in range(T):
        for n in range(N):
            want = sum(w[t, j] * Y[pos[t, j], n] for j in range(topk))
            assert abs(ref[t, n] - want) <= 1e-12 * absref[t, n]
            assert abs(absref[t, n] - sum(abs(w[t, j] * Y[pos[t, j], n]) for j in range(topk))) <= 1e-12 * absref[t, n]


def test_combine_exact_case_and_bound():
    # weights 2^-k and small-integer Y: every sum is exact in float64
    rng = np.random.default_rng(4)
    T, topk, N = 5, 4, 8
    Y = rng.integers(-50, 51, (T * topk, N)).astype(np.float64)
    pos = rng.permutation(T * topk).reshape(T, topk)
    w = 2.0 ** -rng.integers(0, 4, (T, topk))
    ref, absref = combine_ref(Y, pos, w)
    for t in range(T):
        for n in range(N):
            exact = sum(Fraction(w[t, j]) * Fraction(Y[pos[t, j], n]) for j in range(topk))
            assert Fraction(ref[t, n]) == exact
    # the bound accepts the exact value in BF16 when representable, rejects a wrong slot
    bits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok, _ = check_combine(bits, ref, absref, topk)
    assert ok.all()
    wrong, _ = combine_ref(Y, pos[:, ::-1], w)
    bits = torch.from_numpy(wrong.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok, _ = check_combine(bits, ref, absref, topk)
    assert not ok.all()
