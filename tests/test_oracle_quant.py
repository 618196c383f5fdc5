"""Pins for the oracle's group quantizers.

Checked against: exactly known power-of-two groups, an exact rational
computation of the scale, torch's independent float32 division and
float8_e4m3fn cast, sign and power-of-two invariants, the group geometry
(changing one element only changes its own group), and the identities
between the three layouts.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (e4m3_decode, quant_act_1x128, quant_act_128x1_T, quant_w_128x128)


def _pow2_group_data(rng, shape, group_view, j):
    """Random finite codes with one 448 per group, scaled by 2^j."""
    codes = rng.integers(0, 256, shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    g = group_view(codes)
    g[..., 0] = np.where(rng.random(g.shape[:-1]) < 0.5, 0x7E, 0xFE)
    x = (e4m3_decode(codes) * 2.0 ** j).astype(np.float32)
    return codes, x


def test_pow2_groups_exact_1x128():
    rng = np.random.default_rng(0)
    for j in (-20, -3, 0, 5, 20):
        codes, x = _pow2_group_data(rng, (7, 384), lambda c: c.reshape(7, 3, 128), j)
        q, s = quant_act_1x128(x)
        assert np.array_equal(q, codes)
        assert s.shape == (3, 7) and np.all(s == np.float32(2.0 ** j))


def test_pow2_groups_exact_128x128():
    rng = np.random.default_rng(1)
    for j in (-15, 0, 9):
        codes = rng.integers(0, 256, (256, 384)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11
        for nb in range(2):
            for kb in range(3):
                codes[nb * 128 + 5, kb * 128 + 7] = 0xFE
        x = (e4m3_decode(codes) * 2.0 ** j).astype(np.float32)
        q, s, qT, sT = quant_w_128x128(x, transposed=True)
        assert np.array_equal(q, codes)
        assert s.shape == (2, 3) and np.all(s == np.float32(2.0 ** j))
        assert np.array_equal(qT, codes.T) and np.array_equal(sT, s.T)


def test_pow2_groups_exact_128x1_T():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, (256, 5)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x01
    codes[3, :] = 0x7E
    codes[130, :] = 0xFE
    x = (e4m3_decode(codes) * 2.0 ** -7).astype(np.float32)
    qT, sT = quant_act_128x1_T(x)
    assert qT.shape == (5, 256) and sT.shape == (2, 5)
    assert np.array_equal(qT, codes.T)
    assert np.all(sT == np.float32(2.0 ** -7))


def _f32_round(fr):
    """Nearest float32 to a Fraction (ties to even), by exhaustive neighbour search."""
    f = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(3)
    amaxes = np.concatenate([rng.standard_normal(200).astype(np.float32) ** 2 * 10,
                             np.array([1.0, 448.0, 3.0e38, 1e-30, 1e-40, 7.0], np.float32)])
    x = np.zeros((len(amaxes), 128), np.float32)
    x[:, 17] = -amaxes
    _, s = quant_act_1x128(x)
    for i, a in enumerate(amaxes):
        expect = _f32_round(Fraction(float(a)) / 448)
        if expect == 0:
            expect = np.float32(1.0)
        assert s[0, i] == expect, (a, s[0, i], expect)


def test_zero_and_negative_zero_groups():
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = -0.0
    q, s = quant_act_1x128(x)
    assert np.all(s == 1.0)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0x80) and np.all(q[1, 128:] == 0)


def test_matches_torch_division_and_cast():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 1024)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    x[:, 37] *= 100
    q, s = quant_act_1x128(x)
    xt = torch.from_numpy(x).reshape(64, 8, 128)
    amax = xt.abs().amax(dim=2)
    st = amax / torch.tensor(448.0, dtype=torch.float32)
    st = torch.where(st == 0, torch.ones_like(st), st)
    y = xt / st[:, :, None]
    qt = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 1024).numpy()
    assert np.array_equal(s, st.numpy().T)
    assert np.array_equal(q, qt)


def test_negation_and_pow2_scaling_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 512)).astype(np.float32)
    q, s = quant_act_1x128(x)
    qn, sn = quant_act_1x128(-x)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)
    for j in (-30, 7, 40):
        q2, s2 = quant_act_1x128((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_group_geometry_locality():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((256, 256)).astype(np.float32)
    # 1x128: bump one element of group (m=3, kb=1)
    q0, s0 = quant_act_1x128(x)
    y = x.copy(); y[3, 200] = 1000.0
    q1, s1 = quant_act_1x128(y)
    diff_s = np.argwhere(s1 != s0)
    assert diff_s.tolist() == [[1, 3]]
    dq = np.argwhere(q1 != q0)
    assert set(map(tuple, dq[:, :1].tolist())) == {(3,)} and dq[:, 1].min() >= 128
    # 128x128: bump element of block (nb=1, kb=0)
    q0, s0 = quant_w_128x128(x)
    y = x.copy(); y[140, 5] = 1000.0
    q1, s1 = quant_w_128x128(y)
    assert np.argwhere(s1 != s0).tolist() == [[1, 0]]
    dq = np.argwhere(q1 != q0)
    assert dq[:, 0].min() >= 128 and dq[:, 1].max() < 128
    # 128x1: bump element of group (tb=1, c=9)
    q0, s0 = quant_act_128x1_T(x)
    y = x.copy(); y[130, 9] = 1000.0
    q1, s1 = quant_act_128x1_T(y)
    assert np.argwhere(s1 != s0).tolist() == [[1, 9]]
    dq = np.argwhere(q1 != q0)
    assert set(dq[:, 0].tolist()) == {9} and dq[:, 1].min() >= 128


def test_layout_identities():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((384, 256)).astype(np.float32)
    x[:, 11] *= 300
    qT, sT = quant_act_128x1_T(x)
    q, s = quant_act_1x128(np.ascontiguousarray(x.T))
    assert np.array_equal(qT, q) and np.array_equal(sT, s)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    qa, sa, qTa, sTa = quant_w_128x128(w, transposed=True)
    qb, sb = quant_w_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(qTa, qb) and np.array_equal(sTa, sb)


def test_bf16_bits_input_equals_widened_float():
    rng = np.random.default_rng(8)
    xb = torch.from_numpy(rng.standard_normal((5, 256)).astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    q1, s1 = quant_act_1x128(bits)
    q2, s2 = quant_act_1x128(xb.to(torch.float32).numpy())
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_dequantized_error_within_half_e4m3_step():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, 1024)).astype(np.float32)
    q, s = quant_act_1x128(x)
    deq = e4m3_decode(q) * np.repeat(s.T, 128, axis=1)
    # relative spacing of E4M3 normals is 2^-3, so half a step is 2^-4 relative,
    # and subnormals are spaced 2^-9 * s apart
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(s.T, 128, axis=1) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)


def test_shape_errors():
    with pytest.raises(ValueError):
        quant_act_1x128(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        quant_w_128x128(np.zeros((100, 128), np.float32))
    with pytest.raises(ValueError):
        quant_act_128x1_T(np.zeros((100, 4), np.float32))
