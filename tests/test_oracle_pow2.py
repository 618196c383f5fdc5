"""Pins for the oracle's power-of-two scale variant.

Checked against: the rule restated with an integer search over exponents
(smallest 2^k with k >= -126 not below the FP32 quotient amax / 448; 1.0
where that quotient is zero, as in the FP32 rule), torch's
float8_e4m3fn cast of x / s (exact for a power-of-two s), and the property the
rule exists for: every group's largest magnitude lands in (224, 448] (the top
binade of E4M3) unless the 2^-126 floor applies.
"""

import math

import numpy as np
import torch

from oracle import e4m3_decode, pow2_scale, quant_act_1x128, quant_act_128x1_T, quant_w_128x128


def _amax_samples():
    rng = np.random.default_rng(0)
    bits = rng.integers(1, 0x7F800000, 20000, dtype=np.int64).astype(np.uint32)
    special = np.array([0.0, 448.0, 448.0 * 2.0 ** -20, 448.0 * 2.0 ** 30, 1e-45, 2.0 ** -126 * 448,
                        2.0 ** -126 * 447, 3.4e38, 1.0, 0.5, 224.0, 224.0000153], np.float32)
    return np.concatenate([bits.view(np.float32), special])


def test_pow2_scale_is_the_smallest_power_of_two_not_below_the_quotient():
    amax = _amax_samples()
    s = pow2_scale(amax)
    for a, got in zip(amax.tolist(), s.tolist()):
        r = float(np.float32(a) / np.float32(448.0))
        if r == 0.0:                 # zero group, or a quotient that underflows: 1.0 as in the FP32 rule
            assert got == 1.0
            continue
        k = -126
        while 2.0 ** k < r:
            k += 1
        assert got == 2.0 ** k, (a, got, k)


def test_pow2_codes_are_the_torch_cast_and_fill_the_top_binade():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    q, s = quant_act_1x128(x, pow2=True)
    g = torch.from_numpy(x).reshape(64, 4, 128)
    st = torch.from_numpy(np.ascontiguousarray(s.T))                   # [64][4]
    want = (g / st[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 512)
    assert np.array_equal(q, want.numpy())
    top = np.abs(e4m3_decode(q)).reshape(64, 4, 128).max(axis=2)
    nz = np.abs(x).reshape(64, 4, 128).max(axis=2) > 0
    assert np.all(top[nz] > 224.0 * (1 - 2.0 ** -20)) and np.all(top[nz] <= 448.0)
    assert np.all(s[:, 3] == 1.0) and np.all(q[3] == 0)


def test_pow2_layouts_agree_with_the_fp32_scale_quantizers_where_scales_coincide():
    # groups whose FP32 quotient is already a power of two get identical
    # outputs from both rules; 128x1 and 128x128 geometries included
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, (256, 256)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    codes[::128, :] = 0x7E                       # one 448 per 128x128 block and per 128x1 column group
    codes[:, ::128] = 0x7E                       # and per 1x128 row group
    x = (e4m3_decode(codes) * 2.0 ** -5).astype(np.float32)
    for f in (quant_act_1x128, quant_act_128x1_T, quant_w_128x128):
        a, b = f(x), f(x, pow2=True)
        for u, v in zip(a, b):
            assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))
    assert math.isclose(float(quant_act_1x128(x, pow2=True)[1][0, 0]), 2.0 ** -5)
