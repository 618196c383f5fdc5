"""Pins for the oracle's E4M3 codec.

Independent of the oracle's own arithmetic: closed-form values of the OCP
E4M3FN format (4-bit exponent, 3-bit mantissa as the pages state, bias 7,
max 448), torch's float8_e4m3fn decode and cast (a separate implementation),
and a brute-force nearest-value search with ties to the even code.
"""

import numpy as np
import pytest
import torch

from oracle import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_finite_values


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_closed_form_points():
    d = e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x40, 0x7E, 0xFE, 0x7F, 0xFF, 0x39],
                             np.uint8))
    assert d[0] == 0.0 and not np.signbit(d[0])
    assert d[1] == 0.0 and np.signbit(d[1])
    assert d[2] == 2.0 ** -9                 # smallest subnormal
    assert d[3] == 7 * 2.0 ** -9             # largest subnormal
    assert d[4] == 2.0 ** -6                 # smallest normal
    assert d[5] == 1.0
    assert d[6] == 2.0
    assert d[7] == 448.0 == E4M3_MAX == 1.75 * 2 ** 8
    assert d[8] == -448.0
    assert np.isnan(d[9]) and np.isnan(d[10])
    assert d[11] == 1.125


def test_decode_matches_torch_all_codes():
    ours = e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    assert fin.sum() == 254


def test_finite_table_strictly_increasing():
    t = e4m3_finite_values()
    assert t.shape == (127,)
    assert np.all(np.diff(t) > 0)
    # every finite value is an integer multiple of 2^-9 (used by the GEMM exactness argument)
    assert np.all(np.floor(t * 512) == t * 512)


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def _brute_force_encode(y):
    """Nearest finite E4M3 magnitude, ties to the even code; sign kept.

    The two finite grid values that bracket |y| are found by comparison
    against torch's decode table; the nearer one wins, the even code on a tie.
    Above 448 there is no upper neighbour, so the nearest finite value is 448.
    Both differences are exact in float64 except for |y| far below 2^-9,
    where no tie is possible.
    """
    y = np.asarray(y, np.float32)
    a = np.abs(y.astype(np.float64))
    table = _torch_decode_all()[:127]
    lo = np.array([np.nonzero(table <= v)[0].max() for v in a])
    hi = np.minimum(lo + 1, 126)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick = np.where(hi == lo, lo,
                    np.where(d_lo < d_hi, lo,
                             np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi))))
    pick = np.where(a >= table[126], 126, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def test_encode_exhaustive_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    y = (bits << 16).view(np.float32)
    y = y[np.isfinite(y)]
    for part in np.array_split(y, 8):
        assert np.array_equal(e4m3_encode(part), _brute_force_encode(part))


def test_encode_around_every_midpoint():
    t = e4m3_finite_values()
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)       # exactly representable in float32
    assert np.array_equal(mids.astype(np.float64), (t[:-1] + t[1:]) / 2)
    ys = []
    for k in range(-4, 5):
        m = mids.copy()
        for _ in range(abs(k)):
            m = np.nextafter(m, np.float32(np.inf if k > 0 else -np.inf))
        ys.append(m)
    above = np.nextafter(np.float32(448.0), np.float32(np.inf))
    ys.append(np.array([448.0, above, 464.0, 479.9, 1e6, 3.4e38, 2.0 ** -10, 2.0 ** -11,
                        1e-30, 1e-45, 0.0], np.float32))
    y = np.concatenate(ys)
    y = np.concatenate([y, -y])
    assert np.array_equal(e4m3_encode(y), _brute_force_encode(y))


def test_midpoint_ties_go_to_even_code():
    t = e4m3_finite_values()
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    got = e4m3_encode(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect.astype(np.uint8))


def test_encode_matches_torch_cast_random():
    rng = np.random.default_rng(1234)
    y = np.concatenate([
        rng.standard_normal(300_000).astype(np.float32) * 100,
        (rng.standard_normal(300_000) * 2.0 ** rng.integers(-14, 9, 300_000)).astype(np.float32),
        rng.uniform(-448, 448, 300_000).astype(np.float32),
    ])
    y = y[np.abs(y) <= 448]
    ours = e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_saturation_and_signed_zero():
    y = np.array([449.0, 1e9, -500.0, -0.0, 0.0, -1e-20, 1e-20, -2.0 ** -10, 2.0 ** -10,
                  -(2.0 ** -10 + 2.0 ** -30)], np.float32)
    assert list(e4m3_encode(y)) == [0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80, 0x00, 0x80, 0x00, 0x81]


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan], np.float32))


def test_code_threshold_table_reproduces_the_encoder():
    # the table the device converter sweep derives its expected codes from
    from helpers import E4M3_MAX_BITS, e4m3_code_thresholds, e4m3_encode_parallel
    T = e4m3_code_thresholds()
    assert np.all(np.diff(T) > 0)
    assert T[0] == int(np.float32(2.0 ** -10).view(np.uint32)) + 1   # above half the smallest subnormal
    near = np.unique(np.clip((T[:, None] + np.arange(-64, 65)[None, :]).ravel(), 0, E4M3_MAX_BITS))
    stride = np.arange(0, E4M3_MAX_BITS + 1, 4099, dtype=np.int64)
    p = np.concatenate([near, stride]).astype(np.uint32)
    want = e4m3_encode_parallel(p.view(np.float32)).astype(np.int64)
    got = np.searchsorted(T, p.astype(np.int64), side="right")
    assert np.array_equal(got, want)
