"""Device sweeps of the FP32-input quantizer arithmetic, through the C ABI,
against the oracle.

The quantizers form the scale amax/448 and the quotients x/s from fused
multiply-adds and the hardware E4M3 converter rather than from IEEE division
(their exactness argument is in the device code). For BF16 inputs every
(amax, x) pair is swept by test_gpu_quant_exhaustive.py; these sweeps cover
the FP32 path:

* scale: one group per FP32 amax pattern, every one of the 2^23 mantissas of
  a mid binade [1, 2), of the two binades whose quotient crosses the
  normal/subnormal boundary ([2^-119, 2^-117): amax/448 = 2^-126 at amax =
  1.75 * 2^-118), of the top binade [2^127, 2^128) and of the subnormal
  amax values; each group also holds two signed values below its amax, whose
  codes are checked too. Scales must equal the oracle's fl32(amax/448) bit for
  bit, codes the oracle's E4M3(fl32(x/s)).
* converter: every FP32 pattern with |x| <= 448, both signs, in groups whose
  amax is 448, so s = 1 and the code is E4M3(x) itself: the hardware
  converter with its clamp must agree with the oracle's encoder on all
  2,277,507,074 values. The expected codes come from the oracle's encoder
  through its 126 rounding thresholds (the encoder is monotonic in |x|: the
  code of magnitude pattern p is the number of thresholds at or below p),
  found by bisection with the oracle itself (the table is checked against the
  oracle's encoder on the CPU in test_oracle_e4m3.py).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import E4M3_MAX_BITS, e4m3_code_thresholds, e4m3_encode_parallel, f32_bits

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu

G = 128


def _pattern_groups(dev, amax_bits, seed):
    """X[n][128] float32 on the device: group m holds +-amax_m at column p0 = m % 128
    (the sign alternating with m), +x1 at (p0 + 37) % 128 and -x2 at (p0 + 91) % 128,
    x1, x2 random patterns at most 2^26 - 1 below amax_m's (clamped at +0); the rest +0."""
    n = len(amax_bits)
    rng = np.random.default_rng(seed)
    a = amax_bits.astype(np.int64)
    x1 = np.maximum(a - rng.integers(0, 1 << 26, n), 0).astype(np.uint32)
    x2 = np.maximum(a - rng.integers(0, 1 << 26, n), 0).astype(np.uint32)
    m = np.arange(n)
    p0 = m % G
    cols = np.stack([p0, (p0 + 37) % G, (p0 + 91) % G], axis=1)
    sign = ((m >> 7) & 1).astype(np.uint32) << 31
    vals = np.stack([amax_bits.astype(np.uint32) | sign, x1, x2 | np.uint32(0x80000000)], axis=1)
    X = torch.zeros((n, G), dtype=torch.int32, device=dev)
    X.scatter_(1, torch.from_numpy(cols).to(dev), torch.from_numpy(vals.view(np.int32)).to(dev))
    return X.view(torch.float32), cols, vals.view(np.float32)


def _scale_sweep(dev, amax_bits, seed, what):
    X, cols, vals = _pattern_groups(dev, amax_bits, seed)
    q, s = fb.fp8_quant_act_1x128(X)
    del X
    # oracle: scale of each group, codes of its three non-zero values
    amax = np.abs(vals[:, 0])
    so = oracle.group_scale(amax)
    y = (vals / so[:, None]).astype(np.float32)           # IEEE float32 division, as the oracle's cast
    codes = e4m3_encode_parallel(y.ravel()).reshape(-1, 3)
    want = torch.zeros_like(q)
    want.scatter_(1, torch.from_numpy(cols).to(dev), torch.from_numpy(codes).to(dev))
    got_s = s[0].cpu().numpy()
    bad = np.nonzero(f32_bits(got_s) != f32_bits(so))[0]
    assert bad.size == 0, (f"{what}: {bad.size} scales differ, first amax {amax[bad[0]]!r}: "
                           f"got {got_s[bad[0]]!r}, want {so[bad[0]]!r}")
    neq = (q != want).any(dim=1).nonzero()
    if neq.numel():
        m = int(neq[0])
        raise AssertionError(f"{what}: {neq.numel()} groups with wrong codes, first group {m} "
                             f"values {vals[m].tolist()} scale {so[m]!r}: got "
                             f"{q[m, cols[m]].tolist()}, want {codes[m].tolist()}")


BINADES = {
    "mid [1,2)": 127,
    "quotient crosses 2^-126, low [2^-119,2^-118)": 8,
    "quotient crosses 2^-126, high [2^-118,2^-117)": 9,
    "top [2^127,2^128)": 254,
}


@pytest.mark.parametrize("what", sorted(BINADES))
def test_f32_scale_every_mantissa_of_binade(dev, what):
    e = BINADES[what]
    amax_bits = (np.uint32(e) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)
    _scale_sweep(dev, amax_bits, e, what)


def test_f32_scale_every_subnormal_amax(dev):
    amax_bits = np.arange(1 << 23, dtype=np.uint32)      # 0 (a zero group) and every subnormal
    _scale_sweep(dev, amax_bits, 1, "subnormal amax")


def test_f32_converter_every_pattern_up_to_448(dev):
    T = torch.from_numpy(e4m3_code_thresholds()).to(dev)
    total = 2 * (E4M3_MAX_BITS + 1)                           # every magnitude pattern with both signs
    per_group = G - 1                                    # column 0 holds the amax 448
    chunk_groups = 1 << 21                               # 267M values per launch
    done = 0
    while done < total:
        n = min(chunk_groups * per_group, total - done)
        groups = -(-n // per_group)
        idx = torch.arange(done, done + groups * per_group, dtype=torch.int64, device=dev)
        idx = torch.where(idx < total, idx, torch.zeros_like(idx))        # pad the last group with +0
        mag = idx >> 1
        bits = (mag | ((idx & 1) << 31)).to(torch.int64)
        X = torch.empty((groups, G), dtype=torch.int32, device=dev)
        X[:, 0] = int(np.float32(448.0).view(np.int32))
        X[:, 1:] = (bits - ((bits >> 31) << 32)).to(torch.int32).view(groups, per_group)
        q, s = fb.fp8_quant_act_1x128(X.view(torch.float32))
        assert torch.all(s == 1.0), "the groups' scale must be exactly 1"
        want_mag = torch.searchsorted(T, mag, right=True).to(torch.int32)
        want = (want_mag | (((idx & 1) << 7).to(torch.int32))).to(torch.uint8).view(groups, per_group)
        got = q[:, 1:]
        assert torch.all(q[:, 0] == 0x7E)
        bad = (got != want).nonzero()
        if bad.numel():
            g0, c0 = (int(v) for v in bad[0])
            b = int(bits.view(groups, per_group)[g0, c0]) & 0xFFFFFFFF
            raise AssertionError(f"{bad.shape[0]} codes differ from the oracle's encoder; first: "
                                 f"x = {np.uint32(b).view(np.float32)!r} (bits 0x{b:08x}): got "
                                 f"0x{int(got[g0, c0]):02x}, want 0x{int(want[g0, c0]):02x}")
        done += groups * per_group
        del X, q, s, want, got, idx, mag, bits
