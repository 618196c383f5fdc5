"""Shared helpers for the GPU parity tests: conversions between torch tensors
and the numpy arrays the oracle takes, and adversarial inputs."""

import numpy as np
import torch


def to_oracle(x):
    """CPU numpy view for the oracle: float32 values, or BF16 bit patterns."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(x.dtype)


def u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def f32_bits(a):
    return np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_codes_equal(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatching codes, first at {i}: "
                             f"got 0x{int(got[i]):02x}, want 0x{int(want[i]):02x}")


def assert_scales_equal(got, want, what):
    g, w = f32_bits(got), f32_bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatching scales, first at {i}: "
                             f"got {np.asarray(got)[i]!r}, want {np.asarray(want)[i]!r}")


# the 127 non-negative finite E4M3 magnitudes in code order, from torch's decoder
_E4M3 = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def adversarial_rows(n_rows, K, seed=0):
    """float32 [n_rows][K]: each 128-wide group has one of several hard patterns.

    Patterns: all +0; all -0; zeros with one subnormal; subnormal amax; exact
    E4M3 midpoints (ties) at a power-of-two scale; values 1 ulp around those
    midpoints; amax exactly 448 * 2^j; huge values; tiny next to huge (codes
    that round to +-0); random normals with an x100 outlier.
    """
    rng = np.random.default_rng(seed)
    x = np.zeros((n_rows, K), np.float32)
    mids = (_E4M3[:-1] + _E4M3[1:]) / 2
    for r in range(n_rows):
        for g in range(K // 128):
            sl = slice(g * 128, g * 128 + 128)
            kind = (r * (K // 128) + g) % 10
            if kind == 0:
                v = np.zeros(128)
            elif kind == 1:
                v = -np.zeros(128)
            elif kind == 2:
                v = np.zeros(128); v[rng.integers(128)] = -1e-42
            elif kind == 3:
                v = rng.standard_normal(128) * 1e-39
            elif kind == 4:
                j = int(rng.integers(-10, 10))
                v = rng.choice(mids, 128) * rng.choice([-1, 1], 128) * 2.0 ** j
                v[0] = 448 * 2.0 ** j
            elif kind == 5:
                j = int(rng.integers(-5, 5))
                m = (rng.choice(mids, 128) * 2.0 ** j).astype(np.float32)
                v = np.where(rng.random(128) < 0.5, np.nextafter(m, np.float32(np.inf)),
                             np.nextafter(m, np.float32(-np.inf)))
                v[0] = 448 * 2.0 ** j
            elif kind == 6:
                j = int(rng.integers(-20, 20))
                v = rng.choice(_E4M3, 128) * rng.choice([-1, 1], 128) * 2.0 ** j
                v[5] = -448 * 2.0 ** j
            elif kind == 7:
                v = rng.standard_normal(128) * 1e30
            elif kind == 8:
                v = rng.standard_normal(128) * 1e-6
                v[3] = 1e4
            else:
                v = rng.standard_normal(128)
                v[int(rng.integers(128))] *= 100
            x[r, sl] = np.asarray(v, np.float64).astype(np.float32)
    return x


def oracle_threads():
    """Worker threads for splitting large oracle computations (numpy releases the GIL)."""
    import os
    return max(1, min(16, os.cpu_count() or 1))


def parallel_rows(fn, x, pieces=None):
    """Apply a row-local oracle function to row blocks of x on a thread pool and
    return the list of per-block results, in order."""
    from concurrent.futures import ThreadPoolExecutor
    n = x.shape[0]
    pieces = pieces or 4 * oracle_threads()
    bounds = np.linspace(0, n, pieces + 1).astype(np.int64)
    blocks = [x[bounds[i]:bounds[i + 1]] for i in range(pieces) if bounds[i + 1] > bounds[i]]
    with ThreadPoolExecutor(oracle_threads()) as ex:
        return list(ex.map(fn, blocks))


def oracle_quant_act_1x128_big(x):
    """oracle.quant_act_1x128 of a large [M][K] array, computed in row blocks in
    parallel (the groups of distinct rows are independent)."""
    import oracle
    parts = parallel_rows(oracle.quant_act_1x128, x)
    return np.concatenate([p[0] for p in parts], axis=0), np.concatenate([p[1] for p in parts], axis=1)


def oracle_quant_w_128x128_big(w):
    """oracle.quant_w_128x128 of a large [N][K] array, by 128-row block bands in parallel."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    N = w.shape[0]
    bands = [w[i:i + 1024] for i in range(0, N, 1024)]
    with ThreadPoolExecutor(oracle_threads()) as ex:
        parts = list(ex.map(oracle.quant_w_128x128, bands))
    return np.concatenate([p[0] for p in parts], axis=0), np.concatenate([p[1] for p in parts], axis=0)


def e4m3_encode_parallel(y):
    """oracle.e4m3_encode of a large 1-D float32 array on a thread pool."""
    from oracle.e4m3 import e4m3_encode
    parts = parallel_rows(e4m3_encode, np.asarray(y, np.float32).ravel())
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


E4M3_MAX_BITS = int(np.float32(448.0).view(np.uint32))     # 0x43E00000


def e4m3_code_thresholds():
    """T[c-1] = the smallest non-negative float32 bit pattern whose oracle E4M3
    code is >= c, for c = 1..126, found by bisection with oracle.e4m3_encode.

    The encoder rounds magnitudes to nearest (ties to even) and saturates, so it
    is monotonic in |x|, and non-negative float32 patterns are ordered as their
    values: the code of magnitude pattern p <= 448 is searchsorted(T, p, 'right').
    """
    from oracle.e4m3 import e4m3_encode
    lo = np.zeros(126, np.int64)                        # encodes below c
    hi = np.full(126, E4M3_MAX_BITS, np.int64)          # encodes to >= c
    target = np.arange(1, 127)
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        c = e4m3_encode(mid.astype(np.uint32).view(np.float32)).astype(np.int64)
        up = c >= target
        hi = np.where(up, mid, hi)
        lo = np.where(up, lo, mid)
    return hi
