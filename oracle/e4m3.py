"""E4M3 codec (test infrastructure; see the package docstring).

The pages fix only the bit split: E4M3 has a 4-bit exponent and a 3-bit
mantissa and is used on all tensors (DeepSeek-V3 report section 3.3.2, as
paraphrased on the innerforce.co.kr page). The reading taken here is the OCP
"E4M3FN" variant: exponent bias 7, subnormals at exponent field 0, no
infinities, the two all-ones patterns 0x7F / 0xFF are NaN, largest finite
magnitude 1.75 * 2**8 = 448. Codes are plain ``uint8`` bytes ``S EEEE MMM``.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each E4M3 code, as float64 (NaN for 0x7F and 0xFF).

    Closed form: exponent field E, mantissa field M, sign S:
      E >= 1: (-1)^S * 2^(E-7) * (1 + M/8)
      E == 0: (-1)^S * 2^(-6) * (M/8)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64) / 8.0, -6),
                   np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64)))
    val = np.where(s == 1, -mag, mag)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val


def e4m3_finite_values():
    """The 127 non-negative finite magnitudes, indexed by their code 0..126."""
    return e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(y):
    """Encode float32 values to E4M3 codes: saturating, round to nearest even.

    Reading of the pages (they give only the 4/3 bit split): magnitudes above
    448 saturate to 448 (code 0x7E); otherwise the magnitude is rounded to the
    nearest point of the E4M3 grid, ties to the even code. The grid spacing in
    binade e (e = floor(log2 |y|), clamped below at -6, the subnormal binade)
    is 2^(e-3). The sign bit is always kept, so -0 and small negatives that
    round to zero give 0x80. Input must be finite.
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3_encode: non-finite input")
    neg = np.signbit(y)
    a = np.abs(y.astype(np.float64))          # exact widening
    a = np.minimum(a, E4M3_MAX)               # saturate
    # floor(log2 a) computed exactly with frexp: a = f * 2^x, f in [0.5, 1).
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(x - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    n = np.rint(a / quantum)                  # rint = round half to even; a/quantum is exact
    v = n * quantum                           # n may be 16: carries into the next binade
    v = np.minimum(v, E4M3_MAX)               # cannot exceed 448 after the clamp, kept for clarity
    table = e4m3_finite_values()              # ascending in code order for codes 0..126
    mag_code = np.searchsorted(table, v)
    assert np.array_equal(table[mag_code], v), "rounded value off the E4M3 grid"
    code = mag_code.astype(np.uint8) | np.where(neg, np.uint8(0x80), np.uint8(0))
    return code.astype(np.uint8)
