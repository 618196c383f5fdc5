"""Exhaustive check of the BF16 quantizer arithmetic on the GPU.

For BF16 inputs the quantizers form x / s with one FMA correction of
RN(x * RN(1/s)) instead of an IEEE division (see device_common.h). That is
exact for the E4M3 code but not for every FP32 quotient, so it is checked here
over its whole domain: every pair of a positive finite BF16 amax and a BF16 x
with |x| <= amax, about 1.07e9 pairs, each placed in a 128-element group whose
first element is amax. The reference is plain PyTorch on the GPU, independent
of the HIP kernels: amax / 448 and x / s in float64 rounded once to FP32 (a
double-precision quotient rounded to single precision is the correctly rounded
single-precision quotient, since 53 >= 2*24 + 2), then the float8_e4m3fn cast
after clamping to +-448 (saturation, as in the method's reading). Codes and
scales must match bit for bit.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_x1_amd as fb

pytestmark = pytest.mark.gpu

_AMAX_MAX = 0x7F7F          # largest finite BF16 bit pattern
_GROUPS_PER_CALL = 1_000_000  # rows of one fp8_quant_act_1x128 call (K = 128)


def _chunks():
    """Ranges [a0, a1) of amax bit patterns, about _GROUPS_PER_CALL groups each."""
    a = np.arange(1, _AMAX_MAX + 1, dtype=np.int64)
    groups = (2 * (a + 1) + 126) // 127
    cum = np.cumsum(groups)
    out, start, base = [], 1, 0
    while start <= _AMAX_MAX:
        idx = int(np.searchsorted(cum, base + _GROUPS_PER_CALL, side="right"))
        end = max(idx + 1, start + 1)          # amax patterns start .. end-1
        end = min(end, _AMAX_MAX + 1)
        out.append((start, end))
        base = int(cum[end - 2]) if end - 2 >= 0 else 0
        start = end
    return out


def _groups(a0, a1, dev):
    """BF16 bit patterns [G][128]: amax, then the x with |x| <= amax, padded with amax."""
    a = torch.arange(a0, a1, device=dev, dtype=torch.int64)
    n = 2 * (a + 1)                       # bits 0..a and 0x8000..0x8000+a
    g = (n + 126) // 127
    ga = torch.repeat_interleave(a, g)
    first = torch.cumsum(g, 0) - g
    j = torch.arange(int(g.sum()), device=dev) - torch.repeat_interleave(first, g)
    k = j[:, None] * 127 + torch.arange(127, device=dev)[None, :]
    aa = ga[:, None]
    bits = torch.where(k <= aa, k, 0x8000 + (k - aa - 1))
    bits = torch.where(k < 2 * (aa + 1), bits, aa)
    grp = torch.cat([aa, bits], dim=1).to(torch.int32)
    return grp.to(torch.int16).view(torch.bfloat16)


def test_bf16_quotient_codes_exhaustive(dev):
    total = 0
    for a0, a1 in _chunks():
        x = _groups(a0, a1, dev)
        q, s = fb.fp8_quant_act_1x128(x)
        xf = x.float()
        amax = xf.abs().amax(dim=1)
        s_ref = (amax.double() / 448.0).float()
        s_ref = torch.where(s_ref == 0, torch.ones_like(s_ref), s_ref)
        q_ref = (xf.double() / s_ref.double()[:, None]).float().clamp(-448.0, 448.0)
        codes_ref = q_ref.to(torch.float8_e4m3fn).view(torch.uint8)
        bad_s = (s.view(-1).view(torch.int32) != s_ref.view(torch.int32)).sum().item()
        bad_q = (q != codes_ref).sum().item()
        assert bad_s == 0, f"amax patterns {a0:#x}..{a1 - 1:#x}: {bad_s} scales differ"
        if bad_q:
            r, c = torch.nonzero(q != codes_ref)[0].tolist()
            raise AssertionError(
                f"amax patterns {a0:#x}..{a1 - 1:#x}: {bad_q} codes differ, first at amax "
                f"{x[r, 0].view(torch.int16).item() & 0xFFFF:#06x}, x {x[r, c].view(torch.int16).item() & 0xFFFF:#06x}: "
                f"{q[r, c].item():#04x} vs {codes_ref[r, c].item():#04x}")
        total += x.shape[0]
    # every amax pattern contributes ceil(2 (a + 1) / 127) groups
    a = np.arange(1, _AMAX_MAX + 1, dtype=np.int64)
    assert total == int(((2 * (a + 1) + 126) // 127).sum())
