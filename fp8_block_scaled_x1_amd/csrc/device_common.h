// Device helpers shared by the gfx950 kernels of libfp8bs.
//
// Numerics follow the DeepSeek-V3 report section 3.3.2 as paraphrased on the
// innerforce.co.kr page (E4M3 on all tensors, per-group scales along K), with
// these readings: OCP E4M3FN codes (bias 7, max 448, no infinities), scale =
// amax/448 in FP32 (1.0 for a zero group), codes = E4M3(x / scale) using an
// IEEE-rounded FP32 division, round to nearest even, saturation at 448, the
// sign bit always kept (so -0 encodes as 0x80).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr int kGroup = 128;          // quantization group / promotion interval along K
constexpr float kE4M3Max = 448.0f;

// Float -> E4M3 code, saturating, round to nearest even, by integer operations
// on the FP32 bit pattern.
//   * |y| >= 2^-6 (E4M3 normal binades): drop the low 20 mantissa bits with
//     round-half-even, then rebias the exponent from 127 to 7. A carry out of
//     the mantissa moves into the exponent field, which is the correct next
//     binade. Everything above 448 clamps to 0x7E.
//   * |y| <  2^-6 (E4M3 subnormals, spacing 2^-9): the code is the integer
//     round-half-even(|y| * 2^9), in 0..8; 8 is the smallest normal, 0x08.
//     The multiply by 2^9 is exact.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t normal = (rounded >> 20) - (120u << 3);
  normal = normal < 0x7Eu ? normal : 0x7Eu;
  const uint32_t a_sub = a < 0x3C800000u ? a : 0x3C800000u;   // keeps the product <= 8
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a_sub) * 512.0f);
  const uint32_t mag = a < 0x3C800000u ? sub : normal;
  return mag | sign;
}

// Four values -> four E4M3 codes packed little-endian in one dword, with the
// hardware converter (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950, round to nearest
// even). An exhaustive run over every finite FP32 bit pattern on MI355X gave
// results identical to e4m3_code() above for all |y| < 464, the converter
// returning NaN above that; the clamp to +-448 first (which keeps -0 as -0)
// turns that range into the saturated code 0x7E / 0xFE that e4m3_code gives.
__device__ __forceinline__ uint32_t e4m3_pack4(float y0, float y1, float y2, float y3) {
  y0 = __builtin_amdgcn_fmed3f(y0, -kE4M3Max, kE4M3Max);
  y1 = __builtin_amdgcn_fmed3f(y1, -kE4M3Max, kE4M3Max);
  y2 = __builtin_amdgcn_fmed3f(y2, -kE4M3Max, kE4M3Max);
  y3 = __builtin_amdgcn_fmed3f(y3, -kE4M3Max, kE4M3Max);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
}

// Codes of x[i] / s for four values, identical to e4m3_pack4(x[i] / s) with
// IEEE division, at a fraction of the cost. r must be RN(1/s) and s_fast must
// say whether s lies in [2^-126, 2^125] (s and r normal).
//
// Why it is exact: q0 = RN(x * r) carries two roundings of at most 2^-24
// relative each, so |q0 - x/s| < 2.0001 ulp of x/s, which is at most 5 steps
// of the FP32 grid around q0 even where the spacing halves at a power of two;
// |RN(x/s)| is therefore one of the FP32 magnitudes within 6 steps of |q0|
// (down to zero), and RN(x/s) has the sign of q0 (the sign of x, s > 0). The
// E4M3 encoding of a magnitude is monotonic and the code of a signed value is
// its sign bit over the code of its magnitude, so if the magnitudes 6 steps
// below (saturating at zero) and 6 steps above |q0| encode to the same code,
// every candidate does and the code of q0 is the code of RN(x/s). Otherwise
// (q0 near an E4M3 rounding boundary, rare) the lane recomputes with the IEEE
// division. With s normal, |x/s| <= 448*(1 + 2^-23), so |q0| + 6 steps stays
// far below 464, where the converter stops saturating. The check is straight
// line code: two neighbour codes per value from one conversion, compared four
// bytes at a time.
__device__ __forceinline__ uint32_t e4m3_div_pack4(float x0, float x1, float x2, float x3, float s, float r,
                                                   bool s_fast) {
  const float q0 = x0 * r, q1 = x1 * r, q2 = x2 * r, q3 = x3 * r;
  const float q[4] = {q0, q1, q2, q3};
  float lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = __float_as_uint(q[i]) & 0x7FFFFFFFu;
    lo[i] = __uint_as_float(__builtin_elementwise_sub_sat(m, 6u));
    hi[i] = __uint_as_float(m + 6u);
  }
  // bytes: code(lo0) code(hi0) code(lo1) code(hi1), and the same for 2, 3
  const uint32_t n01 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      lo[1], hi[1], __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], hi[0], 0, false), true);
  const uint32_t n23 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
      lo[3], hi[3], __builtin_amdgcn_cvt_pk_fp8_f32(lo[2], hi[2], 0, false), true);
  const uint32_t bad = ((n01 ^ (n01 >> 8)) | (n23 ^ (n23 >> 8))) & 0x00FF00FFu;
  if (__builtin_expect(s_fast & (bad == 0u), 1)) {
    const int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, c01, true);
  }
  return e4m3_pack4(x0 / s, x1 / s, x2 / s, x3 / s);
}


__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// FP32 -> BF16 bits, round to nearest even (finite inputs; overflow gives inf).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Group scale from the group's amax: amax / 448 rounded to nearest (the IEEE
// quotient), 1.0 if zero. Where the quotient is a normal number it is formed
// as q0 = RN(amax * RN(1/448)) plus one FMA correction; a sweep over every
// positive finite FP32 amax on MI355X gave the IEEE quotient bit for bit
// wherever that quotient is normal. Below that the IEEE division runs.
__device__ __forceinline__ float group_scale(float amax) {
  constexpr float c = 1.0f / kE4M3Max;
  float s;
  if (__builtin_expect(amax >= 0x1.cp-118f, 1)) {   // 448 * 2^-126
    const float q0 = amax * c;
    s = fmaf(fmaf(-q0, kE4M3Max, amax), c, q0);
  } else {
    s = amax / kE4M3Max;
  }
  return s == 0.0f ? 1.0f : s;
}

// RN(1/s) for s in [2^-126, 2^125]: the hardware reciprocal estimate and one
// Newton step; a sweep over every FP32 s in that range on MI355X gave the IEEE
// quotient 1/s bit for bit. Outside that range the result is not used.
__device__ __forceinline__ float recip_rn(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  return fmaf(fmaf(-s, y0, 1.0f), y0, y0);
}

// Per-group division state: the scale, RN(1/scale) and whether the fast
// quotient paths below apply to it.
struct GroupDiv {
  float s, r;
  bool fast;
};
// BF16 inputs use the one-correction quotient, which is exact for scales in
// [2^-64, 2^125]; F32 inputs use the checked quotient, exact for [2^-126, 2^125].
template <bool BF16>
__device__ __forceinline__ GroupDiv group_div_of_scale(float s) {
  GroupDiv g;
  g.s = s;
  g.r = recip_rn(s);
  g.fast = s >= (BF16 ? 0x1p-64f : 0x1p-126f) && s <= 0x1p125f;
  return g;
}
template <bool BF16>
__device__ __forceinline__ GroupDiv group_div(float amax) {
  return group_div_of_scale<BF16>(group_scale(amax));
}

// Codes of x[i] / s for four values taken from BF16 inputs, identical to
// e4m3_pack4(x[i] / s) with IEEE division when s lies in [2^-64, 2^125] and
// r = RN(1/s). The quotient is q0 = RN(x * r) with one FMA correction,
// fma(x - q0 * s, r, q0), where the residual x - q0 * s is one FMA too, given
// the sign of x (the correction turns -0 into +0). The result is
// not always the correctly rounded FP32 quotient, but a sweep over every pair
// of a positive finite BF16 amax and a BF16 x with |x| <= amax on MI355X, with
// s = RN(amax / 448) in that range, gave the E4M3 code of the IEEE quotient in
// every case. Outside the range the IEEE division runs.
__device__ __forceinline__ uint32_t e4m3_div_pack4_bf16(float x0, float x1, float x2, float x3, const GroupDiv& g) {
  if (__builtin_expect(g.fast, 1)) {
    const float x[4] = {x0, x1, x2, x3};
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q0 = x[i] * g.r;
      q[i] = __builtin_copysignf(fmaf(fmaf(-q0, g.s, x[i]), g.r, q0), x[i]);
    }
    const int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c01, true);
  }
  return e4m3_pack4(x0 / g.s, x1 / g.s, x2 / g.s, x3 / g.s);
}

// Codes of x[r] / g[r].s for four values with four different scales (BF16
// numbers as inputs), packed little-endian: each quotient as in
// e4m3_div_pack4_bf16 (one FMA correction where that scale allows it, else the
// IEEE division), then the clamp and the converter of e4m3_pack4 (the clamp
// leaves every correction-path quotient's code unchanged: those stay below
// 464, where the converter already saturates to 448).
__device__ __forceinline__ uint32_t e4m3_div_cols4_bf16(const float x[4], const GroupDiv g[4]) {
  float q[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (g[r].fast) {
      const float q0 = x[r] * g[r].r;
      q[r] = __builtin_copysignf(fmaf(fmaf(-q0, g[r].s, x[r]), g[r].r, q0), x[r]);
    } else {
      q[r] = x[r] / g[r].s;
    }
  }
  return e4m3_pack4(q[0], q[1], q[2], q[3]);
}

// The quotient codes for the input type: checked for F32, one-correction for BF16.
template <bool BF16>
__device__ __forceinline__ uint32_t e4m3_div_pack4_t(float x0, float x1, float x2, float x3, const GroupDiv& g) {
  if constexpr (BF16)
    return e4m3_div_pack4_bf16(x0, x1, x2, x3, g);
  else
    return e4m3_div_pack4(x0, x1, x2, x3, g.s, g.r, g.fast);
}

// ---------------------------------------------------------------------------
// Power-of-two scales (the E8M0-compatible variant): the scale is the smallest
// power of two not below RN(amax / 448), and not below 2^-126 (a normal FP32,
// so its exponent field is its E8M0 encoding); a zero group keeps 1.0. The
// codes are then E4M3(x * 2^-e): a product with a power of two is exact
// wherever it is a normal number, and below that the code is +-0 either way.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pow2_scale(float amax) {
  const uint32_t b = __float_as_uint(group_scale(amax));
  return __uint_as_float((b + 0x7FFFFFu) & 0xFF800000u);
}
// 1/s for a power-of-two s = 2^(E-127), E in [1, 253]: exponent field 254 - E
__device__ __forceinline__ float pow2_recip(float s) { return __uint_as_float((254u << 23) - __float_as_uint(s)); }

// The quantizers' scale rule: POW2 selects the power-of-two variant.
template <bool POW2>
__device__ __forceinline__ float scale_rule(float amax) {
  if constexpr (POW2)
    return pow2_scale(amax);
  else
    return group_scale(amax);
}
template <bool BF16, bool POW2>
__device__ __forceinline__ GroupDiv div_of_scale_rule(float s) {
  if constexpr (POW2) {
    GroupDiv g;
    g.s = s;
    g.r = pow2_recip(s);
    g.fast = true;
    return g;
  } else {
    return group_div_of_scale<BF16>(s);
  }
}
template <bool BF16, bool POW2>
__device__ __forceinline__ GroupDiv div_rule(float amax) {
  return div_of_scale_rule<BF16, POW2>(scale_rule<POW2>(amax));
}
template <bool BF16, bool POW2>
__device__ __forceinline__ uint32_t pack4_rule(float x0, float x1, float x2, float x3, const GroupDiv& g) {
  if constexpr (POW2)
    return e4m3_pack4(x0 * g.r, x1 * g.r, x2 * g.r, x3 * g.r);
  else
    return e4m3_div_pack4_t<BF16>(x0, x1, x2, x3, g);
}

// Max over the 16 lanes of a DPP row (lanes 16r..16r+15), result in every lane
// of the row. row_ror rotates within the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));  // ror 8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));  // ror 4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, false)));  // ror 2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, false)));  // ror 1
  return v;
}

// Max over a whole wave64, result in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  // combine the four rows: lanes l and l^16, then l and l^32
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Pack four codes (low byte of each) into one little-endian dword.
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// ---------------------------------------------------------------------------
// Per-expert work lists. Expert e owns rows [a_e, b_e) with
// a_e = clamp(off[e], 0, M_total) and b_e = clamp(off[e+1], a_e, M_total);
// it has units(e) = ceil((b_e - a_e) / unit_rows) * mult work units (none if
// it has min_rows rows or fewer), numbered expert-major. Lane l of the calling wave examines expert e0 + l of each
// batch of 64 (the offsets of a batch are read at once) and a prefix sum over
// the lanes finds the answer; every result is wave-uniform.
// ---------------------------------------------------------------------------
struct ExpertSlot {
  int e;        // expert of the unit, -1 if the unit is past the last
  int r0, r1;   // its row range
  int base;     // units of the experts before it
};

__device__ __forceinline__ ExpertSlot locate_expert(const int32_t* __restrict__ off, int E, int M_total,
                                                    int unit, int unit_rows, int mult, int min_rows = 0) {
  const int lane = threadIdx.x & 63;
  ExpertSlot r{-1, 0, 0, 0};
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int a = 0, b = 0, ue = 0;
    if (e < E) {
      a = min(max(off[e], 0), M_total);
      b = min(max(off[e + 1], a), M_total);
      ue = b - a > min_rows ? ((b - a + unit_rows - 1) / unit_rows) * mult : 0;
    }
    int incl = ue;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const uint64_t hit = __ballot(e < E && unit < base + incl);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      r.e = e0 + l;
      r.r0 = __shfl(a, l, 64);
      r.r1 = __shfl(b, l, 64);
      base += __shfl(incl, l, 64) - __shfl(ue, l, 64);
      break;
    }
    base += __shfl(incl, 63, 64);
  }
  r.e = __builtin_amdgcn_readfirstlane(r.e);
  r.r0 = __builtin_amdgcn_readfirstlane(r.r0);
  r.r1 = __builtin_amdgcn_readfirstlane(r.r1);
  r.base = __builtin_amdgcn_readfirstlane(base);
  return r;
}

// Units (as above) of all experts together; wave-uniform.
__device__ __forceinline__ int total_units(const int32_t* __restrict__ off, int E, int M_total, int unit_rows,
                                           int mult, int min_rows = 0) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    if (e < E) {
      const int a = min(max(off[e], 0), M_total);
      const int b = min(max(off[e + 1], a), M_total);
      sum += b - a > min_rows ? ((b - a + unit_rows - 1) / unit_rows) * mult : 0;
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d, 64);
  return __builtin_amdgcn_readfirstlane(sum);
}

// Units (as above, mult = 1) of the experts before expert e, with e's own
// row range; wave-uniform.
__device__ __forceinline__ ExpertSlot units_before(const int32_t* __restrict__ off, int M_total, int e,
                                                   int unit_rows) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int e0 = 0; e0 < e; e0 += 64) {
    const int x = e0 + lane;
    if (x < e) {
      const int a = min(max(off[x], 0), M_total);
      const int b = min(max(off[x + 1], a), M_total);
      sum += (b - a + unit_rows - 1) / unit_rows;
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d, 64);
  ExpertSlot r;
  r.e = e;
  r.r0 = min(max(off[e], 0), M_total);
  r.r1 = min(max(off[e + 1], r.r0), M_total);
  r.r0 = __builtin_amdgcn_readfirstlane(r.r0);
  r.r1 = __builtin_amdgcn_readfirstlane(r.r1);
  r.base = __builtin_amdgcn_readfirstlane(sum);
  return r;
}

}  // namespace fp8bs
