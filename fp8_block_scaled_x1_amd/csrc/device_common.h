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

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// FP32 -> BF16 bits, round to nearest even (finite inputs; overflow gives inf).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Group scale from the group's amax: amax / 448 (IEEE division), 1.0 if zero.
__device__ __forceinline__ float group_scale(float amax) {
  const float s = amax / kE4M3Max;
  return s == 0.0f ? 1.0f : s;
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

}  // namespace fp8bs
