// Fine-grained E4M3 quantizers for gfx950 (memory-bound; one pass over the
// input, amax reduction and cast fused).
//
// The method: DeepSeek-V3 report section 3.3.2, as paraphrased on the
// innerforce.co.kr page -- elements are quantized in small groups that share a
// scaling factor, with the groups laid along the GEMM's inner dimension, and
// E4M3 is used for every tensor. The pages wish for the FP8 conversion to be
// fused with the data movement itself (report section 3.5.2); on gfx950 the
// equivalent is a single streaming kernel that reads each element once from
// HBM, reduces amax in registers (DPP) and writes codes and scales.
//
// Group geometry (a reading; the pages only say "small groups"):
//   quant_act_1x128   one row x 128 consecutive K           s[K/128][M]
//   quant_w_128x128   128 x 128 block                        s[N/128][K/128]
//   quant_act_128x1_T 128 consecutive tokens of one channel, written
//                     transposed (the pages call a transposition fused into
//                     the GEMM cumbersome, report section 3.5.2)  sT[M/128][C]

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8bs {

// ---------------------------------------------------------------------------
// 16-byte load with a non-temporal hint (the `nt` bit of the load). The
// quantizers read every input byte exactly once; with the hint their BF16
// passes ran 5-15% faster from HBM on the MI355X (128x1 over a 4096x7168
// tensor 25.4 -> 21.7 us, 1x128 over 65536x7168 245 -> 227 us, 128x128 over
// 7168x7168 29.9 -> 28.5 us), where without it the 128x1 pass's address unit
// was stalled by the vector L1 seven times longer than the 1x128 pass's.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Loads of 8 consecutive high-precision elements as FP32 (exact widening);
// BF16 inputs through the streaming load above.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float v[8]) {
  if constexpr (BF16) {
    const uint4 d = load16_stream(reinterpret_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// codes of v[i] / s (IEEE FP32 division, then E4M3)
template <bool BF16, bool POW2>
__device__ __forceinline__ uint2 cast8(const float v[8], const GroupDiv& g) {
  return make_uint2(pack4_rule<BF16, POW2>(v[0], v[1], v[2], v[3], g),
                    pack4_rule<BF16, POW2>(v[4], v[5], v[6], v[7], g));
}

// ---------------------------------------------------------------------------
// 1x128 activation quantizer.
// Block of 4 waves: rows 8*rb .. 8*rb+7 (wave w: rows 8*rb + 2w, 8*rb + 2w + 1)
// with rb = blockIdx.y + gridDim.y * blockIdx.z, K chunks 4*bx .. 4*bx+3 (the
// fastest grid index, so consecutive workgroups read consecutive 1 KB pieces
// of the same rows). Lane l covers elements (l%16)*8 .. +7 of chunk
// 4*bx + l/16, so each load instruction reads 1 KB of one row and the 16 lanes
// of a DPP row form one group (amax is a 4-step row rotation). Both loads of a
// lane are issued before any compute (row and chunk indices are clamped,
// stores masked).
// ---------------------------------------------------------------------------
constexpr int kActRows = 2;   // rows per wave

template <bool BF16, bool POW2>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(
    const void* __restrict__ x, int64_t M, int K, uint8_t* __restrict__ q,
    float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nkb = K / kGroup;
  const int part = lane & 15;
  const int kb = blockIdx.x * 4 + (lane >> 4);
  const int kbc = min(kb, nkb - 1);
  const int64_t rb = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t row0 = (rb * 4 + wave) * kActRows;
  if (row0 - wave * kActRows >= M) return;   // whole block past the last row

  float v[kActRows][8];
#pragma unroll
  for (int u = 0; u < kActRows; ++u) {
    const int64_t row = min(row0 + u, M - 1);
    load8<BF16>(x, row * K + (int64_t)kbc * kGroup + part * 8, v[u]);
  }
#pragma unroll
  for (int u = 0; u < kActRows; ++u) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
    amax = row16_max(amax);
    const GroupDiv g = div_rule<BF16, POW2>(amax);
    const uint2 codes = cast8<BF16, POW2>(v[u], g);
    const int64_t row = row0 + u;
    if (row < M && kb < nkb) {
      *reinterpret_cast<uint2*>(q + row * K + (int64_t)kb * kGroup + part * 8) = codes;
      if (part == 0) s[(int64_t)kb * M + row] = g.s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight quantizer: one workgroup (256 threads) per block (nb, kb).
// Thread t covers rows i*16 + t/16 (i = 0..7), elements (t%16)*8 .. +7 of the
// block: 8 independent 16-byte loads in flight, 64 values in registers.
// With a transposed copy requested, the codes also go through an LDS tile and
// leave as 4x4-byte transposed pieces so that qT rows are written coalesced.
// ---------------------------------------------------------------------------
constexpr int kTileStride = kGroup + 4;   // LDS row pitch in bytes (padding against bank conflicts)

template <bool BF16, bool TRANS, bool POW2>
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(
    const void* __restrict__ w, int N, int K, uint8_t* __restrict__ q, float* __restrict__ s,
    uint8_t* __restrict__ qT, float* __restrict__ sT) {
  __shared__ float red[4];
  __shared__ __align__(16) uint8_t tile[TRANS ? kGroup * kTileStride : 4];
  const int t = threadIdx.x;
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int nkb = K / kGroup, nnb = N / kGroup;
  const int r0 = t >> 4, part = t & 15;

  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = (int64_t)nb * kGroup + i * 16 + r0;
    load8<BF16>(w, row * K + (int64_t)kb * kGroup + part * 8, v[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const GroupDiv g = div_rule<BF16, POW2>(amax);
  const float sc = g.s;

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = i * 16 + r0;
    const uint2 codes = cast8<BF16, POW2>(v[i], g);
    *reinterpret_cast<uint2*>(q + ((int64_t)nb * kGroup + rl) * K + (int64_t)kb * kGroup + part * 8) = codes;
    if constexpr (TRANS) {
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + rl * kTileStride + part * 8);
      d[0] = codes.x;
      d[1] = codes.y;
    }
  }
  if (t == 0) {
    s[nb * nkb + kb] = sc;
    if constexpr (TRANS) sT[kb * nnb + nb] = sc;
  }
  if constexpr (TRANS) {
    __syncthreads();
    // 32x32 pieces of 4x4 bytes; piece (pr, pc) covers tile rows 4pr..4pr+3,
    // columns 4pc..4pc+3 and lands in qT rows kb*128 + 4pc + j, columns
    // nb*128 + 4pr .. +3.
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int piece = t + 256 * j4;
      const int pr = piece & 31, pc = piece >> 5;
      uint32_t d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d[i] = *reinterpret_cast<const uint32_t*>(tile + (4 * pr + i) * kTileStride + 4 * pc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t out = ((d[0] >> (8 * j)) & 0xFFu) | (((d[1] >> (8 * j)) & 0xFFu) << 8) |
                             (((d[2] >> (8 * j)) & 0xFFu) << 16) | (((d[3] >> (8 * j)) & 0xFFu) << 24);
        *reinterpret_cast<uint32_t*>(qT + ((int64_t)kb * kGroup + 4 * pc + j) * N +
                                     (int64_t)nb * kGroup + 4 * pr) = out;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 transposed quantizer: one workgroup per (token chunk tb, 64 channels).
// Thread t: channel pair cp = t%32 (channels c0+2cp, c0+2cp+1), token slice
// tg = t/32 (tokens 16tg .. 16tg+15 of the chunk). Loads of consecutive lanes
// cover 128 contiguous bytes of an input row (BF16). Per-channel amax is
// combined across the 8 token slices through LDS; each thread then writes its
// 16 codes per channel as one 16-byte piece of a qT row.
// ---------------------------------------------------------------------------
template <bool BF16, bool PAIR, bool POW2>
__global__ __launch_bounds__(256) void quant_act_128x1_T_kernel(
    const void* __restrict__ x, int64_t M, int C, uint8_t* __restrict__ qT, float* __restrict__ sT) {
  __shared__ float red[8][64];
  __shared__ float scl[64];
  const int t = threadIdx.x;
  const int cp = t & 31, tg = t >> 5;
  const int tb = blockIdx.y;
  const int c0 = blockIdx.x * 64;
  const int ch = c0 + 2 * cp;
  const bool ok0 = ch < C, ok1 = ch + 1 < C;
  const int64_t tok0 = (int64_t)tb * kGroup + tg * 16;

  float v0[16], v1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t e = (tok0 + i) * C + ch;
    if constexpr (PAIR) {
      if (ok0) {   // C even: ch < C implies ch + 1 < C
        if constexpr (BF16) {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(x) + e);
          v0[i] = __uint_as_float(d << 16);
          v1[i] = __uint_as_float(d & 0xFFFF0000u);
        } else {
          const float2 d = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(x) + e);
          v0[i] = d.x;
          v1[i] = d.y;
        }
      } else {
        v0[i] = 0.0f;
        v1[i] = 0.0f;
      }
    } else {
      if constexpr (BF16) {
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
        v0[i] = ok0 ? bf16_bits_to_float(xb[e]) : 0.0f;
        v1[i] = ok1 ? bf16_bits_to_float(xb[e + 1]) : 0.0f;
      } else {
        const float* xf = reinterpret_cast<const float*>(x);
        v0[i] = ok0 ? xf[e] : 0.0f;
        v1[i] = ok1 ? xf[e + 1] : 0.0f;
      }
    }
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a0 = fmaxf(a0, fabsf(v0[i]));
    a1 = fmaxf(a1, fabsf(v1[i]));
  }
  red[tg][2 * cp] = a0;
  red[tg][2 * cp + 1] = a1;
  __syncthreads();
  if (t < 64) {
    float amax = red[0][t];
#pragma unroll
    for (int g = 1; g < 8; ++g) amax = fmaxf(amax, red[g][t]);
    const float sc = scale_rule<POW2>(amax);
    scl[t] = sc;
    if (c0 + t < C) sT[(int64_t)tb * C + c0 + t] = sc;
  }
  __syncthreads();
  const GroupDiv g0 = div_of_scale_rule<BF16, POW2>(scl[2 * cp]);
  const GroupDiv g1 = div_of_scale_rule<BF16, POW2>(scl[2 * cp + 1]);
  uint32_t w0[4], w1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w0[j] = pack4_rule<BF16, POW2>(v0[4 * j], v0[4 * j + 1], v0[4 * j + 2], v0[4 * j + 3], g0);
    w1[j] = pack4_rule<BF16, POW2>(v1[4 * j], v1[4 * j + 1], v1[4 * j + 2], v1[4 * j + 3], g1);
  }
  if (ok0) *reinterpret_cast<uint4*>(qT + (int64_t)ch * M + tok0) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
  if (ok1) *reinterpret_cast<uint4*>(qT + (int64_t)(ch + 1) * M + tok0) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
}

// ---------------------------------------------------------------------------
// 128x1 transposed quantizer for C % 8 == 0, launched for F32 inputs (BF16
// inputs take the wave kernel below): one workgroup per (token group g, 64
// channels), 16-byte loads and an LDS transpose of the codes.
// Lane l of wave w holds channels c0 + 8(l%8) .. +7 of tokens
// 32w + 4(l/8) .. +3 of the group: each load instruction reads 8 whole
// 128-byte token rows. Per-channel amax: a max over the lane's 4 tokens, then
// over the 32 token slices through LDS. Each lane encodes its 4 tokens of each
// of its channels (4 bytes of a qT row) into an LDS tile [channel][token],
// which is written out as 16-byte pieces, 8 lanes per 128-byte qT row.
//
// GROUPED: the tokens are per-expert row ranges [off[e], off[e+1]); each
// expert's tokens are cut into groups of 128 from its first row, its last
// group padded with zeros (+0 codes) to 128 columns of qT, and the groups of
// all experts are numbered expert-major: group g = (experts' groups before e)
// + j covers rows off[e] + 128 j .. and qT columns 128 g .. 128 g + 127, with
// scales in row g of sT. Otherwise group g is rows 128 g .. 128 g + 127.
// ld is the row length of qT (M when not grouped).
// ---------------------------------------------------------------------------
constexpr int kTPitch = kGroup + 16;   // tile row pitch in bytes (16-byte aligned)

template <bool BF16, bool GROUPED, bool POW2>
__global__ __launch_bounds__(256) void quant_act_128x1_T_v8_kernel(
    const void* __restrict__ x, int64_t M, int C, uint8_t* __restrict__ qT, float* __restrict__ sT,
    const int32_t* __restrict__ off, int E, int64_t ld) {
  __shared__ float red[32][65];
  __shared__ float scl[64];
  __shared__ __align__(16) uint8_t tile[64 * kTPitch];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int cg = lane & 7, ts = lane >> 3;
  const int g = blockIdx.y;
  int64_t row0 = (int64_t)g * kGroup;   // first input row of the group
  int n_rows = kGroup;                  // its valid rows
  if constexpr (GROUPED) {
    const ExpertSlot es = locate_expert(off, E, (int)M, g, kGroup, 1);
    if (es.e < 0) return;               // past the last group (uniform over the workgroup)
    row0 = es.r0 + (int64_t)kGroup * (g - es.base);
    n_rows = min(kGroup, es.r1 - (int)row0);
  }
  const int c0 = blockIdx.x * 64;
  const int ch = c0 + 8 * cg;
  const bool cok = ch < C;   // C % 8 == 0: all 8 channels valid or none
  const int tl = 32 * w + 4 * ts;            // first of this lane's 4 tokens within the group

  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = GROUPED ? min(tl + i, n_rows - 1) : tl + i;
    load8<BF16>(x, (row0 + r) * C + (cok ? ch : 0), v[i]);
    if (GROUPED && tl + i >= n_rows) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float m = fmaxf(fmaxf(fabsf(v[0][j]), fabsf(v[1][j])), fmaxf(fabsf(v[2][j]), fabsf(v[3][j])));
    red[w * 8 + ts][8 * cg + j] = m;
  }
  __syncthreads();
  if (t < 64) {
    float amax = red[0][t];
#pragma unroll
    for (int r = 1; r < 32; ++r) amax = fmaxf(amax, red[r][t]);
    const float sc = scale_rule<POW2>(amax);
    scl[t] = sc;
    if (c0 + t < C) sT[(int64_t)g * C + c0 + t] = sc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const GroupDiv gd = div_of_scale_rule<BF16, POW2>(scl[8 * cg + j]);
    *reinterpret_cast<uint32_t*>(tile + (8 * cg + j) * kTPitch + tl) =
        pack4_rule<BF16, POW2>(v[0][j], v[1][j], v[2][j], v[3][j], gd);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = t + 256 * k;
    const int r = p >> 3, piece = p & 7;
    if (c0 + r < C)
      *reinterpret_cast<uint4*>(qT + (int64_t)(c0 + r) * ld + (int64_t)g * kGroup + 16 * piece) =
          *reinterpret_cast<const uint4*>(tile + r * kTPitch + 16 * piece);
  }
}

// ---------------------------------------------------------------------------
// 128x1 transposed quantizer for BF16 inputs with C % 8 == 0: one wave per
// (token group g, 64 channels), no LDS and no barrier. Lane l holds channels
// c0 + 8(l%8) .. +7 of the 16 consecutive tokens 16(l/8) .. +15 of the group:
// load i reads token 16(l/8) + i, so each load instruction covers 8 whole
// 128-byte token rows, and all 16 are issued before any compute. A channel's
// amax is the max over the lane's 16 tokens, then over the 8 lanes sharing the
// channel (lane bits 3..5: a DPP rotation by 8 within the 16-lane row, then
// xor 16 and xor 32). Each lane then encodes its 16 tokens of each of its
// channels, 16 consecutive bytes of a qT row, and stores them directly: one
// store instruction writes 8 whole 128-byte pieces of qT rows.
// (F32 inputs keep the kernel above: 8 F32 channels are 32 bytes, which would
// split every load into two half-line requests.)
// GROUPED and the group numbering as for the kernel above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t word_of(const uint4& d, int k) {
  return k == 0 ? d.x : k == 1 ? d.y : k == 2 ? d.z : d.w;
}

template <bool GROUPED, bool POW2>
__global__ __launch_bounds__(256) void quant_act_128x1_T_wave_kernel(
    const uint16_t* __restrict__ x, int64_t M, int C, uint8_t* __restrict__ qT, float* __restrict__ sT,
    const int32_t* __restrict__ off, int E, int64_t ld) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.y;
  int64_t row0 = (int64_t)g * kGroup;   // first input row of the group
  int n_rows = kGroup;                  // its valid rows
  if constexpr (GROUPED) {
    const ExpertSlot es = locate_expert(off, E, (int)M, g, kGroup, 1);
    if (es.e < 0) return;               // past the last group
    row0 = es.r0 + (int64_t)kGroup * (g - es.base);
    n_rows = min(kGroup, es.r1 - (int)row0);
  }
  const int c0 = (blockIdx.x * 4 + w) * 64;
  if (c0 >= C) return;                  // no barrier below: a wave may leave alone
  const int ch = c0 + 8 * (lane & 7);
  const bool cok = ch < C;              // C % 8 == 0: all 8 channels valid or none
  const int tb = 16 * (lane >> 3);      // first of the lane's 16 tokens

  uint4 raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = GROUPED ? min(tb + i, n_rows - 1) : tb + i;
    raw[i] = load16_stream(x + (row0 + r) * C + (cok ? ch : 0));
  }
  // token tb + i, channel ch + j, widened exactly to FP32 (rows past the
  // group's end read as zeros)
  auto val = [&](int i, int j) {
    const uint32_t d = word_of(raw[i], j >> 1);
    const float f = __uint_as_float((j & 1) ? (d & 0xFFFF0000u) : (d << 16));
    return GROUPED && tb + i >= n_rows ? 0.0f : f;
  };
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(val(i, j)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x128, 0xF, 0xF, false)));  // ror 8
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    sc[j] = scale_rule<POW2>(m);
  }
  // Widen again for the encoding rather than keep 128 widened values live:
  // the packed loads take half the registers.
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
  if (lane < 8 && cok) {
    float4* sp = reinterpret_cast<float4*>(sT + (int64_t)g * C + ch);
    sp[0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
    sp[1] = make_float4(sc[4], sc[5], sc[6], sc[7]);
  }
  if (!cok) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const GroupDiv gd = div_of_scale_rule<true, POW2>(sc[j]);
    uint32_t wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wd[k] = pack4_rule<true, POW2>(val(4 * k, j), val(4 * k + 1, j), val(4 * k + 2, j), val(4 * k + 3, j), gd);
    *reinterpret_cast<uint4*>(qT + (int64_t)(ch + j) * ld + (int64_t)g * kGroup + tb) =
        make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
}

// ---------------------------------------------------------------------------
// Both quantizations of one BF16 activation in one pass over it (C a multiple
// of 256): the 128x1 groups, written transposed, exactly as the wave kernel
// above forms them, and the 1x128 groups along each token's channels, as the
// 1x128 kernel forms them. The backward pass needs dY both ways (1x128 for
// Dgrad, 128x1 for Wgrad); one pass reads it once. Lane layout of the wave
// kernel: wave w holds channels c0 .. c0+63 (c0 = 256 bx + 64 w), lane l the
// 8 channels c0 + 8(l%8) .. of the 16 tokens 16(l/8) .. of the group. A
// token's 128-channel group is the channels of the wave pair (2p, 2p+1): its
// maximum is reduced over the 8 lanes that hold the token in each wave
// (xor 1, 2, 4) and over the pair through LDS. Each lane then writes, per
// channel, its 16 tokens' codes (16 bytes of a qT row) and, per token, its 8
// channels' codes (8 bytes of a q row).
// GROUPED as for the wave kernel: rows past the group's valid rows read as
// zeros for the 128x1 groups, and are neither read as tokens of their own
// nor written to q and s.
// ---------------------------------------------------------------------------
template <bool GROUPED>
__global__ __launch_bounds__(256) void quant_act_dual_kernel(
    const uint16_t* __restrict__ x, int64_t M, int C, uint8_t* __restrict__ q, float* __restrict__ s,
    uint8_t* __restrict__ qT, float* __restrict__ sT, const int32_t* __restrict__ off, int E, int64_t ld) {
  __shared__ float red[4][kGroup];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = blockIdx.y;
  int64_t row0 = (int64_t)g * kGroup;   // first input row of the group
  int n_rows = kGroup;                  // its valid rows
  if constexpr (GROUPED) {
    const ExpertSlot es = locate_expert(off, E, (int)M, g, kGroup, 1);
    if (es.e < 0) return;               // past the last group (the same for every wave)
    row0 = es.r0 + (int64_t)kGroup * (g - es.base);
    n_rows = min(kGroup, es.r1 - (int)row0);
  }
  const int c0 = (blockIdx.x * 4 + w) * 64;   // C % 256 == 0: every wave has its 64 channels
  const int ch = c0 + 8 * (lane & 7);
  const int tb = 16 * (lane >> 3);

  uint4 raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = GROUPED ? min(tb + i, n_rows - 1) : tb + i;
    raw[i] = load16_stream(x + (row0 + r) * C + ch);
  }
  auto val = [&](int i, int j) {
    const uint32_t d = word_of(raw[i], j >> 1);
    const float f = __uint_as_float((j & 1) ? (d & 0xFFFF0000u) : (d << 16));
    return GROUPED && tb + i >= n_rows ? 0.0f : f;
  };
  // 128x1: per channel, over the group's tokens
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(val(i, j)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x128, 0xF, 0xF, false)));  // ror 8
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    sc[j] = scale_rule<false>(m);
  }
  // widen again for each later use rather than keep 128 widened values live
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
  if (lane < 8) {
    float4* sp = reinterpret_cast<float4*>(sT + (int64_t)g * C + ch);
    sp[0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
    sp[1] = make_float4(sc[4], sc[5], sc[6], sc[7]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const GroupDiv gd = div_of_scale_rule<true, false>(sc[j]);
    uint32_t wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wd[k] = pack4_rule<true, false>(val(4 * k, j), val(4 * k + 1, j), val(4 * k + 2, j), val(4 * k + 3, j), gd);
    *reinterpret_cast<uint4*>(qT + (int64_t)(ch + j) * ld + (int64_t)g * kGroup + tb) =
        make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
  // 1x128: per token, over the wave pair's 128 channels
  float tm[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(val(i, j)));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    tm[i] = m;
  }
  if ((lane & 7) == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[w][tb + i] = tm[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) tm[i] = fmaxf(tm[i], red[w ^ 1][tb + i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));

  const int kb = c0 / kGroup;   // the 1x128 group column of this wave's channels
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (GROUPED && tb + i >= n_rows) continue;
    const int64_t row = row0 + tb + i;
    const GroupDiv gt = div_rule<true, false>(tm[i]);
    const uint2 codes = make_uint2(pack4_rule<true, false>(val(i, 0), val(i, 1), val(i, 2), val(i, 3), gt),
                                   pack4_rule<true, false>(val(i, 4), val(i, 5), val(i, 6), val(i, 7), gt));
    *reinterpret_cast<uint2*>(q + row * C + ch) = codes;
    if ((lane & 7) == 0 && (w & 1) == 0) s[(int64_t)kb * M + row] = gt.s;
  }
}

// ---------------------------------------------------------------------------
// Launchers (shapes validated by the C ABI layer).
// ---------------------------------------------------------------------------
hipError_t launch_quant_act_1x128(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, uint8_t* q,
                                  float* s, hipStream_t stream) {
  const int64_t nkb = K / kGroup;
  const int64_t nrb = (M + 4 * kActRows - 1) / (4 * kActRows);
  const int64_t gy = nrb < 65535 ? nrb : 65535;
  const dim3 grid((unsigned)((nkb + 3) / 4), (unsigned)gy, (unsigned)((nrb + gy - 1) / gy));
  auto go = [&](auto bf, auto p2) {
    hipLaunchKernelGGL((quant_act_1x128_kernel<decltype(bf)::value, decltype(p2)::value>), grid, dim3(256), 0,
                       stream, x, M, (int)K, q, s);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (bf16) pow2 ? go(T{}, T{}) : go(T{}, F{});
  else pow2 ? go(F{}, T{}) : go(F{}, F{});
  return hipGetLastError();
}

hipError_t launch_quant_w_128x128(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, uint8_t* q,
                                  float* s, uint8_t* qT, float* sT, hipStream_t stream) {
  const dim3 grid((unsigned)(K / kGroup), (unsigned)(N / kGroup));
  auto go = [&](auto bf, auto tr, auto p2) {
    hipLaunchKernelGGL((quant_w_128x128_kernel<decltype(bf)::value, decltype(tr)::value, decltype(p2)::value>),
                       grid, dim3(256), 0, stream, w, (int)N, (int)K, q, s, qT, sT);
  };
  using T = std::true_type;
  using F = std::false_type;
  auto with_tr = [&](auto bf, auto p2) { qT != nullptr ? go(bf, T{}, p2) : go(bf, F{}, p2); };
  if (bf16) pow2 ? with_tr(T{}, T{}) : with_tr(T{}, F{});
  else pow2 ? with_tr(F{}, T{}) : with_tr(F{}, F{});
  return hipGetLastError();
}

hipError_t launch_quant_act_128x1_T(const void* x, bool bf16, bool pow2, int64_t M, int64_t C, uint8_t* qT,
                                    float* sT, hipStream_t stream) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(M / kGroup));
  using T = std::true_type;
  using F = std::false_type;
  if (C % 8 == 0 && bf16) {
    const dim3 wgrid((unsigned)((C + 255) / 256), (unsigned)(M / kGroup));
    auto go = [&](auto p2) {
      hipLaunchKernelGGL((quant_act_128x1_T_wave_kernel<false, decltype(p2)::value>), wgrid, dim3(256), 0, stream,
                         static_cast<const uint16_t*>(x), M, (int)C, qT, sT, nullptr, 0, M);
    };
    pow2 ? go(T{}) : go(F{});
    return hipGetLastError();
  }
  if (C % 8 == 0) {
    auto go = [&](auto p2) {
      hipLaunchKernelGGL((quant_act_128x1_T_v8_kernel<false, false, decltype(p2)::value>), grid, dim3(256), 0,
                         stream, x, M, (int)C, qT, sT, nullptr, 0, M);
    };
    pow2 ? go(T{}) : go(F{});
    return hipGetLastError();
  }
  auto go = [&](auto bf, auto pair, auto p2) {
    hipLaunchKernelGGL((quant_act_128x1_T_kernel<decltype(bf)::value, decltype(pair)::value, decltype(p2)::value>),
                       grid, dim3(256), 0, stream, x, M, (int)C, qT, sT);
  };
  auto with_pair = [&](auto bf, auto p2) { (C % 2) == 0 ? go(bf, T{}, p2) : go(bf, F{}, p2); };
  if (bf16) pow2 ? with_pair(T{}, T{}) : with_pair(T{}, F{});
  else pow2 ? with_pair(F{}, T{}) : with_pair(F{}, F{});
  return hipGetLastError();
}

hipError_t launch_quant_act_128x1_T_grouped(const void* x, bool bf16, int64_t M_total, int64_t C,
                                            const int32_t* offsets, int E, int64_t ld, uint8_t* qT,
                                            float* sT, hipStream_t stream) {
  // ld / 128 bounds the number of groups (validated: ld >= M_total + 127 E)
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(ld / kGroup));
  if (bf16)
    hipLaunchKernelGGL((quant_act_128x1_T_wave_kernel<true, false>), dim3((unsigned)((C + 255) / 256), grid.y),
                       dim3(256), 0, stream, static_cast<const uint16_t*>(x), M_total, (int)C, qT, sT, offsets, E,
                       ld);
  else
    hipLaunchKernelGGL((quant_act_128x1_T_v8_kernel<false, true, false>), grid, dim3(256), 0, stream, x, M_total,
                       (int)C, qT, sT, offsets, E, ld);
  return hipGetLastError();
}

hipError_t launch_quant_act_dual(const void* x, bool bf16, int64_t M, int64_t C, uint8_t* q, float* s,
                                 uint8_t* qT, float* sT, const int32_t* offsets, int E, int64_t ld,
                                 hipStream_t stream) {
  const bool grouped = offsets != nullptr;
  if (bf16 && C % 256 == 0) {
    const dim3 grid((unsigned)(C / 256), (unsigned)((grouped ? ld : M) / kGroup));
    if (grouped)
      hipLaunchKernelGGL((quant_act_dual_kernel<true>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                         M, (int)C, q, s, qT, sT, offsets, E, ld);
    else
      hipLaunchKernelGGL((quant_act_dual_kernel<false>), grid, dim3(256), 0, stream,
                         static_cast<const uint16_t*>(x), M, (int)C, q, s, qT, sT, nullptr, 0, M);
    return hipGetLastError();
  }
  // other inputs: the two passes, one after the other
  const hipError_t e = launch_quant_act_1x128(x, bf16, false, M, C, q, s, stream);
  if (e != hipSuccess) return e;
  if (grouped) return launch_quant_act_128x1_T_grouped(x, bf16, M, C, offsets, E, ld, qT, sT, stream);
  return launch_quant_act_128x1_T(x, bf16, false, M, C, qT, sT, stream);
}

}  // namespace fp8bs
