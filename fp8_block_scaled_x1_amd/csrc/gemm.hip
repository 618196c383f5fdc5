// Block-scaled FP8 GEMM with per-chunk FP32 promotion, for gfx950.
//
// The method (DeepSeek-V3 report section 3.3.2; the promotion scheme of its
// Figure 7(b) as paraphrased on the why-be.why-be.co.kr page, the per-group
// scaling along K on the innerforce.co.kr page): the FP8 product is formed one
// 128-wide K chunk at a time; each chunk's partial result is promoted to FP32,
// multiplied by the A row's and the B column's group scale for that chunk and
// added to an FP32 accumulator:
//
//   C[m][n] = bf16( sum_kb sA[kb][m] * sb(kb,n) * sum_{k in kb} A[m][k] * B[n][k] )
//
// On H800 the partial lives in Tensor Core accumulators and promotion is a
// copy to CUDA-core registers. On gfx950 the MFMA result already lands in the
// wave's VGPRs, so promotion is one VALU FMA per output element per chunk on
// registers the MFMA just wrote; the hardware co-issues it with the MFMAs of
// the next subtile.
//
// Structure (one BM x BN output tile per workgroup of 8 waves; 4 for the
// 64x64 tiles and the hardware-scaled variant's 256x256 tiles):
//   * one pipeline stage = one K chunk: A[BM][128] + B[BN][128] bytes plus the
//     chunk's scale vectors, moved L2 -> LDS with direct-to-LDS loads (no VGPR
//     staging); two to four stages per operand; one barrier per chunk;
//   * every direct-to-LDS load instruction reads 8 whole 128-byte rows (full
//     cache lines); inside LDS the 16-byte column of row r is XOR-swizzled with
//     (r & 7) ^ ((r >> 3) & 1), which keeps the MFMA fragment reads free of
//     bank conflicts;
//   * each wave owns a WM x WN subtile made of 16x16 E4M3 MFMA tiles
//     (v_mfma_f32_16x16x128_f8f6f4): exactly one MFMA per 16x16 tile per
//     chunk, so the MFMA covers the whole promotion interval and starts from
//     zero every chunk; the fragments of the smaller operand are held for the
//     chunk, those of the other are streamed subtile by subtile, and the MFMAs
//     of one step are issued before the promotion FMAs of the previous step;
//   * MFMA operands are swapped (src0 = B rows, src1 = A rows) so that each
//     lane's four results share one A row (one sA value) and sit at four
//     consecutive n (one 8-byte BF16 store);
//   * the chunk's sA vector (and sB in row mode) travels with the stage through
//     LDS; a block-mode B scale is a scalar load;
//   * workgroup -> tile mapping is XCD-aware: consecutive tiles in a grouped
//     (8 m-tiles wide) order land on the same XCD, so the A and B panels they
//     share stay in that XCD's L2;
//   * the kernel (tile shape and ring depth) is chosen on the host per problem
//     from an estimate of its time: large tiles in whole rounds of the CUs for
//     large problems, small ones spread over all CUs for problems with few
//     tiles; the grouped GEMM leaves a short last round to a second launch of
//     small subtiles.

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace gemm {

constexpr int BK = kGroup;
// tile-order grouping for L2 reuse (m-tiles per group): measured best at 4
// for the dense GEMM (up to 6% over 8 on the shapes timed) and at 8 for the
// grouped MoE GEMMs (MoE up 2% slower at 4 and at 16, MoE down 1% slower at 16)
constexpr int kGroupM = 8, kGroupMDense = 4;
constexpr int kXcds = 8;

template <int BM_, int BN_, int WGM_, int WGN_, int DA_, int DB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int DA = DA_, DB = DB_;                    // ring depth per operand
  static constexpr int WM = BM / WGM, WN = BN / WGN;          // wave subtile
  static constexpr int MS = WM / 16, NS = WN / 16;            // MFMA tiles per wave
  // one ring slot: the operand's 128-wide K chunk, then its scale vector
  // (sA[BM]; sB[BN] in row mode) padded to whole 64-float pieces
  static constexpr int kAPieces = (BM + 63) / 64, kBPieces = (BN + 63) / 64;  // scale loads
  static constexpr int kASlot = BM * BK + 256 * kAPieces, kBSlot = BN * BK + 256 * kBPieces;
  static constexpr int kBRing = DA * kASlot;                  // B ring follows the A ring
  static constexpr int kLdsBytes = DA * kASlot + DB * kBSlot;
  static constexpr int kASlices = BM / 8, kBSlices = BN / 8;  // 1 KB load slices per chunk
  static constexpr int kWaves = WGM * WGN, kThreads = 64 * kWaves;
  static constexpr int kASlicesPerWave = (kASlices + kWaves - 1) / kWaves;
  static constexpr int kBSlicesPerWave = (kBSlices + kWaves - 1) / kWaves;
  static constexpr bool kHoldB = NS <= MS;                    // hold the smaller operand
  static_assert(WGM * WGN == 8 || WGM * WGN == 4, "8 or 4 waves");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BM % 8 == 0 && BN % 8 == 0, "tile shape");
  static_assert((DA >= 2 && DA <= 3 && DB >= 2 && DB <= 3) || (DA == 4 && DB == 4),
                "rings two or three deep, or both four deep");
  static_assert(kAPieces <= 4 && kBPieces <= 4, "scale loads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// 256x256, waves 2x4 of 128x64, both operands two deep;
// 256x224, waves 4x2 of 64x112, A three deep; 224x256, waves 2x4 of 112x64, B three deep
using Cfg256x256 = Cfg<256, 256, 2, 4, 2, 2>;
using Cfg256x224 = Cfg<256, 224, 4, 2, 3, 2>;
using Cfg224x256 = Cfg<224, 256, 2, 4, 2, 3>;
// Smaller tiles for problems with few output tiles (skinny M, few tokens),
// which the large tiles would leave on a fraction of the CUs: 128x256, waves
// 2x4 of 64x64; 128x128, waves 4x2 of 32x64; 64x64, 4 waves 2x2 of 32x32.
// The two smallest leave registers and LDS for two or more workgroups per CU.
using Cfg128x256 = Cfg<128, 256, 2, 4, 2, 2>;
using Cfg128x128 = Cfg<128, 128, 4, 2, 2, 2>;
using Cfg64x64 = Cfg<64, 64, 2, 2, 2, 2>;
// The same two with deeper rings: loads run two or three chunks ahead, which
// a lone workgroup on its CU needs to cover the load latency, at the price of
// co-residency (128x128 four deep: one workgroup per CU; 64x64 three deep:
// three; 64x64 four deep: two)
using Cfg128x128d4 = Cfg<128, 128, 4, 2, 4, 4>;
using Cfg64x64d3 = Cfg<64, 64, 2, 2, 3, 3>;
using Cfg64x64d4 = Cfg<64, 64, 2, 2, 4, 4>;
// For the two-layout quantizing epilogue on problems with few tiles: 128x128
// with 8 waves of 128x16, so that each wave's rows are one 128x1 group
using Cfg128x128q2 = Cfg<128, 128, 1, 8, 4, 4>;
// Subtiles of the tail launches (a last partial round of 256x256 tiles, dense
// or grouped, recomputed over every CU), and how many of their workgroups
// share a CU (LDS and registers)
using TailCfg = Cfg64x64d3;
constexpr int kTailPerCu = 3;
// 256x256 with 4 waves of 128x128 (one per SIMD, up to 512 registers each):
// only for the hardware-scaled variant, whose accumulators the MFMA updates
// in place (they can live in AGPRs), so no promotion needs them in VGPRs
using Cfg256x256w4 = Cfg<256, 256, 2, 2, 2, 2>;

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct HBM/L2 -> LDS load of 16 (or 4) bytes per lane: lane i writes LDS
// bytes lds_addr + i*16 (i*4) from global address base + voff. Written as asm
// rather than the compiler builtin because the compiler cannot tell the two
// pipeline stages apart and would otherwise wait for the next stage's loads
// before every read of the current one. The caller waits (s_waitcnt + barrier)
// before reading what these loads wrote. M0 is declared clobbered (one
// scalar move per load instead of a save and a restore); the asm has no VGPR
// outputs.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)p);
}

// Workgroups are dispatched round-robin over the XCDs. Renumber them so that
// the ids one XCD receives form one contiguous range (a bijection for any grid).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Grouped tile order: group_m m-tiles by all n-tiles, column-major inside a group.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn,
                                            int group_m = kGroupM) {
  const int group = group_m * tiles_n;
  const int g = pid / group;
  const int first = g * group_m;
  const int gm = min(tiles_m - first, group_m);
  const int in = pid - g * group;
  tm = first + in % gm;
  tn = in / gm;
}

// 16-byte column swizzle of LDS row r.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// MFMA operand fragment of the 16-row subtile starting at tile row 16*subtile:
// lane l gets row l%16, K bytes 32*(l/16) .. +31 of the chunk.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int subtile, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* rowp = tile + (subtile * 16 + r) * BK;
  const int x = swz(r);
  const uint4 lo = *reinterpret_cast<const uint4*>(rowp + (((2 * g) ^ x) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((2 * g + 1) ^ x) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

struct Tile {
  const uint8_t* A;   // whole A, row-major [rows][K]
  const float* sA;    // [K/128][sa_stride]
  int sa_stride;
  const uint8_t* B;   // this tile's B, [N][K]
  const float* sB;    // block: [N/128][K/128]; row: [K/128][N]
  uint16_t* C;        // [rows][N] (BF16 output)
  uint8_t* Q;         // [rows][N] (quantized output: E4M3 codes)
  float* sQ;          // [N/128][rows] (quantized output: 1x128 group scales)
  uint8_t* QT;        // [N][rows] (quantized output, 128x1 groups, transposed codes)
  float* sQT;         // [rows/128][N] (its scales)
  int m0, row_end;    // tile rows m0 .. m0+BM-1, valid below row_end
  int n0, N, K;       // K: inner length of this tile's product (a multiple of 128)
  int ld;             // row stride of A and B in bytes (K for a plain GEMM)
};

// Wait until at most N of this wave's vector-memory operations are pending
// (direct-to-LDS loads complete in issue order) and all its LDS reads and
// scalar loads have returned, then meet the other waves at the barrier. The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// QOUT: the epilogue writes the 1x128 quantization (E4M3 codes and FP32
// scales per row and 128 columns) of the BF16-rounded result instead of the
// BF16 result itself; QOUT == 2 also writes its 128x1 quantization (128 rows
// of one column per group), transposed.
// HW: the scales are powers of two and the MFMA applies them itself, as E8M0
// block scales of its operands (the exponent field of an FP32 power of two is
// its E8M0 code); each MFMA then accumulates straight into the FP32
// accumulator and no promotion FMAs run.
template <class G, int ROW_MODE, int QOUT = 0, int HW = 0>
__device__ __forceinline__ void run_tile(const Tile& t, uint8_t* smem) {
  constexpr int MS = G::MS, NS = G::NS, WM = G::WM, WN = G::WN;
  constexpr bool kDeepA = G::DA >= 3, kDeepB = G::DB >= 3, kDeep = kDeepA || kDeepB;
  constexpr int kAhead = G::DA == 4 ? 3 : 2;   // chunks a deep ring loads ahead
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int kW = G::kWaves;
  __builtin_assume(wave >= 0 && wave < kW);
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  const int nkb = t.K / BK;
  const int a_last = t.row_end - 1;
  const int b_last = t.N - 1;

  // Direct-to-LDS operand loads. Slice s (1 KB) of an operand covers its tile
  // rows 8s .. 8s+7; this wave loads slices wave, wave+W, ... (W waves). Lane p fetches
  // row 8s + p/8, logical 16-byte column (p%8) ^ swz(row), and writes physical
  // column p%8. Offsets are 32-bit from a uniform base (M*K, N*K < 2^31); rows
  // past the end are clamped (their results are never stored). A wave whose
  // last slice index is past the tile repeats its previous slice (same bytes
  // to the same place), so every wave issues the same number of loads.
  auto slice_of = [&](int j, int slices) { return wave + kW * j < slices ? wave + kW * j : wave + kW * (j - 1); };
  auto slice_off = [&](int s, int first, int last) {
    const int rr = s * 8 + (lane >> 3);
    const uint32_t col = (uint32_t)(((lane & 7) ^ swz(rr)) << 4);
    return (uint32_t)min(first + rr, last) * (uint32_t)t.ld + col;
  };
  constexpr int kAL = G::kASlicesPerWave, kBL = G::kBSlicesPerWave;
  uint32_t aoffs[kAL], boffs[kBL], alds[kAL], blds[kBL];
#pragma unroll
  for (int j = 0; j < kAL; ++j) {
    const int sl = slice_of(j, G::kASlices);
    aoffs[j] = slice_off(sl, t.m0, a_last);
    alds[j] = (uint32_t)sl * 1024u;
  }
#pragma unroll
  for (int j = 0; j < kBL; ++j) {
    const int sl = slice_of(j, G::kBSlices);
    boffs[j] = slice_off(sl, t.n0, b_last);
    blds[j] = (uint32_t)sl * 1024u;
  }
  // Scale vectors: piece q = (waves - 1 - wave) mod pieces (64 floats, one 4-byte load
  // per lane) of sA[kb][m0 ..] and, in row mode, of sB[kb][n0 ..]; rows are
  // clamped, lanes past the tile write into the slot's padding, and pieces
  // loaded by two waves carry the same bytes. In block mode every wave loads
  // the chunk's B scales of the tile's (at most kSBlk) 128-column blocks,
  // sB[n0/128 + l][kb] for lane l (lanes past them repeat the last one), so no
  // scalar memory load sits in the loop (its return would gate every LDS wait).
  const int qa = (kW - 1 - wave) % G::kAPieces, qb = (kW - 1 - wave) % G::kBPieces;
  const uint32_t sa_off = 4u * (uint32_t)min(t.m0 + 64 * qa + lane, a_last);
  constexpr int kSBlk = G::BN / BK + 2;
  const int blk_first = t.n0 / BK;
  const uint32_t sb_off = ROW_MODE ? 4u * (uint32_t)min(t.n0 + 64 * qb + lane, b_last)
                                   : 4u * (uint32_t)(min(blk_first + min(lane, kSBlk - 1), b_last / BK) * nkb);
  // loads per wave per chunk of each operand
  constexpr int kNA = kAL + 1, kNB = kBL + 1;

  const uint32_t lds = lds_addr_of(smem);
  // j-th load of this wave for operand A (B) of chunk kb into ring slot `slot`
  auto a_load = [&](int j, int kb, int slot) {
    const uint32_t st = lds + (uint32_t)(slot * G::kASlot);
    if (j < kAL)
      lds_dma16(t.A + (int64_t)kb * BK, aoffs[j], st + alds[j]);
    else
      lds_dma4(t.sA + (int64_t)kb * t.sa_stride, sa_off, st + (uint32_t)(G::BM * BK + 256 * qa));
  };
  auto b_load = [&](int j, int kb, int slot) {
    const uint32_t st = lds + (uint32_t)(G::kBRing + slot * G::kBSlot);
    if (j < kBL)
      lds_dma16(t.B + (int64_t)kb * BK, boffs[j], st + blds[j]);
    else if (ROW_MODE)
      lds_dma4(t.sB + (int64_t)kb * t.N, sb_off, st + (uint32_t)(G::BN * BK + 256 * qb));
    else
      lds_dma4(t.sB + kb, sb_off, st + (uint32_t)(G::BN * BK));
  };
  auto issue_a = [&](int kb, int slot) {
#pragma unroll
    for (int j = 0; j < kNA; ++j) a_load(j, kb, slot);
  };
  auto issue_b = [&](int kb, int slot) {
#pragma unroll
    for (int j = 0; j < kNB; ++j) b_load(j, kb, slot);
  };

  v4f acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Block mode: the B scale of n-subtile j is sB[(n of the subtile)/128][kb],
  // uniform over the subtile. A wave's WN <= 128 columns span at most two
  // 128-column blocks: subtiles below `split` lie in the first, the rest in
  // the second.
  static_assert(WN <= BK, "a wave's columns span at most two scale blocks");
  const int ncol0 = t.n0 + wn * WN;
  const int blk_lo = min(ncol0, b_last) / BK;
  const int blk_hi = min(blk_lo + 1, b_last / BK);
  const int split = min(NS, (BK - (ncol0 & (BK - 1))) / 16);
  // the slot's B-scale area holds the chunk's scales of blocks blk_first ..
  const int sbi_lo = blk_lo - blk_first, sbi_hi = blk_hi - blk_first;

  // The fragments of the smaller operand ("held", NH of them) are read once per
  // chunk; those of the other ("streamed", NT) one step ahead of their use.
  // Step t issues the MFMAs of streamed subtile t against every held subtile,
  // then the promotion of step t-1, so each promotion waits on MFMAs issued a
  // whole step earlier.
  constexpr bool HA = !G::kHoldB;                 // A held, B streamed
  constexpr int NH = HA ? MS : NS, NT = HA ? NS : MS;
  const int h_sub = HA ? wm * MS : wn * NS;       // first held / streamed subtile
  const int t_sub = HA ? wn * NS : wm * MS;

  // Per-lane scale values. sa: the lane's A row of subtile i (sA of the chunk,
  // staged in LDS); sb: block mode one uniform value per n-subtile, row mode the
  // lane's four columns of n-subtile j.
  // Per-lane scale values of a chunk: sa[i] for the lane's A row of subtile i;
  // row mode sbr[j] for its four columns of n-subtile j, block mode the B
  // scales lo / hi of the wave's first and second 128-column block.
  struct Scales {
    float sa[MS];
    float sbr[NS][4];
    float lo, hi;
  };
  // Block mode: the products sa[i] * lo and sa[i] * hi, formed once per chunk.
  struct Factors {
    float flo[MS], fhi[MS];
  };
  auto factors = [&](const Scales& sc) {
    Factors f;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      f.flo[i] = sc.sa[i] * sc.lo;
      f.fhi[i] = sc.sa[i] * sc.hi;
    }
    return f;
  };

  auto slot_a = [&](int kb) { return smem + (kb % G::DA) * G::kASlot; };
  auto slot_b = [&](int kb) { return smem + G::kBRing + (kb % G::DB) * G::kBSlot; };
  auto read_t = [&](int kb, int t) {
    return read_frag(HA ? slot_b(kb) : slot_a(kb), t_sub + t, lane);
  };
  // The streamed fragment first, then the held ones in order of use, so that
  // the chunk's first MFMAs wait only for the reads they need.
  auto read_chunk_start = [&](int kb, v8i (&hf)[NH], v8i& tf, Scales& sc) {
    const uint8_t* As = slot_a(kb);
    const uint8_t* Bs = slot_b(kb);
    tf = read_t(kb, 0);
#pragma unroll
    for (int h = 0; h < NH; ++h) hf[h] = read_frag(HA ? As : Bs, h_sub + h, lane);
    const float* sAs = reinterpret_cast<const float*>(As + G::BM * BK) + wm * WM + (lane & 15);
    const float* sBs = reinterpret_cast<const float*>(Bs + G::BN * BK) + wn * WN + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < MS; ++i) sc.sa[i] = sAs[16 * i];
    if constexpr (ROW_MODE) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(sBs + 16 * j);
        sc.sbr[j][0] = v.x; sc.sbr[j][1] = v.y; sc.sbr[j][2] = v.z; sc.sbr[j][3] = v.w;
      }
    } else {
      const float* sBb = reinterpret_cast<const float*>(Bs + G::BN * BK);
      sc.lo = sBb[sbi_lo];
      sc.hi = sBb[sbi_hi];
    }
  };
  // promotion of MFMA tile (i, j): scaled FP32 partial into the FP32
  // accumulator; S is the wave's block split (a compile-time constant)
  auto promote = [&](int i, int j, const v4f& p, const Scales& sc, const Factors& fc, int S) {
    if constexpr (ROW_MODE) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r] * sc.sbr[j][r], sc.sa[i], acc[i][j][r]);
    } else {
      const float f = j < S ? fc.flo[i] : fc.fhi[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r], f, acc[i][j][r]);
    }
  };
  auto promote_step = [&](int t, const v4f (&p)[NH], const Scales& sc, const Factors& fc, int S) {
#pragma unroll
    for (int h = 0; h < NH; ++h) promote(HA ? h : t, HA ? t : h, p[h], sc, fc, S);
  };

  // Chunk x is readable after barrier x. Before it each wave waits for its own
  // loads of chunk x and for its LDS reads of chunk x-1, so after it every
  // wave's loads of chunk x are visible and chunk x-1's slots are free. While
  // chunk x is computed they are refilled, a few loads per step so that no
  // wave stalls on a full load queue: first a shallow operand's chunk x+1,
  // then a deep operand's chunk x+2 (both operands' chunk x+1 without a deep
  // ring, in the first half of the steps; both operands' chunk x+2 when both
  // are three deep). Only the deep loads, issued last, may still be in flight
  // at the next barrier. Chunk indices past the end are clamped: those loads
  // land in free slots and go unused.
  // deep loads that may be in flight at a barrier: those of the kAhead - 1
  // chunks after the one it waits for
  constexpr int kND = ((kDeepA ? kNA : 0) + (kDeepB ? kNB : 0)) * (kAhead - 1);
  constexpr int kItems = kNA + kNB;
  constexpr int kSpread = kDeep ? NT : (NT + 1) / 2;
  auto barrier = [&](int x) {
    if (kDeep && x < nkb)
      wait_and_barrier<kND>();
    else
      wait_and_barrier<0>();
  };
  // load k (0 <= k < kItems) of the refill issued while chunk kb is computed
  auto refill_load = [&](int k, int kb) {
    const int k1 = min(kb + 1, nkb - 1), k2 = min(kb + 2, nkb - 1);
    if constexpr (kDeepA && kDeepB) {
      const int kd = min(kb + kAhead, nkb - 1);
      if (k < kNA) a_load(k, kd, (kb + kAhead) % G::DA);
      else b_load(k - kNA, kd, (kb + kAhead) % G::DB);
    } else if constexpr (kDeepA) {
      if (k < kNB) b_load(k, k1, (kb + 1) % G::DB);
      else a_load(k - kNB, k2, (kb + 2) % G::DA);
    } else if constexpr (kDeepB) {
      if (k < kNA) a_load(k, k1, (kb + 1) % G::DA);
      else b_load(k - kNA, k2, (kb + 2) % G::DB);
    } else {
      if (k < kNA) a_load(k, k1, (kb + 1) % G::DA);
      else b_load(k - kNA, k1, (kb + 1) % G::DB);
    }
  };
  auto refill_step = [&](int t, int kb) {
#pragma unroll
    for (int k = 0; k < kItems; ++k)
      if (k * kSpread / kItems == t) refill_load(k, kb);
  };

  // prologue: chunk 0 of both operands, chunks 1 .. kAhead - 1 of a deep one
  issue_a(0, 0);
  issue_b(0, 0);
#pragma unroll
  for (int c = 1; c < kAhead; ++c) {
    if constexpr (kDeepA) issue_a(min(c, nkb - 1), c);
    if constexpr (kDeepB) issue_b(min(c, nkb - 1), c);
  }
  barrier(0);
  // Retire every scalar load issued so far (kernel arguments), as the
  // compiler sees it: with one pending, each LDS wait in the loop would have
  // to drain all LDS reads (lgkmcnt(0)) instead of only those it needs.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained

  // The main loop, compiled once per block split that can occur.
  auto main_loop = [&](auto split_c) {
    constexpr int S = decltype(split_c)::value;
    v8i hf[NH];
    v8i tf;
    Scales sc;
    read_chunk_start(0, hf, tf, sc);
    // Block mode carries the promotion of a chunk's last step into the first
    // step of the next chunk (zero partials before the first chunk), so every
    // step interleaves MFMAs with promotions; row mode, short of registers for
    // a second set of column scales, finishes it right after the barrier.
    constexpr bool kCarry = !ROW_MODE;
    v4f p_prev[NH];
    Factors f_prev;
    if constexpr (kCarry) {
#pragma unroll
      for (int h = 0; h < NH; ++h) p_prev[h] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < MS; ++i) f_prev.flo[i] = f_prev.fhi[i] = 0.f;
    }
    for (int kb = 0; kb < nkb; ++kb) {
      Factors fc;
      if constexpr (!ROW_MODE) fc = factors(sc);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        refill_step(t, kb);
        v4f p_cur[NH];
        const v8i t_now = tf;
#pragma unroll
        for (int h = 0; h < NH; ++h)
          p_cur[h] = HA ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(t_now, hf[h], v4f{0.f, 0.f, 0.f, 0.f},
                                                                           0, 0, 0, 0, 0, 0)
                        : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(hf[h], t_now, v4f{0.f, 0.f, 0.f, 0.f},
                                                                           0, 0, 0, 0, 0, 0);
        if (t + 1 < NT) tf = read_t(kb, t + 1);
        const bool promoting = t > 0 || kCarry;
        if (t > 0)
          promote_step(t - 1, p_prev, sc, fc, S);
        else if (kCarry)
          promote_step(NT - 1, p_prev, sc, f_prev, S);
        // one MFMA, then a group of six VALU instructions (the promotion),
        // so the two pipes overlap (row mode, with two operations per
        // element, measured 1-2% faster with six than with eight)
        if (promoting) {
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (h == 0 && t + 1 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          }
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) p_prev[h] = p_cur[h];
        __builtin_amdgcn_sched_barrier(0);
      }
      // Every LDS read of chunk kb is issued and the last step's MFMAs are in
      // flight: cross the next chunk's barrier now and read its first fragments
      // while they run. (After the last chunk the reads repeat it and go unused,
      // which keeps the loop branch-free.) The promoted accumulators are pinned
      // first so that the compiler cannot sink the promotions past the barrier.
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          if (t + 1 < NT || kCarry) asm volatile("" : "+v"(acc[HA ? h : t][HA ? t : h]));
      Scales sc_next;
      barrier(kb + 1);
      read_chunk_start(min(kb + 1, nkb - 1), hf, tf, sc_next);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kCarry) {
        f_prev = fc;
      } else {
        promote_step(NT - 1, p_prev, sc, fc, S);
      }
      sc = sc_next;
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kCarry) promote_step(NT - 1, p_prev, sc, f_prev, S);
  };
  // Hardware-scaled main loop. MFMA operand lane l holds row l%16 of its
  // 16-row subtile (and 32 K bytes of it), and its E8M0 scale operand is that
  // row's scale for those 32 K values; with 128-wide groups all four lanes of
  // a row carry the same scale. src0 = B rows (scale sb of column n), src1 =
  // A rows (scale sa of row m).
  auto read_scales_hw = [&](int kb, int (&ea)[MS], int (&eb)[NS]) {
    const float* sAs = reinterpret_cast<const float*>(slot_a(kb) + G::BM * BK) + wm * WM + (lane & 15);
#pragma unroll
    for (int i = 0; i < MS; ++i) ea[i] = (int)(__float_as_uint(sAs[16 * i]) >> 23);
    if constexpr (ROW_MODE) {
      const float* sBs = reinterpret_cast<const float*>(slot_b(kb) + G::BN * BK) + wn * WN + (lane & 15);
#pragma unroll
      for (int j = 0; j < NS; ++j) eb[j] = (int)(__float_as_uint(sBs[16 * j]) >> 23);
    } else {
      const float* sBb = reinterpret_cast<const float*>(slot_b(kb) + G::BN * BK);
      const int elo = (int)(__float_as_uint(sBb[sbi_lo]) >> 23), ehi = (int)(__float_as_uint(sBb[sbi_hi]) >> 23);
#pragma unroll
      for (int j = 0; j < NS; ++j) eb[j] = j < split ? elo : ehi;
    }
  };
  auto main_loop_hw = [&]() {
    v8i hf[NH];
    v8i tf;
    int ea[MS], eb[NS];
    tf = read_t(0, 0);
#pragma unroll
    for (int h = 0; h < NH; ++h) hf[h] = read_frag(HA ? slot_a(0) : slot_b(0), h_sub + h, lane);
    read_scales_hw(0, ea, eb);
    for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        refill_step(t, kb);
        const v8i t_now = tf;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const int i = HA ? h : t, j = HA ? t : h;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(HA ? t_now : hf[h], HA ? hf[h] : t_now,
                                                                       acc[i][j], 0, 0, 0, eb[j], 0, ea[i]);
        }
        if (t + 1 < NT) tf = read_t(kb, t + 1);
        // one MFMA, then the next step's fragment reads, then the other MFMAs:
        // with one wave per SIMD, reads issued after all of a step's MFMAs
        // land after the next step wants them (5-8% slower)
        if (t + 1 < NT) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NH - 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      barrier(kb + 1);
      const int kn = min(kb + 1, nkb - 1);
      tf = read_t(kn, 0);
#pragma unroll
      for (int h = 0; h < NH; ++h) hf[h] = read_frag(HA ? slot_a(kn) : slot_b(kn), h_sub + h, lane);
      read_scales_hw(kn, ea, eb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (HW) {
    main_loop_hw();
  } else if constexpr (ROW_MODE || (G::BN % BK == 0 && BK % WN == 0)) {
    main_loop(std::integral_constant<int, NS>{});   // every wave within one block
  } else {
    switch (split) {
#define FP8BS_SPLIT_CASE(v) \
  case v:                   \
    if constexpr (v < NS) { \
      main_loop(std::integral_constant<int, v>{}); \
      break;                \
    }
      FP8BS_SPLIT_CASE(1)
      FP8BS_SPLIT_CASE(2)
      FP8BS_SPLIT_CASE(3)
      FP8BS_SPLIT_CASE(4)
      FP8BS_SPLIT_CASE(5)
      FP8BS_SPLIT_CASE(6)
      FP8BS_SPLIT_CASE(7)
#undef FP8BS_SPLIT_CASE
      default:
        main_loop(std::integral_constant<int, NS>{});
    }
  }

  // lane holds C[m][n..n+3] of every MFMA tile. With the accumulators in
  // AGPRs (HW) the lane index is read again here rather than kept in a VGPR
  // through the main loop, where every VGPR is taken.
  int lane_e = lane;
  if constexpr (HW) {
    lane_e = (int)threadIdx.x;
    asm volatile("" : "+v"(lane_e));
    lane_e &= 63;
  }
  const int m_lane = t.m0 + wm * WM + (lane_e & 15);
  const int n_lane = t.n0 + wn * WN + 4 * (lane_e >> 4);
  const int r_lane = wm * WM + (lane_e & 15), c_lane = wn * WN + 4 * (lane_e >> 4);   // the same within the tile
  if constexpr (!QOUT) {
    // BF16 epilogue (round to nearest even) through LDS: each wave writes its
    // values into a row-major copy of the tile in the operand slots, idle by
    // now, and the workgroup then stores whole tile rows 16 bytes per lane
    // (a wave's store covers 1 KB of consecutive row bytes instead of 16 rows
    // x 32 bytes); 5-9% faster on the dense and grouped shapes measured.
    constexpr int kPitch = G::BN * 2 + 16;   // tile row pitch in bytes
    static_assert(G::BM * kPitch <= G::kLdsBytes, "the output tile fits the operand slots");
    wait_and_barrier<0>();                   // every wave is done with the operand slots
    // With the accumulators in AGPRs (HW), keep their conversion below the
    // barrier, tile by tile: converted all at once ahead of it, the packed
    // values do not fit the VGPRs that remain.
    if constexpr (HW) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        uint2 o;
        o.x = float_to_bf16_bits(acc[i][j][0]) | (float_to_bf16_bits(acc[i][j][1]) << 16);
        o.y = float_to_bf16_bits(acc[i][j][2]) | (float_to_bf16_bits(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(smem + (r_lane + 16 * i) * kPitch + 2 * (c_lane + 16 * j)) = o;
      }
    wait_and_barrier<0>();
    constexpr int kPieces = G::BN / 8;       // 16-byte pieces per tile row
#pragma unroll 4
    for (int p = tid; p < G::BM * kPieces; p += G::kThreads) {
      const int row = p / kPieces, piece = p % kPieces;
      const int m = t.m0 + row, n = t.n0 + 8 * piece;
      if (m < t.row_end && n < t.N)
        *reinterpret_cast<uint4*>(t.C + (int64_t)m * t.N + n) =
            *reinterpret_cast<const uint4*>(smem + row * kPitch + 16 * piece);
    }
  } else {
    // Quantizing epilogue: the 1x128 quantizer applied to the BF16-rounded
    // result, fused. A 128-column group spans kGW = 128 / WN waves along n;
    // each row's amax is reduced over the lane's values, the four lanes that
    // share the row (xor 16, xor 32) and, through LDS, the group's waves.
    static_assert(G::BN % kGroup == 0 && kGroup % WN == 0, "tile columns must hold whole 128-column groups");
    constexpr int kGW = kGroup / WN;
    float v[MS][NS][4];
    float ra[MS];
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[i][j][r] = __uint_as_float(float_to_bf16_bits(acc[i][j][r]) << 16);
          a = fmaxf(a, fabsf(v[i][j][r]));
        }
      a = fmaxf(a, __shfl_xor(a, 16, 64));
      a = fmaxf(a, __shfl_xor(a, 32, 64));
      ra[i] = a;
    }
    if constexpr (kGW > 1) {
      // red[wave][row of the wave's subtile]: every wave's row maxima, after
      // all waves are done with the operand slots
      float* red = reinterpret_cast<float*>(smem);
      wait_and_barrier<0>();
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < MS; ++i) red[wave * WM + 16 * i + lane] = ra[i];
      }
      wait_and_barrier<0>();
      const int wn0 = wn - wn % kGW;
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int w2 = 0; w2 < kGW; ++w2)
          ra[i] = fmaxf(ra[i], red[(wm * G::WGN + wn0 + w2) * WM + 16 * i + (lane & 15)]);
    }
    // The codes go through LDS like the BF16 epilogue: a row-major copy of
    // the tile's codes (and, for QOUT == 2, a column-major one), after the
    // row maxima; rows of BN (BM) bytes with their 16-byte pieces XOR-swizzled
    // by the row's low bits (four for rows of 256 bytes, which keeps both the
    // 4-byte writes and the 16-byte reads free of bank conflicts).
    constexpr int kRedBytes = (G::kWaves * WM * 4 + 15) / 16 * 16;
    constexpr int kQOff = kRedBytes, kQTOff = kQOff + G::BM * G::BN;
    static_assert(kQTOff + (QOUT == 2 ? G::BN * G::BM : 0) <= G::kLdsBytes, "code tiles fit the operand slots");
    static_assert((G::BN == 256 || G::BN == 128) && (QOUT == 1 || G::BM == 256 || G::BM == 128),
                  "code tile rows of 8 or 16 pieces");
    // byte offset of (row, col) in a code tile with rows of ROWB bytes
    auto swz_off_in = [](auto rowb, int row, int col) {
      constexpr int R = decltype(rowb)::value, P = R / 16;
      return row * R + ((((col >> 4) ^ row) & (P - 1)) << 4) + (col & 15);
    };
    auto swz_off = [&](int row, int col) { return swz_off_in(std::integral_constant<int, G::BN>{}, row, col); };
    auto swz_off_t = [&](int row, int col) { return swz_off_in(std::integral_constant<int, G::BM>{}, row, col); };
    if constexpr (kGW == 1) wait_and_barrier<0>();   // every wave is done with the operand slots
    const int grp = (t.n0 + wn * WN) / kGroup;
    const bool group_ok = t.n0 + wn * WN < t.N;   // N % 128 == 0: a group is wholly in or out
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int m = m_lane + 16 * i;
      const GroupDiv g = group_div<true>(ra[i]);   // the values are BF16 numbers
#pragma unroll
      for (int j = 0; j < NS; ++j)
        *reinterpret_cast<uint32_t*>(smem + kQOff + swz_off(r_lane + 16 * i, c_lane + 16 * j)) =
            e4m3_div_pack4_t<true>(v[i][j][0], v[i][j][1], v[i][j][2], v[i][j][3], g);
      if (m < t.row_end && group_ok && lane < 16 && wn % kGW == 0) t.sQ[(int64_t)grp * t.row_end + m] = g.s;
    }
    if constexpr (QOUT == 2) {
      // 128x1 groups: a wave's WM = 128 rows are one group of each of its
      // columns. Column amax: over the lane's MS rows, then over the 16 lanes
      // that share the column (xor 1, 2, 4, 8). Each lane encodes its four
      // columns of row 16i + lane%16 into one word; a 4x4 byte transpose
      // inside each quad of lanes (DPP quad broadcasts) turns that into four
      // consecutive rows of one column, one 4-byte piece of a QT row.
      static_assert(WM == kGroup, "a wave's rows must form one 128-row group");
      const int m_grp0 = t.m0 + wm * WM;
      const bool rows_ok = m_grp0 < t.row_end;      // rows % 128 == 0: a group is wholly in or out
      const int q = lane & 3;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        GroupDiv gc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = 0.0f;
#pragma unroll
          for (int i = 0; i < MS; ++i) a = fmaxf(a, fabsf(v[i][j][r]));
          a = fmaxf(a, __shfl_xor(a, 1, 64));
          a = fmaxf(a, __shfl_xor(a, 2, 64));
          a = fmaxf(a, __shfl_xor(a, 4, 64));
          a = fmaxf(a, __shfl_xor(a, 8, 64));
          gc[r] = group_div<true>(a);
        }
        const int n_col = n_lane + 16 * j + q;        // this lane's column after the transpose
        if (rows_ok && group_ok) {
          if ((lane & 15) == 0)
            *reinterpret_cast<float4*>(t.sQT + (int64_t)(m_grp0 / kGroup) * t.N + n_lane + 16 * j) =
                make_float4(gc[0].s, gc[1].s, gc[2].s, gc[3].s);
#pragma unroll
          for (int i = 0; i < MS; ++i) {
            const int w = (int)e4m3_div_cols4_bf16(v[i][j], gc);
            // quad lane qq's word, broadcast in its quad (quad_perm [qq,qq,qq,qq])
            const uint32_t w0 = (uint32_t)__builtin_amdgcn_mov_dpp(w, 0x00, 0xF, 0xF, false);
            const uint32_t w1 = (uint32_t)__builtin_amdgcn_mov_dpp(w, 0x55, 0xF, 0xF, false);
            const uint32_t w2 = (uint32_t)__builtin_amdgcn_mov_dpp(w, 0xAA, 0xF, 0xF, false);
            const uint32_t w3 = (uint32_t)__builtin_amdgcn_mov_dpp(w, 0xFF, 0xF, 0xF, false);
            const uint32_t sh = 8u * (uint32_t)q;
            const uint32_t out = ((w0 >> sh) & 0xFFu) | (((w1 >> sh) & 0xFFu) << 8) |
                                 (((w2 >> sh) & 0xFFu) << 16) | (((w3 >> sh) & 0xFFu) << 24);
            *reinterpret_cast<uint32_t*>(smem + kQTOff + swz_off_t(n_col - t.n0, wm * WM + 16 * i + (lane & 12))) =
                out;
          }
        }
      }
    }
    wait_and_barrier<0>();   // the code tiles are complete
    {
      constexpr int kPieces = G::BN / 16;   // 16-byte pieces per code row
#pragma unroll 4
      for (int p = tid; p < G::BM * kPieces; p += G::kThreads) {
        const int row = p / kPieces, piece = p % kPieces;
        const int m = t.m0 + row, n = t.n0 + 16 * piece;
        if (m < t.row_end && n < t.N)
          *reinterpret_cast<uint4*>(t.Q + (int64_t)m * t.N + n) =
              *reinterpret_cast<const uint4*>(smem + kQOff + swz_off(row, 16 * piece));
      }
    }
    if constexpr (QOUT == 2) {
      constexpr int kPieces = G::BM / 16;   // 16-byte pieces per transposed code row
#pragma unroll 4
      for (int p = tid; p < G::BN * kPieces; p += G::kThreads) {
        const int col = p / kPieces, piece = p % kPieces;
        const int n = t.n0 + col, m = t.m0 + 16 * piece;
        if (n < t.N && m < t.row_end)
          *reinterpret_cast<uint4*>(t.QT + (int64_t)n * t.row_end + m) =
              *reinterpret_cast<const uint4*>(smem + kQTOff + swz_off_t(col, 16 * piece));
      }
    }
  }
}

template <class G, int ROW_MODE, int QOUT, int HW = 0>
__global__ __launch_bounds__(G::kThreads, 1) void gemm_kernel(const uint8_t* __restrict__ A,
                                                            const float* __restrict__ sA,
                                                            const uint8_t* __restrict__ B,
                                                            const float* __restrict__ sB,
                                                            uint16_t* __restrict__ C,
                                                            uint8_t* __restrict__ Q,
                                                            float* __restrict__ sQ,
                                                            uint8_t* __restrict__ QT,
                                                            float* __restrict__ sQT, int M, int N,
                                                            int K) {
  __shared__ __align__(16) uint8_t smem[G::kLdsBytes];
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_n = (N + G::BN - 1) / G::BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_coords(pid, tiles_m, tiles_n, tm, tn, kGroupMDense);
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M;
  t.B = B; t.sB = sB; t.C = C; t.Q = Q; t.sQ = sQ; t.QT = QT; t.sQT = sQT;
  t.m0 = tm * G::BM; t.row_end = M;
  t.n0 = tn * G::BN; t.N = N; t.K = K; t.ld = K;
  run_tile<G, ROW_MODE, QOUT, HW>(t, smem);
}

// Per-expert tiles: expert e owns rows [off[e], off[e+1]); its tiles are
// ceil(rows/BM) x ceil(N/BN), numbered expert-major; experts with min_rows
// rows or fewer have none (the decode kernel takes them). The grid is an
// upper bound on the total; workgroups past the last tile exit at once. The
// tiles are spread over the XCDs by their actual number, not the grid's:
// workgroups go to the XCDs in turn, so the first `total` of them hold an
// equal share on each (renumbered to one contiguous range per XCD), where
// renumbering the whole grid would crowd the tiles onto the first XCDs.
//
// With tail_cus > 0 (the device's CU count), a last round of at most
// tail_max tiles is left to grouped_tail_kernel: alone on their CUs those few
// tiles would take a whole round's time while the other CUs idle.
__device__ __forceinline__ int grouped_tail_tiles(int total, int tail_cus, int tail_max) {
  if (tail_cus <= 0) return 0;
  const int rem = total % tail_cus;
  return rem <= tail_max ? rem : 0;
}

template <class G>
__global__ __launch_bounds__(G::kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
    int E, int M_total, int N, int K, int min_rows, int tail_cus, int tail_max) {
  __shared__ __align__(16) uint8_t smem[G::kLdsBytes];
  const int tiles_n = (N + G::BN - 1) / G::BN;
  const int all = total_units(offsets, E, M_total, G::BM, tiles_n, min_rows);
  const int total = all - grouped_tail_tiles(all, tail_cus, tail_max);
  if ((int)blockIdx.x >= total) return;
  const int pid = xcd_remap(blockIdx.x, total);
  // the expert of tile pid (tiles numbered expert-major)
  const ExpertSlot es = locate_expert(offsets, E, M_total, pid, G::BM, tiles_n, min_rows);
  if (es.e < 0) return;
  const int e_found = es.e, r0 = es.r0, r1 = es.r1, base = es.base;
  int tm, tn;
  tile_coords(pid - base, (r1 - r0 + G::BM - 1) / G::BM, tiles_n, tm, tn);
  const int64_t nkb = K / BK;
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M_total;
  t.B = B + (int64_t)e_found * N * K;
  t.sB = sB + (int64_t)e_found * (N / BK) * nkb;
  t.C = C; t.Q = nullptr; t.sQ = nullptr; t.QT = nullptr; t.sQT = nullptr;
  t.m0 = r0 + tm * G::BM; t.row_end = r1;
  t.n0 = tn * G::BN; t.N = N; t.K = K; t.ld = K;
  run_tile<G, 0>(t, smem);
}

// The tiles grouped_gemm_kernel<G> leaves over (the last `rem` of its
// numbering, as it counts them), each computed as (G::BM / S::BM) x
// (G::BN / S::BN) subtiles of the smaller shape S: a partial round of large
// tiles becomes one round of small ones, spread over every CU. The subtiles
// of one tile are consecutive on one XCD. The arithmetic per output is the
// same as in the large tile (bit-identical).
template <class G, class S>
__global__ __launch_bounds__(S::kThreads, 1) void grouped_tail_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
    int E, int M_total, int N, int K, int tail_cus, int tail_max) {
  static_assert(G::BM % S::BM == 0 && G::BN % S::BN == 0, "subtiles must divide the tile");
  constexpr int kSubM = G::BM / S::BM, kSubN = G::BN / S::BN, kSubs = kSubM * kSubN;
  __shared__ __align__(16) uint8_t smem[S::kLdsBytes];
  const int tiles_n = (N + G::BN - 1) / G::BN;
  const int all = total_units(offsets, E, M_total, G::BM, tiles_n, 0);
  const int rem = grouped_tail_tiles(all, tail_cus, tail_max);
  if ((int)blockIdx.x >= rem * kSubs) return;
  const int sid = xcd_remap(blockIdx.x, rem * kSubs);
  const int tile = all - rem + sid / kSubs, sub = sid % kSubs;
  const ExpertSlot es = locate_expert(offsets, E, M_total, tile, G::BM, tiles_n, 0);
  if (es.e < 0) return;
  int tm, tn;
  tile_coords(tile - es.base, (es.r1 - es.r0 + G::BM - 1) / G::BM, tiles_n, tm, tn);
  const int m0 = es.r0 + tm * G::BM + (sub / kSubN) * S::BM;
  const int n0 = tn * G::BN + (sub % kSubN) * S::BN;
  if (m0 >= es.r1 || n0 >= N) return;     // a subtile past the expert's rows or the last columns
  const int64_t nkb = K / BK;
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M_total;
  t.B = B + (int64_t)es.e * N * K;
  t.sB = sB + (int64_t)es.e * (N / BK) * nkb;
  t.C = C; t.Q = nullptr; t.sQ = nullptr; t.QT = nullptr; t.sQT = nullptr;
  t.m0 = m0; t.row_end = es.r1;
  t.n0 = n0; t.N = N; t.K = K; t.ld = K;
  run_tile<S, 0>(t, smem);
}

// The last gridDim.x / subtiles-per-tile tiles of gemm_kernel<G>'s numbering,
// from tile `first` on (that kernel's grid then covers only the tiles before
// it), each computed as (G::BM / S::BM) x (G::BN / S::BN) subtiles of the
// smaller shape S, spread over every CU. The subtiles of one tile are
// consecutive on one XCD; the arithmetic per output is the large tile's.
template <class G, class S, int ROW_MODE>
__global__ __launch_bounds__(S::kThreads, 1) void dense_tail_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, int M, int N, int K, int first) {
  static_assert(G::BM % S::BM == 0 && G::BN % S::BN == 0, "subtiles must divide the tile");
  constexpr int kSubN = G::BN / S::BN, kSubs = (G::BM / S::BM) * kSubN;
  __shared__ __align__(16) uint8_t smem[S::kLdsBytes];
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_n = (N + G::BN - 1) / G::BN;
  const int sid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = first + sid / kSubs, sub = sid % kSubs;
  int tm, tn;
  tile_coords(tile, tiles_m, tiles_n, tm, tn, kGroupMDense);
  const int m0 = tm * G::BM + (sub / kSubN) * S::BM;
  const int n0 = tn * G::BN + (sub % kSubN) * S::BN;
  if (m0 >= M || n0 >= N) return;     // a subtile past the last rows or columns
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M;
  t.B = B; t.sB = sB; t.C = C; t.Q = nullptr; t.sQ = nullptr; t.QT = nullptr; t.sQT = nullptr;
  t.m0 = m0; t.row_end = M;
  t.n0 = n0; t.N = N; t.K = K; t.ld = K;
  run_tile<S, ROW_MODE>(t, smem);
}

// Per-expert Wgrad: C[e] = A_e B_e^T over expert e's tokens, row-mode scales.
// A[N][ld] and B[K][ld] are the 128x1 transposed codes of the two operands
// with every expert's tokens padded to whole 128-token groups: expert e's
// groups are g = P_e .. P_e + ceil(rows_e / 128) - 1 with P_e the groups of
// the experts before it, its tokens sit at columns 128 P_e .., and the scales
// of group g are sA[g][*], sB[g][*]. Every expert has the same
// ceil(N/BM) x ceil(K/BN) tiles; an expert without tokens gets zeros.
//
// A tile's cost is proportional to its expert's tokens, which vary widely, so
// every expert's tiles are split evenly over the XCDs (workgroup b runs on XCD
// b % 8): XCD x takes the x-th contiguous run of ceil(tiles / 8) tile indices
// of each expert in turn (in the grouped tile order that run is a compact
// block of m- and n-tiles, whose operand panels stay in that XCD's L2).
template <class G>
__global__ __launch_bounds__(G::kThreads, 1) void grouped_wgrad_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
    int M_total, int N, int K, int ld) {
  __shared__ __align__(16) uint8_t smem[G::kLdsBytes];
  const int tiles_m = (N + G::BM - 1) / G::BM, tiles_n = (K + G::BN - 1) / G::BN;
  const int per_expert = tiles_m * tiles_n;
  const int run = (per_expert + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int e = local / run;
  const int idx = xcd * run + local % run;
  if (idx >= per_expert) return;   // the last run of an expert may be short
  int tm, tn;
  tile_coords(idx, tiles_m, tiles_n, tm, tn);
  const ExpertSlot es = units_before(offsets, M_total, e, BK);
  // (with offsets that break the precondition, stay inside the ld / 128 groups)
  const int groups = max(0, min((es.r1 - es.r0 + BK - 1) / BK, ld / BK - es.base));
  uint16_t* Ce = C + (int64_t)e * N * K;
  if (groups == 0) {
    // no tokens: a zero tile (whole 8-byte pieces; K % 128 == 0)
    for (int p = threadIdx.x; p < G::BM * G::BN / 4; p += G::kThreads) {
      const int m = tm * G::BM + p / (G::BN / 4), n = tn * G::BN + 4 * (p % (G::BN / 4));
      if (m < N && n < K) *reinterpret_cast<uint2*>(Ce + (int64_t)m * K + n) = make_uint2(0u, 0u);
    }
    return;
  }
  Tile t;
  t.A = A + (int64_t)es.base * BK; t.sA = sA + (int64_t)es.base * N; t.sa_stride = N;
  t.B = B + (int64_t)es.base * BK; t.sB = sB + (int64_t)es.base * K;
  t.C = Ce; t.Q = nullptr; t.sQ = nullptr; t.QT = nullptr; t.sQT = nullptr;
  t.m0 = tm * G::BM; t.row_end = N;
  t.n0 = tn * G::BN; t.N = K; t.K = groups * BK; t.ld = ld;
  run_tile<G, 1>(t, smem);
}

// Compute units of the device the work runs on (the stream's device; the
// current device for the null stream), looked up once per device. MI355X
// has 256; that is also the answer when the query fails.
int device_cus(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Dense tile shapes, in the order pick_dense numbers them, with the estimate
// it compares (MI355X, K = 7168; measured): a tile takes at least `lat` us
// even alone on its CU, a CU kept busy with such tiles produces at most
// `thr` output elements per us (smaller tiles share a CU between workgroups
// but re-read their operands more often), and each round of tiles adds about
// 4 us (its first loads and its epilogue), where a round is `per_cu` tiles:
// as many workgroups as fit on a CU together (LDS and registers).
struct TileEst {
  int bm, bn, depth, per_cu;
  double lat, thr;
};
enum DenseTile {
  kT256x256, kT256x224, kT224x256, kT128x256, kT128x128, kT64x64, kT128x128d4, kT64x64d3, kT64x64d4, kDenseTiles
};
constexpr TileEst kTileEst[kDenseTiles] = {
    {256, 256, 2, 1, 80.0, 650.0}, {256, 224, 3, 1, 70.0, 637.0}, {224, 256, 3, 1, 70.0, 637.0},
    {128, 256, 2, 1, 54.0, 536.0}, {128, 128, 2, 2, 43.0, 531.0}, {64, 64, 2, 4, 33.0, 333.0},
    {128, 128, 4, 1, 30.0, 512.0}, {64, 64, 3, 3, 23.0, 322.0},    {64, 64, 4, 2, 22.0, 330.0}};
template <class G>
constexpr bool est_matches(DenseTile t) {
  return kTileEst[t].bm == G::BM && kTileEst[t].bn == G::BN && kTileEst[t].depth == (G::DA > G::DB ? G::DA : G::DB);
}
static_assert(est_matches<Cfg256x256>(kT256x256) && est_matches<Cfg256x224>(kT256x224) &&
                  est_matches<Cfg224x256>(kT224x256) && est_matches<Cfg128x256>(kT128x256) &&
                  est_matches<Cfg128x128>(kT128x128) && est_matches<Cfg64x64>(kT64x64) &&
                  est_matches<Cfg128x128d4>(kT128x128d4) && est_matches<Cfg64x64d3>(kT64x64d3) &&
                  est_matches<Cfg64x64d4>(kT64x64d4),
              "the estimate table follows the tile configurations");

static_assert(est_matches<TailCfg>(kT64x64d3), "the tail subtiles are the three-deep 64x64 kernel");
// Cfg128x128q2 (measured with the two-layout epilogue)
constexpr TileEst kQ2Small = {128, 128, 4, 1, 40.0, 380.0};
static_assert(kQ2Small.bm == Cfg128x128q2::BM && kQ2Small.bn == Cfg128x128q2::BN, "estimate of Cfg128x128q2");

// Estimated time (us) of `tiles` tiles of kernel c on `cus` CUs, K = k * 7168.
double tile_estimate(const TileEst& c, int64_t tiles, int cus, double k) {
  const int64_t per_cu = (tiles + cus - 1) / cus;
  const int64_t rounds = (per_cu + c.per_cu - 1) / c.per_cu;
  return std::max(c.lat * k, (double)per_cu * c.bm * c.bn / c.thr * k) + 4.0 * (double)rounds;
}

// The dense GEMM's choice: a kernel of kTileEst and, with 256x256 tiles, how
// many of its last tiles a second launch computes as TailCfg subtiles.
struct DensePick {
  int tile;
  int tail;
};

DensePick pick_dense(int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int cus = device_cus(stream);
  const double k = (double)K / 7168.0;
  int best = 0;
  double best_t = 0.0;
  for (int i = 0; i < kDenseTiles; ++i) {
    // the three-deep 64x64 kernel only computes tails (for a whole problem the
    // four-deep 128x128 kernel beats it wherever it holds three tiles per CU)
    if (i == kT64x64d3) continue;
    const TileEst& c = kTileEst[i];
    const double t = tile_estimate(c, ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn), cus, k);
    if (i == 0 || t < best_t) {
      best = i;
      best_t = t;
    }
  }
  // 256x256 tiles in whole rounds, and a last partial round that one round of
  // subtiles holds (kTailPerCu per CU) as subtiles over every CU, launched
  // behind them (about 2 us between the launches)
  constexpr int subs = (Cfg256x256::BM / TailCfg::BM) * (Cfg256x256::BN / TailCfg::BN);
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t tail = tiles % cus, full = tiles - tail;
  if (full > 0 && tail > 0 && tail * subs <= (int64_t)cus * kTailPerCu) {
    const double t = tile_estimate(kTileEst[kT256x256], full, cus, k) +
                     tile_estimate(kTileEst[kT64x64d3], tail * subs, cus, k) + 2.0;
    if (t < best_t) return {kT256x256, (int)tail};
  }
  return {best, 0};
}

template <class G, int QOUT, int HW = 0>
hipError_t launch_dense(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                        int row_mode, uint16_t* C, uint8_t* Q, float* sQ, int64_t M, int64_t N,
                        int64_t K, hipStream_t stream, uint8_t* QT = nullptr, float* sQT = nullptr) {
  const int tiles = (int)(((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN));
  if (row_mode)
    hipLaunchKernelGGL((gemm_kernel<G, 1, QOUT, HW>), dim3(tiles), dim3(G::kThreads), 0, stream, A, sA, B, sB,
                       C, Q, sQ, QT, sQT, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL((gemm_kernel<G, 0, QOUT, HW>), dim3(tiles), dim3(G::kThreads), 0, stream, A, sA, B, sB,
                       C, Q, sQ, QT, sQT, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

// gemm_kernel<G> over all but the last `tail` tiles, then dense_tail_kernel
// over those (BF16 output).
template <class G, class S>
hipError_t launch_dense_tail(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB, int row_mode,
                             uint16_t* C, int64_t M, int64_t N, int64_t K, int tail, hipStream_t stream) {
  constexpr int subs = (G::BM / S::BM) * (G::BN / S::BN);
  const int tiles = (int)(((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN));
  const int full = tiles - tail;
  auto go = [&](auto rm) {
    constexpr int R = decltype(rm)::value;
    hipLaunchKernelGGL((gemm_kernel<G, R, 0, 0>), dim3(full), dim3(G::kThreads), 0, stream, A, sA, B, sB, C, nullptr,
                       nullptr, nullptr, nullptr, (int)M, (int)N, (int)K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_tail_kernel<G, S, R>), dim3(tail * subs), dim3(S::kThreads), 0, stream, A, sA, B, sB,
                       C, (int)M, (int)N, (int)K, full);
    return hipGetLastError();
  };
  return row_mode ? go(std::integral_constant<int, 1>{}) : go(std::integral_constant<int, 0>{});
}

// ---------------------------------------------------------------------------
// Decode-shaped grouped GEMM (few activation rows per expert, so the weights
// are the stream). One workgroup per (expert, 128 weight rows) covers all of
// the expert's rows, up to 256 per pass, so every weight byte is read once
// (experts with more rows take further passes). Each of the 8 waves streams
// its own 16 weight rows from HBM straight into MFMA operand registers, kDB
// chunks ahead of use. The activation chunk (the pass's rows x 128 bytes and
// their sA) goes through registers into a double-buffered, swizzled LDS tile
// shared by the waves, one chunk ahead, with one barrier per chunk. Every load
// is an ordinary vector load, so the compiler's own waits stay exact; the
// barrier waits for LDS only and leaves the weight loads in flight. A pass
// computes NSUB activation subtiles of 16 rows (its rows rounded up to 16),
// compiled once per NSUB so no subtile branches sit in the chunk loop. The
// operands are swapped as in the tile kernel: lane l holds
// C[m = 16i + l%16][n .. n+3].
// ---------------------------------------------------------------------------
namespace dec {
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kBM = 256;                     // activation rows per pass
constexpr int kBN = 16 * kWaves;             // weight rows per workgroup, 16 per wave
constexpr int kDB = 4;                       // weight chunks loaded ahead of the one in use
constexpr int kR = kDB + 1;                  // weight register ring
constexpr int kOrderMax = 256;               // experts ranked by size in each workgroup, at most
constexpr int kASlot = kBM * BK + kBM * 4;   // codes, then the chunk's sA vector
constexpr int kPitch = kBN * 2 + 16;         // epilogue tile row pitch (bytes)
constexpr int kLds = (2 * kASlot > kBM * kPitch) ? 2 * kASlot : kBM * kPitch;
static_assert((kOrderMax + 1) * 4 <= kLds, "expert counts fit the LDS");

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct Pass {
  const uint8_t* A;     // activation codes [M_total][K]
  const float* sA;      // [K/128][M_total]
  uint16_t* C;          // [M_total][N]
  const uint8_t* brow;  // this lane's first weight row (+ its 16-byte piece offset), see b_load
  const uint8_t* brow8; // the same, 8 rows further
  const float* sbp;     // sB of this wave's 128-row scale block, one value per chunk
  int M_total, N, K, nkb, m0, rows, n_col0;
};

template <int NSUB>
__device__ __forceinline__ void run_pass(const Pass a, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nkb = a.nkb, rows = a.rows;

  // Activation staging: thread t loads 16-byte piece t%8 of rows t/8 + 64q for
  // the kQ rounds that cover the pass's NSUB*16 rows (rows past those in the
  // last round are skipped; rows past the expert's end are clamped, and their
  // results never stored). Named registers written out per round: an array
  // indexed in a loop was left in scratch.
  constexpr int kRowsP = NSUB * 16, kRR = kThreads / 8, kQ = (kRowsP + kRR - 1) / kRR;
  static_assert(kQ <= 4 && kRowsP <= kThreads, "staging rounds; one sA value per thread");
  const int ar = tid >> 3, ap = tid & 7;
  uint4 ast0, ast1, ast2, ast3;
  float sst = 0.0f;
  const uint8_t* abase = a.A + (int64_t)a.m0 * a.K + 16 * ap;
  const float* srow = a.sA + a.m0 + min(tid, rows - 1);
#define FP8BS_DEC_LD(q)                                                                              \
  if constexpr (kQ > q) {                                                                            \
    if (q + 1 < kQ || ar + kRR * q < kRowsP)                                                         \
      ast##q = *reinterpret_cast<const uint4*>(abase + o + (int64_t)min(ar + kRR * q, rows - 1) * a.K); \
  }
#define FP8BS_DEC_ST(q)                                                                              \
  if constexpr (kQ > q) {                                                                            \
    const int r = ar + kRR * q;                                                                      \
    if (q + 1 < kQ || r < kRowsP) *reinterpret_cast<uint4*>(base + r * BK + ((ap ^ swz(r)) << 4)) = ast##q; \
  }
  auto a_load = [&](int kb) {
    const int64_t o = (int64_t)kb * BK;
    FP8BS_DEC_LD(0) FP8BS_DEC_LD(1) FP8BS_DEC_LD(2) FP8BS_DEC_LD(3)
    if (tid < kRowsP) sst = srow[(int64_t)kb * a.M_total];
  };
  auto a_store = [&](int slot) {
    uint8_t* base = smem + slot * kASlot;
    FP8BS_DEC_ST(0) FP8BS_DEC_ST(1) FP8BS_DEC_ST(2) FP8BS_DEC_ST(3)
    if (tid < kRowsP) reinterpret_cast<float*>(base + kBM * BK)[tid] = sst;
  };
#undef FP8BS_DEC_LD
#undef FP8BS_DEC_ST

  // weight ring: chunk c in registers bq[c % kR], its block scale in sbq.
  // The wave's 16 weight rows of a chunk are fetched as two loads of 8 whole
  // 128-byte rows each: lane l = 16g + 8h + r (r < 8) loads 16-byte piece
  // 2g + h of row r (bq[0..3]) and of row 8 + r (bq[4..7]). The MFMA operand
  // wants row l%16 with pieces 2g and 2g+1, so lanes l and l^8 trade halves
  // (frag_of). Loading the operand layout directly, each load touched 16
  // rows for 64 bytes of each; with whole rows the address unit's stalls on
  // the vector L1 fell by 12% and the decode shape ran about 1% faster.
  v8i bq[kR];
  float sbq[kR];
  auto b_load = [&](int c, int u) {
    const int cc = min(c, nkb - 1);
    const uint4 pa = *reinterpret_cast<const uint4*>(a.brow + (int64_t)cc * BK);
    const uint4 pb = *reinterpret_cast<const uint4*>(a.brow8 + (int64_t)cc * BK);
    bq[u] = v8i{(int)pa.x, (int)pa.y, (int)pa.z, (int)pa.w, (int)pb.x, (int)pb.y, (int)pb.z, (int)pb.w};
    sbq[u] = a.sbp[cc];
  };
  const bool low8 = (lane & 8) == 0;
  auto frag_of = [&](const v8i& raw) {
    v8i f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // row_ror 8: the value of lane l^8 (within its 16-lane row)
      const int xa = __builtin_amdgcn_mov_dpp(raw[k], 0x128, 0xF, 0xF, false);
      const int xb = __builtin_amdgcn_mov_dpp(raw[4 + k], 0x128, 0xF, 0xF, false);
      f[k] = low8 ? raw[k] : xb;
      f[4 + k] = low8 ? xa : raw[4 + k];
    }
    return f;
  };
  v4f acc[NSUB];
#pragma unroll
  for (int i = 0; i < NSUB; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // prologue: weights 0 .. kDB-1, activations 0 (in LDS) and 1 (staged)
#pragma unroll
  for (int u = 0; u < kDB; ++u) b_load(u, u);
  a_load(0);
  a_store(0);
  a_load(min(1, nkb - 1));
  lds_barrier();

  // Chunk kb with its weights in ring slot u: fragment i+1 is read while MFMA
  // i runs, and MFMA i's partial is promoted one subtile later. Each promoted
  // accumulator is pinned where it is computed (otherwise the compiler sinks
  // the promotions to the accumulators' next use and keeps every partial).
  auto chunk = [&](int kb, int u) {
    b_load(kb + kDB, (u + kDB) % kR);
    const uint8_t* slot = smem + (kb & 1) * kASlot;
    const float* sAs = reinterpret_cast<const float*>(slot + kBM * BK) + (lane & 15);
    const v8i bf = frag_of(bq[u]);
    v8i af = read_frag(slot, 0, lane);
    v4f pp = v4f{0.f, 0.f, 0.f, 0.f};
    float fp = 0.0f;
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const v8i a_now = af;
      if (i + 1 < NSUB) af = read_frag(slot, i + 1, lane);
      const float f_now = sAs[16 * i] * sbq[u];
      const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, a_now, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                       0, 0, 0, 0);
      if (i > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i - 1][r] = fmaf(pp[r], fp, acc[i - 1][r]);
        asm volatile("" : "+v"(acc[i - 1]));
      }
      pp = pc;
      fp = f_now;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[NSUB - 1][r] = fmaf(pp[r], fp, acc[NSUB - 1][r]);
    asm volatile("" : "+v"(acc[NSUB - 1]));
    if (kb + 1 < nkb) {   // activations kb+1 into the other slot, then the loads of kb+2
      a_store((kb + 1) & 1);
      a_load(min(kb + 2, nkb - 1));
    }
    lds_barrier();
  };
  int kb = 0;
  for (; kb + kR <= nkb; kb += kR) {
#pragma unroll
    for (int u = 0; u < kR; ++u) chunk(kb + u, u);
  }
#pragma unroll
  for (int u = 0; u < kR; ++u)
    if (kb + u < nkb) chunk(kb + u, u);

  // epilogue through LDS: row-major BF16 tile [NSUB*16][kBN], whole rows out
#pragma unroll
  for (int i = 0; i < NSUB; ++i) {
    uint2 o;
    o.x = float_to_bf16_bits(acc[i][0]) | (float_to_bf16_bits(acc[i][1]) << 16);
    o.y = float_to_bf16_bits(acc[i][2]) | (float_to_bf16_bits(acc[i][3]) << 16);
    const int r = 16 * i + (lane & 15), c = 16 * wave + 4 * (lane >> 4);
    *reinterpret_cast<uint2*>(smem + r * kPitch + 2 * c) = o;
  }
  lds_barrier();
  constexpr int kPieces = kBN / 8;
  for (int p = tid; p < kRowsP * kPieces; p += kThreads) {
    const int row = p / kPieces, piece = p % kPieces;
    const int n = a.n_col0 + 8 * piece;
    if (row < rows && n < a.N)
      *reinterpret_cast<uint4*>(a.C + (int64_t)(a.m0 + row) * a.N + n) =
          *reinterpret_cast<const uint4*>(smem + row * kPitch + 16 * piece);
  }
  lds_barrier();   // the next pass reuses the LDS
}
}  // namespace dec

// Experts with more than max_rows rows are left to the tile kernel.
__global__ __launch_bounds__(dec::kThreads, 1) void grouped_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, int E,
    int M_total, int N, int K, int max_rows) {
  __shared__ __align__(16) uint8_t smem[dec::kLds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = (N + dec::kBN - 1) / dec::kBN;
  // consecutive ids on one XCD: an expert's weight blocks share that XCD's L2
  // copy of its activations instead of every XCD fetching them
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  const int slot = pid / nblk, nb = pid % nblk;
  auto rows_of = [&](int x, int& lo, int& hi) {
    lo = min(max(offsets[x], 0), M_total);
    hi = min(max(offsets[x + 1], lo), M_total);
  };
  // Expert order: largest, smallest, second largest, second smallest, ... by
  // row count (ties by index), so that workgroups bound by MFMA and LDS work
  // (many rows) run beside workgroups that only stream weights (few rows);
  // launched in index order, or sorted either way, the same experts take 5-10%
  // longer. Each workgroup ranks the experts itself (E <= kOrderMax).
  int e = slot;
  if (E <= dec::kOrderMax) {
    int* cnt = reinterpret_cast<int*>(smem);   // E counts, then the chosen expert
    for (int i = threadIdx.x; i < E; i += dec::kThreads) {
      int lo, hi;
      rows_of(i, lo, hi);
      cnt[i] = hi - lo;
    }
    __syncthreads();
    const int want = (slot & 1) ? E - 1 - (slot >> 1) : (slot >> 1);   // descending rank
    for (int i = threadIdx.x; i < E; i += dec::kThreads) {
      const int ci = cnt[i];
      int rank = 0;
      for (int j = 0; j < E; ++j) rank += (cnt[j] > ci) | ((cnt[j] == ci) & (j < i));
      if (rank == want) cnt[E] = i;
    }
    __syncthreads();
    e = cnt[E];
    __syncthreads();   // the passes reuse the LDS
  }
  int r0, r1;
  rows_of(e, r0, r1);
  if (r1 <= r0 || r1 - r0 > max_rows) return;     // no rows, or the tile kernel's expert
  dec::Pass a;
  a.A = A; a.sA = sA; a.C = C; a.M_total = M_total; a.N = N; a.K = K; a.nkb = K / BK;
  a.n_col0 = nb * dec::kBN;
  const int nw0 = a.n_col0 + 16 * wave;            // this wave's first weight row
  const int piece = 2 * (lane >> 4) + ((lane >> 3) & 1);
  a.brow = B + (int64_t)e * N * K + (int64_t)min(nw0 + (lane & 7), N - 1) * K + 16 * piece;
  a.brow8 = B + (int64_t)e * N * K + (int64_t)min(nw0 + 8 + (lane & 7), N - 1) * K + 16 * piece;
  // the wave's 16 rows lie in one 128-row scale block
  a.sbp = sB + (int64_t)e * (N / BK) * a.nkb + (int64_t)(min(nw0, N - 1) / BK) * a.nkb;
  for (int m0 = r0; m0 < r1; m0 += dec::kBM) {
    a.m0 = m0;
    a.rows = min(dec::kBM, r1 - m0);
    switch ((a.rows + 15) / 16) {
      case 1: dec::run_pass<1>(a, smem); break;
      case 2: dec::run_pass<2>(a, smem); break;
      case 3: dec::run_pass<3>(a, smem); break;
      case 4: dec::run_pass<4>(a, smem); break;
      case 5: dec::run_pass<5>(a, smem); break;
      case 6: dec::run_pass<6>(a, smem); break;
      case 7: dec::run_pass<7>(a, smem); break;
      case 8: dec::run_pass<8>(a, smem); break;
      case 9: dec::run_pass<9>(a, smem); break;
      case 10: dec::run_pass<10>(a, smem); break;
      case 11: dec::run_pass<11>(a, smem); break;
      case 12: dec::run_pass<12>(a, smem); break;
      case 13: dec::run_pass<13>(a, smem); break;
      case 14: dec::run_pass<14>(a, smem); break;
      case 15: dec::run_pass<15>(a, smem); break;
      default: dec::run_pass<16>(a, smem); break;
    }
  }
}

}  // namespace gemm

hipError_t launch_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, int row_mode, uint16_t* C, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream) {
  using namespace gemm;
  const DensePick p = pick_dense(M, N, K, stream);
  if (p.tail > 0)
    return launch_dense_tail<Cfg256x256, TailCfg>(A, sA, B, sB, row_mode, C, M, N, K, p.tail, stream);
  switch (p.tile) {
    case kT256x224: return launch_dense<Cfg256x224, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT224x256: return launch_dense<Cfg224x256, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT128x256: return launch_dense<Cfg128x256, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT128x128: return launch_dense<Cfg128x128, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT64x64: return launch_dense<Cfg64x64, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT128x128d4:
      return launch_dense<Cfg128x128d4, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT64x64d4: return launch_dense<Cfg64x64d4, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    default: return launch_dense<Cfg256x256, 0>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
  }
}

void gemm_blockscaled_tile(int64_t M, int64_t N, int64_t K, int row_mode, int* bm, int* bn, int* depth,
                           int* tail) {
  using namespace gemm;
  (void)row_mode;
  const DensePick p = pick_dense(M, N, K, nullptr);
  *bm = kTileEst[p.tile].bm;
  *bn = kTileEst[p.tile].bn;
  if (depth) *depth = kTileEst[p.tile].depth;
  if (tail) *tail = p.tail;
}

hipError_t launch_gemm_blockscaled_pow2(const uint8_t* A, const float* sA, const uint8_t* B,
                                        const float* sB, int row_mode, uint16_t* C, int64_t M,
                                        int64_t N, int64_t K, hipStream_t stream) {
  using namespace gemm;
  // Large problems: 4 waves of 128x128 with the accumulators in AGPRs, 11%
  // faster than the 8-wave tiles at 4096x7168x7168, on a par or better on
  // the other shapes measured. Problems with few tiles: the four-deep
  // 128x128 or 64x64 kernels, by the dense GEMM's time estimate (the large
  // tile counted as a 256x256 one).
  const int cus = device_cus(stream);
  const double k = (double)K / 7168.0;
  const DenseTile cand[] = {kT256x256, kT128x128d4, kT64x64d4};
  DenseTile best = kT256x256;
  double best_t = 0.0;
  for (const DenseTile c : cand) {
    const TileEst& e = kTileEst[c];
    const double t = tile_estimate(e, ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn), cus, k);
    if (c == kT256x256 || t < best_t) {
      best = c;
      best_t = t;
    }
  }
  switch (best) {
    case kT128x128d4:
      return launch_dense<Cfg128x128d4, 0, 1>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    case kT64x64d4: return launch_dense<Cfg64x64d4, 0, 1>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
    default: return launch_dense<Cfg256x256w4, 0, 1>(A, sA, B, sB, row_mode, C, nullptr, nullptr, M, N, K, stream);
  }
}

hipError_t launch_gemm_blockscaled_q1x128(const uint8_t* A, const float* sA, const uint8_t* B,
                                          const float* sB, int row_mode, uint8_t* Q, float* sQ,
                                          int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  using namespace gemm;
  // tiles whose columns hold whole 128-column groups, by the dense GEMM's
  // time estimate: 256x256, 224x256, and for problems with few tiles
  // 128x256 or 128x128 (four deep)
  const int cus = device_cus(stream);
  const double k = (double)K / 7168.0;
  const DenseTile cand[] = {kT256x256, kT224x256, kT128x256, kT128x128d4};
  DenseTile best = kT256x256;
  double best_t = 0.0;
  for (const DenseTile c : cand) {
    const TileEst& e = kTileEst[c];
    const double t = tile_estimate(e, ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn), cus, k);
    if (c == kT256x256 || t < best_t) {
      best = c;
      best_t = t;
    }
  }
  switch (best) {
    case kT224x256: return launch_dense<Cfg224x256, 1>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream);
    case kT128x256: return launch_dense<Cfg128x256, 1>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream);
    case kT128x128d4:
      return launch_dense<Cfg128x128d4, 1>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream);
    default: return launch_dense<Cfg256x256, 1>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream);
  }
}

hipError_t launch_gemm_blockscaled_q1x128_q128x1T(const uint8_t* A, const float* sA, const uint8_t* B,
                                                  const float* sB, int row_mode, uint8_t* Q, float* sQ,
                                                  uint8_t* QT, float* sQT, int64_t M, int64_t N, int64_t K,
                                                  hipStream_t stream) {
  using namespace gemm;
  // tiles whose waves hold 128 whole rows (one 128x1 group) and whose columns
  // hold whole 128-column groups: 256x256, or for problems with few tiles
  // 128x128 with 8 waves of 128x16, by the dense GEMM's time estimate
  const int cus = device_cus(stream);
  const double k = (double)K / 7168.0;
  const TileEst& big = kTileEst[kT256x256];
  const double t_big = tile_estimate(big, ((M + 255) / 256) * ((N + 255) / 256), cus, k);
  const double t_small = tile_estimate(kQ2Small, ((M + 127) / 128) * ((N + 127) / 128), cus, k);
  if (t_small < t_big)
    return launch_dense<Cfg128x128q2, 2>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream, QT, sQT);
  return launch_dense<Cfg256x256, 2>(A, sA, B, sB, row_mode, nullptr, Q, sQ, M, N, K, stream, QT, sQT);
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                           const float* sB, uint16_t* C, const int32_t* offsets,
                                           int E, int64_t M_total, int64_t N, int64_t K,
                                           hipStream_t stream) {
  using namespace gemm;
  using G = Cfg256x256;
  const int64_t tiles_n = (N + G::BN - 1) / G::BN;
  // More than 256 rows per expert on average: the tile kernel for every
  // expert; every expert adds at most one partial m-tile beyond M_total / BM.
  // (At 256 rows per expert the weight-streaming kernel below is the faster:
  // 384 against 450 us for 32 experts of 256 rows, N 4096, K 7168; routing a
  // MoE batch's few small experts to it, in a launch of its own ahead of the
  // tile kernel, costs more than the tile rounds it saves: 2,041 against
  // 1,966 us for the MoE up projection.)
  if (M_total > (int64_t)E * dec::kBM) {
    // a last round that one round of the tail kernel's subtiles can hold
    // (kTailPerCu of them per CU) goes to the tail kernel; the tail count is
    // only known on the device, and with none the tail launch exits at once
    using S = TailCfg;
    constexpr int subs_per_tile = (G::BM / S::BM) * (G::BN / S::BN);
    const int cus = device_cus(stream);
    const int tail_max = cus * kTailPerCu / subs_per_tile;
    const int64_t tiles = ((M_total + G::BM - 1) / G::BM + E) * tiles_n;
    hipLaunchKernelGGL((grouped_gemm_kernel<G>), dim3((unsigned)tiles), dim3(G::kThreads), 0, stream, A, sA, B,
                       sB, C, offsets, E, (int)M_total, (int)N, (int)K, 0, cus, tail_max);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess || tail_max == 0) return e0;
    hipLaunchKernelGGL((grouped_tail_kernel<G, S>), dim3((unsigned)(tail_max * subs_per_tile)), dim3(S::kThreads), 0,
                       stream, A, sA, B, sB, C, offsets, E, (int)M_total, (int)N, (int)K, cus, tail_max);
    return hipGetLastError();
  }
  // Few rows per expert on average (decode): the weight-streaming kernel for
  // experts of at most one 256-row pass, which reads their weights once
  // whatever their rows; the offsets live on the device, so any expert with
  // more rows (a skewed batch) is left to the tile kernel, launched behind it
  // for those experts only: at most M_total / 257 of them, adding at most
  // one partial m-tile each.
  const int64_t blocks = (int64_t)E * ((N + dec::kBN - 1) / dec::kBN);
  hipLaunchKernelGGL(grouped_decode_kernel, dim3((unsigned)blocks), dim3(dec::kThreads), 0, stream, A, sA, B, sB,
                     C, offsets, E, (int)M_total, (int)N, (int)K, dec::kBM);
  const int64_t big = M_total / (dec::kBM + 1);
  if (big == 0) return hipGetLastError();
  const hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess) return e1;
  const int64_t tiles = ((M_total + G::BM - 1) / G::BM + big) * tiles_n;
  hipLaunchKernelGGL((grouped_gemm_kernel<G>), dim3((unsigned)tiles), dim3(G::kThreads), 0, stream, A, sA, B, sB,
                     C, offsets, E, (int)M_total, (int)N, (int)K, dec::kBM, 0, 0);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_wgrad(const uint8_t* A, const float* sA, const uint8_t* B,
                                     const float* sB, uint16_t* C, const int32_t* offsets, int E,
                                     int64_t M_total, int64_t N, int64_t K, int64_t ld,
                                     hipStream_t stream) {
  using namespace gemm;
  using G = Cfg256x256;
  const int64_t per_expert = ((N + G::BM - 1) / G::BM) * ((K + G::BN - 1) / G::BN);
  const int64_t tiles = (int64_t)E * kXcds * ((per_expert + kXcds - 1) / kXcds);
  hipLaunchKernelGGL((grouped_wgrad_kernel<G>), dim3((unsigned)tiles), dim3(G::kThreads), 0, stream, A, sA, B,
                     sB, C, offsets, (int)M_total, (int)N, (int)K, (int)ld);
  return hipGetLastError();
}

}  // namespace fp8bs
