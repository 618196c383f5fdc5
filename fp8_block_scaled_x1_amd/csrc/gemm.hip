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
// Structure (one BM x BN output tile per workgroup of 8 waves):
//   * one pipeline stage = one K chunk: A[BM][128] + B[BN][128] bytes plus the
//     chunk's scale vectors, moved L2 -> LDS with direct-to-LDS loads (no VGPR
//     staging); two stages; one barrier per chunk;
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
//   * the tile shape is chosen on the host per problem so that the number of
//     tiles fills whole rounds of the 256 CUs where possible.

#include "device_common.h"
#include "internal.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace gemm {

constexpr int BK = kGroup;
constexpr int kThreads = 512;        // 8 waves
constexpr int kGroupM = 8;           // tile-order grouping for L2 reuse
constexpr int kXcds = 8;

template <int BM_, int BN_, int WGM_, int WGN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int WM = BM / WGM, WN = BN / WGN;          // wave subtile
  static constexpr int MS = WM / 16, NS = WN / 16;            // MFMA tiles per wave
  static constexpr int kABytes = BM * BK, kBBytes = BN * BK;
  static constexpr int kScaleOfs = kABytes + kBBytes;         // then sA[BM], sB[BN] floats
  static constexpr int kStageBytes = kScaleOfs + (BM + BN) * 4;
  static constexpr int kSlices = (BM + BN) / 8;               // 1 KB load slices per stage
  static constexpr int kSlicesPerWave = (kSlices + 7) / 8;
  static constexpr bool kHoldB = NS <= MS;                    // hold the smaller operand
  static_assert(WGM * WGN == 8, "8 waves");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BM % 8 == 0 && BN % 8 == 0, "tile shape");
  static_assert(2 * kStageBytes <= 160 * 1024, "LDS");
};

// 256x256, waves 2x4 of 128x64; 256x224, waves 4x2 of 64x112; 224x256, waves 2x4 of 112x64
using Cfg256x256 = Cfg<256, 256, 2, 4>;
using Cfg256x224 = Cfg<256, 224, 4, 2>;
using Cfg224x256 = Cfg<224, 256, 2, 4>;

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct HBM/L2 -> LDS load of 16 (or 4) bytes per lane: lane i writes LDS
// bytes lds_addr + i*16 (i*4) from global address base + voff. Written as asm
// rather than the compiler builtin because the compiler cannot tell the two
// pipeline stages apart and would otherwise wait for the next stage's loads
// before every read of the current one. The caller waits (s_waitcnt + barrier)
// before reading what these loads wrote. M0 is saved and restored around the
// load; the asm has no VGPR outputs.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
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

// Grouped tile order: kGroupM m-tiles by all n-tiles, column-major inside a group.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = kGroupM * tiles_n;
  const int g = pid / group;
  const int first = g * kGroupM;
  const int gm = min(tiles_m - first, kGroupM);
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
  uint16_t* C;        // [rows][N]
  int m0, row_end;    // tile rows m0 .. m0+BM-1, valid below row_end
  int n0, N, K;
};

template <class G, int ROW_MODE>
__device__ __forceinline__ void run_tile(const Tile& t, uint8_t* stage0, uint8_t* stage1) {
  constexpr int MS = G::MS, NS = G::NS, WM = G::WM, WN = G::WN;
  constexpr int SLA = G::BM / 8;                         // A slices come first
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  const int nkb = t.K / BK;
  const int a_last = t.row_end - 1;
  const int b_last = t.N - 1;

  // Direct-to-LDS operand loads. Slice s (1 KB) covers tile rows 8s .. 8s+7 of
  // A (s < BM/8) or of B; this wave loads slices wave, wave+8, ... Lane p
  // fetches row 8s + p/8, logical 16-byte column (p%8) ^ swz(row), and writes
  // physical column p%8. Offsets are 32-bit from a uniform base (M*K,
  // N*K < 2^31); rows past the end are clamped (their results are never stored).
  uint32_t offs[G::kSlicesPerWave];
#pragma unroll
  for (int j = 0; j < G::kSlicesPerWave; ++j) {
    const int s = wave + 8 * j;
    const bool isA = s < SLA;
    const int rr = (isA ? s : s - SLA) * 8 + (lane >> 3);
    const uint32_t col = (uint32_t)(((lane & 7) ^ swz(rr)) << 4);
    const int row = isA ? min(t.m0 + rr, a_last) : min(t.n0 + rr, b_last);
    offs[j] = (uint32_t)row * (uint32_t)t.K + col;
  }
  // Scale vectors: sA[kb][m0 .. m0+BM-1] by wave 0 and, in row mode,
  // sB[kb][n0 .. n0+BN-1] by wave 1, 64 floats per 4-byte load, clamped.
  uint32_t soff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    soff[j] = 4u * (uint32_t)(wave == 0 ? min(t.m0 + 64 * j + lane, a_last) : min(t.n0 + 64 * j + lane, b_last));

  auto issue_stage = [&](int kb, uint32_t st) {
    const uint8_t* Ak = t.A + (int64_t)kb * BK;
    const uint8_t* Bk = t.B + (int64_t)kb * BK;
#pragma unroll
    for (int j = 0; j < G::kSlicesPerWave; ++j) {
      const int s = wave + 8 * j;
      if (s < G::kSlices) lds_dma16(s < SLA ? Ak : Bk, offs[j], st + (uint32_t)s * 1024u);
    }
    if (wave == 0) {
      const float* sk = t.sA + (int64_t)kb * t.sa_stride;
#pragma unroll
      for (int j = 0; j < (G::BM + 63) / 64; ++j)
        if (64 * j + lane < G::BM) lds_dma4(sk, soff[j], st + (uint32_t)G::kScaleOfs + j * 256u);
    } else if (ROW_MODE && wave == 1) {
      const float* sk = t.sB + (int64_t)kb * t.N;
#pragma unroll
      for (int j = 0; j < (G::BN + 63) / 64; ++j)
        if (64 * j + lane < G::BN)
          lds_dma4(sk, soff[j], st + (uint32_t)(G::kScaleOfs + G::BM * 4) + j * 256u);
    }
  };

  v4f acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // block mode: B scale of n-subtile j is sB[(n of the subtile)/128][kb], uniform
  const float* sbb_ptr[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    sbb_ptr[j] = t.sB + (int64_t)(min(t.n0 + wn * WN + 16 * j, b_last) / BK) * nkb;

  // One chunk: wait for its stage, start the next stage's loads into the other
  // buffer, then compute.
  auto chunk = [&](int kb, const uint8_t* st, uint32_t other) {
    __builtin_amdgcn_s_waitcnt(0);      // this wave's direct-to-LDS loads landed
    __syncthreads();                    // everyone's landed; everyone finished the other stage
    if (kb + 1 < nkb) issue_stage(kb + 1, other);
    const uint8_t* As = st;
    const uint8_t* Bs = st + G::kABytes;
    const float* sAs = reinterpret_cast<const float*>(st + G::kScaleOfs) + wm * WM + (lane & 15);
    const float* sBs = reinterpret_cast<const float*>(st + G::kScaleOfs + G::BM * 4) + wn * WN + 4 * (lane >> 4);

    float sbb[NS];
    float sbr[NS][4];
    if constexpr (ROW_MODE) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(sBs + 16 * j);
        sbr[j][0] = v.x; sbr[j][1] = v.y; sbr[j][2] = v.z; sbr[j][3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) sbb[j] = sbb_ptr[j][kb];
    }

    // promotion of MFMA tile (i, j): scaled FP32 partial into the FP32 accumulator
    auto promote = [&](int i, int j, const v4f& p, float sa) {
      if constexpr (ROW_MODE) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r] * sbr[j][r], sa, acc[i][j][r]);
      } else {
        const float sc = sa * sbb[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r], sc, acc[i][j][r]);
      }
    };

    if constexpr (G::kHoldB) {
      // hold the NS B fragments, stream the MS A subtiles
      v8i bf[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) bf[j] = read_frag(Bs, wn * NS + j, lane);
      v4f p_prev[NS];
      float sa_prev = 0.f;
      v8i af = read_frag(As, wm * MS, lane);
#pragma unroll
      for (int i = 0; i <= MS; ++i) {
        v4f p_cur[NS];
        float sa_cur = 0.f;
        if (i < MS) {
          const v8i a_now = af;
          if (i + 1 < MS) af = read_frag(As, wm * MS + i + 1, lane);
          sa_cur = sAs[16 * i];
#pragma unroll
          for (int j = 0; j < NS; ++j)
            p_cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], a_now, v4f{0.f, 0.f, 0.f, 0.f},
                                                                        0, 0, 0, 0, 0, 0);
        }
        if (i > 0) {
#pragma unroll
          for (int j = 0; j < NS; ++j) promote(i - 1, j, p_prev[j], sa_prev);
        }
        if (i < MS) {
#pragma unroll
          for (int j = 0; j < NS; ++j) p_prev[j] = p_cur[j];
          sa_prev = sa_cur;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // hold the MS A fragments (and their scales), stream the NS B subtiles
      v8i af[MS];
      float sa[MS];
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        af[i] = read_frag(As, wm * MS + i, lane);
        sa[i] = sAs[16 * i];
      }
      v4f p_prev[MS];
      v8i bf = read_frag(Bs, wn * NS, lane);
#pragma unroll
      for (int j = 0; j <= NS; ++j) {
        v4f p_cur[MS];
        if (j < NS) {
          const v8i b_now = bf;
          if (j + 1 < NS) bf = read_frag(Bs, wn * NS + j + 1, lane);
#pragma unroll
          for (int i = 0; i < MS; ++i)
            p_cur[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_now, af[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                        0, 0, 0, 0, 0, 0);
        }
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < MS; ++i) promote(i, j - 1, p_prev[i], sa[i]);
        }
        if (j < NS) {
#pragma unroll
          for (int i = 0; i < MS; ++i) p_prev[i] = p_cur[i];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const uint32_t lds0 = lds_addr_of(stage0), lds1 = lds_addr_of(stage1);
  issue_stage(0, lds0);
  for (int kb = 0; kb < nkb; kb += 2) {
    chunk(kb, stage0, lds1);
    if (kb + 1 < nkb) chunk(kb + 1, stage1, lds0);
  }

  // BF16 epilogue, round to nearest even: lane holds C[m][n..n+3]
  const int m_lane = t.m0 + wm * WM + (lane & 15);
  const int n_lane = t.n0 + wn * WN + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int m = m_lane + 16 * i;
    if (m >= t.row_end) continue;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int n = n_lane + 16 * j;
      if (n >= t.N) continue;
      uint2 o;
      o.x = float_to_bf16_bits(acc[i][j][0]) | (float_to_bf16_bits(acc[i][j][1]) << 16);
      o.y = float_to_bf16_bits(acc[i][j][2]) | (float_to_bf16_bits(acc[i][j][3]) << 16);
      *reinterpret_cast<uint2*>(t.C + (int64_t)m * t.N + n) = o;
    }
  }
}

template <class G, int ROW_MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const uint8_t* __restrict__ A,
                                                            const float* __restrict__ sA,
                                                            const uint8_t* __restrict__ B,
                                                            const float* __restrict__ sB,
                                                            uint16_t* __restrict__ C, int M, int N,
                                                            int K) {
  __shared__ __align__(16) uint8_t stage0[G::kStageBytes];
  __shared__ __align__(16) uint8_t stage1[G::kStageBytes];
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_n = (N + G::BN - 1) / G::BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_coords(pid, tiles_m, tiles_n, tm, tn);
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M;
  t.B = B; t.sB = sB; t.C = C;
  t.m0 = tm * G::BM; t.row_end = M;
  t.n0 = tn * G::BN; t.N = N; t.K = K;
  run_tile<G, ROW_MODE>(t, stage0, stage1);
}

// Per-expert tiles: expert e owns rows [off[e], off[e+1]); its tiles are
// ceil(rows/BM) x ceil(N/BN), numbered expert-major. The grid is an upper
// bound on the total; workgroups past the last tile exit at once.
template <class G>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
    int E, int M_total, int N, int K) {
  __shared__ __align__(16) uint8_t stage0[G::kStageBytes];
  __shared__ __align__(16) uint8_t stage1[G::kStageBytes];
  const int tiles_n = (N + G::BN - 1) / G::BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  int base = 0, e_found = -1, r0 = 0, r1 = 0;
  for (int e = 0; e < E; ++e) {
    const int a = min(max(offsets[e], 0), M_total);
    const int b = min(max(offsets[e + 1], a), M_total);
    const int te = ((b - a + G::BM - 1) / G::BM) * tiles_n;
    if (pid < base + te) {
      e_found = e; r0 = a; r1 = b;
      break;
    }
    base += te;
  }
  if (e_found < 0) return;
  int tm, tn;
  tile_coords(pid - base, (r1 - r0 + G::BM - 1) / G::BM, tiles_n, tm, tn);
  const int64_t nkb = K / BK;
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M_total;
  t.B = B + (int64_t)e_found * N * K;
  t.sB = sB + (int64_t)e_found * (N / BK) * nkb;
  t.C = C;
  t.m0 = r0 + tm * G::BM; t.row_end = r1;
  t.n0 = tn * G::BN; t.N = N; t.K = K;
  run_tile<G, 0>(t, stage0, stage1);
}

// Estimated cost of a tile shape: full rounds of tiles over the CUs times the
// tile area (per-tile time is proportional to its area).
template <class G>
int64_t round_cost(int64_t tiles, int cus) {
  return ((tiles + cus - 1) / cus) * (int64_t)G::BM * G::BN;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// 0: 256x256, 1: 256x224, 2: 224x256
int pick_dense(int64_t M, int64_t N) {
  const int cus = device_cus();
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int64_t c0 = round_cost<Cfg256x256>(tiles(256, 256), cus);
  const int64_t c1 = round_cost<Cfg256x224>(tiles(256, 224), cus);
  const int64_t c2 = round_cost<Cfg224x256>(tiles(224, 256), cus);
  if (c0 <= c1 && c0 <= c2) return 0;
  return c1 <= c2 ? 1 : 2;
}

template <class G>
hipError_t launch_dense(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                        int row_mode, uint16_t* C, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
  const int tiles = (int)(((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN));
  if (row_mode)
    hipLaunchKernelGGL((gemm_kernel<G, 1>), dim3(tiles), dim3(kThreads), 0, stream, A, sA, B, sB, C,
                       (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL((gemm_kernel<G, 0>), dim3(tiles), dim3(kThreads), 0, stream, A, sA, B, sB, C,
                       (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace gemm

hipError_t launch_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, int row_mode, uint16_t* C, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream) {
  using namespace gemm;
  switch (pick_dense(M, N)) {
    case 1: return launch_dense<Cfg256x224>(A, sA, B, sB, row_mode, C, M, N, K, stream);
    case 2: return launch_dense<Cfg224x256>(A, sA, B, sB, row_mode, C, M, N, K, stream);
    default: return launch_dense<Cfg256x256>(A, sA, B, sB, row_mode, C, M, N, K, stream);
  }
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                           const float* sB, uint16_t* C, const int32_t* offsets,
                                           int E, int64_t M_total, int64_t N, int64_t K,
                                           hipStream_t stream) {
  using namespace gemm;
  using G = Cfg256x256;
  // every expert adds at most one partial m-tile beyond M_total / BM
  const int64_t tiles = ((M_total + G::BM - 1) / G::BM + E) * ((N + G::BN - 1) / G::BN);
  hipLaunchKernelGGL((grouped_gemm_kernel<G>), dim3((unsigned)tiles), dim3(kThreads), 0, stream, A,
                     sA, B, sB, C, offsets, E, (int)M_total, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace fp8bs
