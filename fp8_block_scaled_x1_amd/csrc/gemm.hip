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
// registers the MFMA just wrote, with no data movement at all; the hardware
// overlaps it with the MFMAs of the next subtile.
//
// Structure (one 256x256 output tile per workgroup, 8 waves):
//   * one pipeline stage = one K chunk: A[256][128] + B[256][128] bytes, moved
//     HBM/L2 -> LDS with direct-to-LDS 16-byte loads (no VGPR staging), two
//     stages (132 KB of the 160 KB LDS), one barrier per chunk;
//   * LDS rows are 128 bytes; the 16-byte column index is XOR-swizzled with the
//     row (mod 8) so that fragment reads are bank-conflict free;
//   * each wave owns a 128(m) x 64(n) subtile = 8 x 4 MFMA 16x16x128 E4M3
//     tiles, i.e. exactly one MFMA per 16x16 tile per chunk: the MFMA covers
//     the whole promotion interval and starts from zero every chunk;
//   * MFMA operands are swapped (src0 = B rows, src1 = A rows) so that each
//     lane's four results share one A row (one sA value) and sit at four
//     consecutive n (one 8-byte BF16 store);
//   * the chunk's scale vectors (sA rows, and sB columns in row mode) travel
//     with the stage through LDS; a block-mode B scale is a scalar load;
//   * workgroup -> tile mapping is XCD-aware: consecutive tiles in a grouped
//     (8 m-tiles wide) order land on the same XCD, so the A and B panels they
//     share stay in that XCD's L2.

#include "device_common.h"
#include "internal.h"

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace gemm {

constexpr int BM = 256, BN = 256, BK = kGroup;
constexpr int kThreads = 512;                    // 8 waves
constexpr int WM = 128, WN = 64;                 // wave subtile
constexpr int MS = WM / 16, NS = WN / 16;        // 8 x 4 MFMA tiles per wave
constexpr int kTileBytes = BM * BK;              // 32 KB per operand per stage
constexpr int kScaleOfs = (BM + BN) * BK;        // stage layout: A tile, B tile, sA[256], sB[256]
constexpr int kStageBytes = kScaleOfs + (BM + BN) * 4;   // 66 KB
constexpr int kGroupM = 8;                       // tile-order grouping for L2 reuse
constexpr int kXcds = 8;

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

// 32 bytes of operand row r (K bytes 32h .. 32h+31, h = lane/16) for a 16x16x128
// MFMA; undoes the XOR swizzle of the 16-byte columns.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int lane) {
  const int h = lane >> 4;
  const int x = lane & 7;
  const uint8_t* rowp = tile + r * BK;
  const uint4 lo = *reinterpret_cast<const uint4*>(rowp + (((2 * h) ^ x) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(rowp + (((2 * h + 1) ^ x) << 4));
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
  int m0, row_end;    // tile rows m0 .. m0+255, valid below row_end
  int n0, N, K;
};

template <int ROW_MODE>
__device__ __forceinline__ void run_tile(const Tile& t, uint8_t* stage0, uint8_t* stage1) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int nkb = t.K / BK;
  const int a_last = t.row_end - 1;
  const int b_last = t.N - 1;

  // Direct-to-LDS operand loads: this wave fills tile rows 8*slice .. 8*slice+7
  // of A and of B for slice = 4*wave + j. Lane p writes LDS bytes p*16 of the
  // slice: row 8*slice + p/8, physical 16-byte column p%8, which holds logical
  // column (p%8) ^ (p/8) (the swizzle; row%8 == p/8). Offsets are 32-bit from
  // a uniform base (M*K, N*K < 2^31).
  const int rsub = lane >> 3;
  const uint32_t lcol16 = (uint32_t)(((lane & 7) ^ rsub) << 4);
  uint32_t offa[4], offb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rr = (wave * 4 + j) * 8 + rsub;
    offa[j] = (uint32_t)min(t.m0 + rr, a_last) * (uint32_t)t.K + lcol16;
    offb[j] = (uint32_t)min(t.n0 + rr, b_last) * (uint32_t)t.K + lcol16;
  }
  // Scale vectors of a stage: sA[kb][m0 .. m0+255] (wave 0) and, in row mode,
  // sB[kb][n0 .. n0+255] (wave 1), as 4 x 256-byte direct loads, clamped.
  uint32_t offs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (wave == 0) offs[j] = (uint32_t)min(t.m0 + 64 * j + lane, a_last);
    else offs[j] = (uint32_t)min(t.n0 + 64 * j + lane, b_last);
  }

  // scale-vector offsets in bytes
#pragma unroll
  for (int j = 0; j < 4; ++j) offs[j] *= 4u;

  auto issue_stage = [&](int kb, uint32_t st) {
    const uint8_t* Ak = t.A + (int64_t)kb * BK;
    const uint8_t* Bk = t.B + (int64_t)kb * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t slice = (uint32_t)(wave * 4 + j);
      lds_dma16(Ak, offa[j], st + slice * 1024u);
      lds_dma16(Bk, offb[j], st + (uint32_t)kTileBytes + slice * 1024u);
    }
    if (wave == 0) {
      const float* sk = t.sA + (int64_t)kb * t.sa_stride;
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_dma4(sk, offs[j], st + (uint32_t)kScaleOfs + j * 256u);
    } else if (ROW_MODE && wave == 1) {
      const float* sk = t.sB + (int64_t)kb * t.N;
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_dma4(sk, offs[j], st + (uint32_t)(kScaleOfs + BM * 4) + j * 256u);
    }
  };

  v4f acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // block mode: one B scale per (128-column block, chunk), uniform per wave
  const float* sbb_ptr = t.sB + (int64_t)(min(t.n0 + wn * WN, b_last) / BK) * nkb;

  // One chunk: wait for its stage, start the next stage's loads into the other
  // buffer, then compute. The two stages are distinct LDS objects so that the
  // compiler can see the next stage's direct-to-LDS writes never alias this
  // stage's fragment reads.
  auto chunk = [&](int kb, const uint8_t* st, uint32_t other) {
    __builtin_amdgcn_s_waitcnt(0);      // this wave's direct-to-LDS loads landed
    __syncthreads();                    // everyone's landed; everyone finished the other stage
    if (kb + 1 < nkb) issue_stage(kb + 1, other);
    const uint8_t* As = st;
    const uint8_t* Bs = st + kTileBytes;
    const float* sAs = reinterpret_cast<const float*>(st + kScaleOfs) + wm * WM + (lane & 15);
    const float* sBs = reinterpret_cast<const float*>(st + kScaleOfs + BM * 4) + wn * WN + 4 * (lane >> 4);
    const float sbb = ROW_MODE ? 0.f : sbb_ptr[kb];

    v8i bf[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) bf[j] = read_frag(Bs, wn * WN + j * 16 + (lane & 15), lane);
    float sbr[NS][4];
    if constexpr (ROW_MODE) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(sBs + 16 * j);
        sbr[j][0] = v.x; sbr[j][1] = v.y; sbr[j][2] = v.z; sbr[j][3] = v.w;
      }
    }

    // Software pipeline over the 8 m-subtiles: the MFMAs of subtile i are
    // issued before the promotion FMAs of subtile i-1, so the VALU work runs
    // while the matrix core is busy.
    v4f p_prev[NS];
    float sa_prev = 0.f;
    v8i af = read_frag(As, wm * WM + (lane & 15), lane);
#pragma unroll
    for (int i = 0; i <= MS; ++i) {
      v4f p_cur[NS];
      float sa_cur = 0.f;
      if (i < MS) {
        const v8i a_now = af;
        if (i + 1 < MS) af = read_frag(As, wm * WM + (i + 1) * 16 + (lane & 15), lane);
        sa_cur = sAs[16 * i];
#pragma unroll
        for (int j = 0; j < NS; ++j)
          p_cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], a_now, v4f{0.f, 0.f, 0.f, 0.f},
                                                                      0, 0, 0, 0, 0, 0);
      }
      if (i > 0) {
        // promotion of subtile i-1: scaled FP32 partial into the FP32 accumulator
        if constexpr (ROW_MODE) {
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i - 1][j][r] = fmaf(p_prev[j][r] * sbr[j][r], sa_prev, acc[i - 1][j][r]);
        } else {
          const float sc = sa_prev * sbb;
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = fmaf(p_prev[j][r], sc, acc[i - 1][j][r]);
        }
      }
      if (i < MS) {
#pragma unroll
        for (int j = 0; j < NS; ++j) p_prev[j] = p_cur[j];
        sa_prev = sa_cur;
      }
      __builtin_amdgcn_sched_barrier(0);
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

template <int ROW_MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const uint8_t* __restrict__ A,
                                                            const float* __restrict__ sA,
                                                            const uint8_t* __restrict__ B,
                                                            const float* __restrict__ sB,
                                                            uint16_t* __restrict__ C, int M, int N,
                                                            int K) {
  __shared__ __align__(16) uint8_t stage0[kStageBytes];
  __shared__ __align__(16) uint8_t stage1[kStageBytes];
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_coords(pid, tiles_m, tiles_n, tm, tn);
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M;
  t.B = B; t.sB = sB; t.C = C;
  t.m0 = tm * BM; t.row_end = M;
  t.n0 = tn * BN; t.N = N; t.K = K;
  run_tile<ROW_MODE>(t, stage0, stage1);
}

// Per-expert tiles: expert e owns rows [off[e], off[e+1]); its tiles are
// ceil(rows/256) x ceil(N/256), numbered expert-major. The grid is an upper
// bound on the total; workgroups past the last tile exit at once.
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sA, const uint8_t* __restrict__ B,
    const float* __restrict__ sB, uint16_t* __restrict__ C, const int32_t* __restrict__ offsets,
    int E, int M_total, int N, int K) {
  __shared__ __align__(16) uint8_t stage0[kStageBytes];
  __shared__ __align__(16) uint8_t stage1[kStageBytes];
  const int tiles_n = (N + BN - 1) / BN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  int base = 0, e_found = -1, r0 = 0, r1 = 0;
  for (int e = 0; e < E; ++e) {
    const int a = min(max(offsets[e], 0), M_total);
    const int b = min(max(offsets[e + 1], a), M_total);
    const int te = ((b - a + BM - 1) / BM) * tiles_n;
    if (pid < base + te) {
      e_found = e; r0 = a; r1 = b;
      break;
    }
    base += te;
  }
  if (e_found < 0) return;
  int tm, tn;
  tile_coords(pid - base, (r1 - r0 + BM - 1) / BM, tiles_n, tm, tn);
  const int64_t nkb = K / BK;
  Tile t;
  t.A = A; t.sA = sA; t.sa_stride = M_total;
  t.B = B + (int64_t)e_found * N * K;
  t.sB = sB + (int64_t)e_found * (N / BK) * nkb;
  t.C = C;
  t.m0 = r0 + tm * BM; t.row_end = r1;
  t.n0 = tn * BN; t.N = N; t.K = K;
  run_tile<0>(t, stage0, stage1);
}

}  // namespace gemm

hipError_t launch_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, int row_mode, uint16_t* C, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream) {
  using namespace gemm;
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  if (row_mode)
    hipLaunchKernelGGL(gemm_kernel<1>, dim3(tiles), dim3(kThreads), 0, stream, A, sA, B, sB, C,
                       (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL(gemm_kernel<0>, dim3(tiles), dim3(kThreads), 0, stream, A, sA, B, sB, C,
                       (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                           const float* sB, uint16_t* C, const int32_t* offsets,
                                           int E, int64_t M_total, int64_t N, int64_t K,
                                           hipStream_t stream) {
  using namespace gemm;
  // every expert adds at most one partial m-tile beyond M_total / 256
  const int64_t tiles = ((M_total + BM - 1) / BM + E) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, A, sA,
                     B, sB, C, offsets, E, (int)M_total, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace fp8bs
