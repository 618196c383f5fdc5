// MoE dispatch payload and combine for gfx950 (memory-bound).
//
// The method (DeepSeek-V3 report section 3.3.3, low-precision storage and
// communication): the activations that enter the MoE experts are quantized to
// FP8 before they are dispatched, so the dispatch payload is FP8 codes plus
// their scales (innerforce.co.kr page), while the combine that sums the
// experts' outputs back per token stays in BF16 (why-be.why-be.co.kr page).
//
// On one GPU the dispatch target is the grouped GEMM itself: the payload is
// written directly in its layout, rows sorted by expert and, inside an
// expert, by (token, slot) -- the order a stable sort by expert gives:
//   route:     per-block expert histograms, their scan (inside the rank
//              kernel for small tables), stable in-block ranks
//              -> offsets[E+1], pos[T][topk] (row of each token copy),
//                 src[T*topk] (token of each row);
//   dispatch:  each token row is read once, quantized 1x128 (the arithmetic of
//              the activation quantizer) and its codes and scales are stored
//              at the rows of all of its copies;
//   combine:   out[t] = bf16( sum_j w[t][j] * Y[pos[t][j]] ), FP32 sums in
//              slot order.

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace fp8bs {

constexpr int kRouteChunk = 1024;   // (token, slot) pairs per routing block
constexpr int kRouteThreads = 256;  // 4 waves, 4 pairs per thread
constexpr int kMaxExperts = 1024;

namespace {

// Streaming accesses: every byte of the payload, of Y and of the combined
// output is touched once, so they bypass the caches' normal retention
// (nontemporal loads and stores; 15-25% faster than plain ones here).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                    __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  __builtin_nontemporal_store(v.x, q);
  __builtin_nontemporal_store(v.y, q + 1);
  __builtin_nontemporal_store(v.z, q + 2);
  __builtin_nontemporal_store(v.w, q + 3);
}
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  __builtin_nontemporal_store(v.x, q);
  __builtin_nontemporal_store(v.y, q + 1);
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return min(max(e, 0), E - 1); }

// Per-block expert histogram: ws[b][e] = pairs of block b routed to expert e.
__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t P, int E,
                                                                    int32_t* __restrict__ ws) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int64_t first = (int64_t)blockIdx.x * kRouteChunk;
#pragma unroll
  for (int r = 0; r < kRouteChunk / kRouteThreads; ++r) {
    const int64_t i = first + r * kRouteThreads + threadIdx.x;
    if (i < P) atomicAdd(&hist[clamp_expert(ids[i], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) ws[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup: ws[b][e] becomes the first row of block b's pairs of expert
// e; offsets[e] the first row of expert e, offsets[E] = P. Thread e walks
// column e of ws in batches of 16 independent loads (stores to ws between
// the loads would otherwise serialize them).
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ ws, int nblocks, int E,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  int total = 0;
  if (t < E) {
    for (int b0 = 0; b0 < nblocks; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = b0 + u < nblocks ? ws[(int64_t)(b0 + u) * E + t] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) total += c[u];
    }
  }
  // exclusive scan of the experts' totals (E <= 1024: one value per thread)
  const int lane = t & 63, w = t >> 6;
  int incl = t < E ? total : 0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < w; ++k) before += wsum[k];
  const int excl = before + incl - (t < E ? total : 0);
  if (t < E) offsets[t] = excl;
  if (t == E - 1) offsets[E] = excl + total;
  if (t < E) {
    int run = excl;   // first row of the expert's pairs in block b0 + u
    for (int b0 = 0; b0 < nblocks; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) c[u] = b0 + u < nblocks ? ws[(int64_t)(b0 + u) * E + t] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < nblocks) ws[(int64_t)(b0 + u) * E + t] = run;
        run += c[u];
      }
    }
  }
}

// Stable ranks: pair i of block b goes to row first(b, e) + (pairs of block
// b before i with the same expert e), first(b, e) being the first row of block
// b's pairs of expert e. Without FUSED, route_scan_kernel has already turned
// ws[b][e] into first(b, e). With FUSED (small tables: blocks x experts <=
// kFusedScanMax) ws holds the raw histograms and every block forms its own
// first(., e) from the whole table (all blocks' counts for the experts'
// offsets, its predecessors' for its own position), which saves the scan's
// launch; block 0 also writes offsets. The block takes its pairs in four
// rounds of 256 consecutive pairs; inside a wave the pairs with the same
// expert are found with one ballot per bit of the expert id; the waves'
// counts meet in LDS, and a per-expert cursor carries the count over the
// rounds.
constexpr int kFusedScanMax = 16384;

template <bool FUSED>
__global__ __launch_bounds__(kRouteThreads) void route_rank_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                                    int E, int topk,
                                                                    const int32_t* __restrict__ ws, int nblocks,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ pos,
                                                                    int32_t* __restrict__ src) {
  __shared__ int cursor[kMaxExperts];
  __shared__ int cnt[4][kMaxExperts];
  __shared__ int wsum[kRouteThreads / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if constexpr (FUSED) {
    // per expert: every block's pairs (cnt[0]) and this block's predecessors' (cursor)
    for (int e = t; e < E; e += kRouteThreads) {
      int all = 0, before = 0;
      for (int b0 = 0; b0 < nblocks; b0 += kScanBatch) {
        int c[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) c[u] = b0 + u < nblocks ? ws[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
          all += c[u];
          if (b0 + u < (int)blockIdx.x) before += c[u];
        }
      }
      cnt[0][e] = all;
      cursor[e] = before;
    }
    __syncthreads();
    // exclusive scan of the experts' totals: thread t holds experts 4t .. 4t+3
    static_assert(4 * kRouteThreads >= kMaxExperts, "four experts per thread");
    int v[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = 4 * t + k < E ? cnt[0][4 * t + k] : 0;
      sum += v[k];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d, 64);
      if (lane >= d) incl += x;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int k = 0; k < w; ++k) run += wsum[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * t + k;
      if (e < E) {
        cursor[e] += run;
        if (blockIdx.x == 0) offsets[e] = run;
      }
      run += v[k];
    }
    if (blockIdx.x == 0 && t == kRouteThreads - 1) offsets[E] = run;   // every pair: P
    __syncthreads();   // cnt is reused below
  } else {
    for (int e = t; e < E; e += kRouteThreads) cursor[e] = ws[(int64_t)blockIdx.x * E + e];
  }
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const int64_t first = (int64_t)blockIdx.x * kRouteChunk;
  for (int r = 0; r < kRouteChunk / kRouteThreads; ++r) {
    const int64_t i = first + r * kRouteThreads + t;
    const bool valid = i < P;
    const int e = valid ? clamp_expert(ids[i], E) : 0;
    uint64_t same = __ballot(valid);
    for (int k = 0; k < bits; ++k) {
      const uint64_t b = __ballot((e >> k) & 1);
      same &= ((e >> k) & 1) ? b : ~b;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    const bool leader = valid && rank == 0;
    for (int x = t; x < 4 * E; x += kRouteThreads) cnt[x / E][x % E] = 0;
    __syncthreads();
    if (leader) cnt[w][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int row = cursor[e] + rank;
      for (int k = 0; k < w; ++k) row += cnt[k][e];
      pos[i] = row;
      src[row] = (int32_t)(i / topk);
    }
    __syncthreads();
    for (int x = t; x < E; x += kRouteThreads) cursor[x] += cnt[0][x] + cnt[1][x] + cnt[2][x] + cnt[3][x];
    __syncthreads();
  }
}

// Dispatch with quantization: block of 4 waves, 2 token rows per wave, K
// chunks 4*bx .. 4*bx+3; lane l covers elements (l%16)*8 .. +7 of chunk
// 4*bx + l/16 (the 1x128 activation quantizer's layout). Every token's codes
// and scales are stored at the rows of all of its topk copies.
template <bool BF16>
__global__ __launch_bounds__(256) void dispatch_quant_kernel(const void* __restrict__ x, int64_t T, int K,
                                                             const int32_t* __restrict__ pos, int topk,
                                                             int64_t M, uint8_t* __restrict__ q,
                                                             float* __restrict__ s) {
  constexpr int kRows = 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nkb = K / kGroup;
  const int part = lane & 15;
  const int kb = blockIdx.x * 4 + (lane >> 4);
  const int kbc = min(kb, nkb - 1);
  const int64_t rb = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t tok0 = (rb * 4 + wave) * kRows;
  if (tok0 - wave * kRows >= T) return;

  float v[kRows][8];
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    const int64_t tok = min(tok0 + u, T - 1);
    const int64_t elem = tok * K + (int64_t)kbc * kGroup + part * 8;
    if constexpr (BF16) {
      const uint4 d = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + elem);
      const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[u][2 * i] = __uint_as_float(wd[i] << 16);
        v[u][2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + elem);
      const float4 a = p[0], b = p[1];
      v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
      v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
    }
  }
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
    amax = row16_max(amax);
    const GroupDiv g = group_div<BF16>(amax);
    const uint2 codes = make_uint2(e4m3_div_pack4_t<BF16>(v[u][0], v[u][1], v[u][2], v[u][3], g),
                                   e4m3_div_pack4_t<BF16>(v[u][4], v[u][5], v[u][6], v[u][7], g));
    const int64_t tok = tok0 + u;
    if (tok < T && kb < nkb) {
      for (int j = 0; j < topk; ++j) {
        const int64_t row = min(max(pos[tok * topk + j], 0), (int32_t)(M - 1));
        store_nt8(q + row * K + (int64_t)kb * kGroup + part * 8, codes);
        if (part == 0) s[(int64_t)kb * M + row] = g.s;
      }
    }
  }
}

// Combine: thread g takes token t = g / (N/8) and columns 8 (g % (N/8)) ..
// +7; it sums its topk rows of Y in slot order with FP32 FMAs, loading up to
// 8 rows at a time before using them, and writes 8 BF16 values (16 bytes).
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y, int64_t M,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ wts, int64_t T, int topk,
                                                      int N, uint16_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = N / 8;
  const int64_t t = g / per_row;
  const int col = 8 * (int)(g - t * per_row);
  if (t >= T) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < topk; j0 += kCombineBatch) {
    uint4 d[kCombineBatch];
    float wj[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int j = min(j0 + u, topk - 1);
      const int64_t row = min(max(pos[t * topk + j], 0), (int32_t)(M - 1));
      wj[u] = j0 + u < topk ? wts[t * topk + j] : 0.0f;
      d[u] = load_nt16(Y + row * N + col);
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (j0 + u >= topk) break;
      const uint32_t wd[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj[u], __uint_as_float(wd[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj[u], __uint_as_float(wd[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = float_to_bf16_bits(acc[0]) | (float_to_bf16_bits(acc[1]) << 16);
  o.y = float_to_bf16_bits(acc[2]) | (float_to_bf16_bits(acc[3]) << 16);
  o.z = float_to_bf16_bits(acc[4]) | (float_to_bf16_bits(acc[5]) << 16);
  o.w = float_to_bf16_bits(acc[6]) | (float_to_bf16_bits(acc[7]) << 16);
  store_nt16(out + t * N + col, o);
}

dim3 row_grid(int64_t x_blocks, int64_t rows_per_y, int64_t rows) {
  const int64_t ny = (rows + rows_per_y - 1) / rows_per_y;
  const int64_t gy = ny < 65535 ? ny : 65535;
  return dim3((unsigned)x_blocks, (unsigned)gy, (unsigned)((ny + gy - 1) / gy));
}

}  // namespace

int64_t moe_route_blocks(int64_t pairs) { return (pairs + kRouteChunk - 1) / kRouteChunk; }

hipError_t launch_moe_dispatch(const void* x, bool bf16, int64_t T, int64_t K, const int32_t* ids, int topk,
                               int E, uint8_t* q, float* s, int32_t* offsets, int32_t* pos, int32_t* src,
                               int32_t* ws, hipStream_t stream) {
  const int64_t P = T * topk;
  const int nb = (int)moe_route_blocks(P);
  if (nb == 0) {   // no tokens: offsets all zero
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, ws, nb, E, offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_hist_kernel, dim3(nb), dim3(kRouteThreads), 0, stream, ids, P, E, ws);
  if ((int64_t)nb * E <= kFusedScanMax) {
    hipLaunchKernelGGL(route_rank_kernel<true>, dim3(nb), dim3(kRouteThreads), 0, stream, ids, P, E, topk, ws, nb,
                       offsets, pos, src);
  } else {
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, ws, nb, E, offsets);
    hipLaunchKernelGGL(route_rank_kernel<false>, dim3(nb), dim3(kRouteThreads), 0, stream, ids, P, E, topk, ws, nb,
                       offsets, pos, src);
  }
  if (K == 0) return hipGetLastError();
  const dim3 grid = row_grid((K / kGroup + 3) / 4, 8, T);
  if (bf16)
    hipLaunchKernelGGL(dispatch_quant_kernel<true>, grid, dim3(256), 0, stream, x, T, (int)K, pos, topk, P, q, s);
  else
    hipLaunchKernelGGL(dispatch_quant_kernel<false>, grid, dim3(256), 0, stream, x, T, (int)K, pos, topk, P, q, s);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* Y, const int32_t* pos, const float* w, int64_t T, int topk,
                              int64_t N, uint16_t* out, hipStream_t stream) {
  const int64_t threads = T * (N / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, Y, T * topk,
                     pos, w, T, topk, (int)N, out);
  return hipGetLastError();
}

int moe_max_experts() { return kMaxExperts; }

// ---------------------------------------------------------------------------
// Scratch memory of the no-allocation dispatch entry point: the routing
// workspace lives in this file-scope device array (each GPU the library runs
// on holds its own copy until the process ends) instead of caller memory.
// Host code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once per device, with that device current,
// and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int32_t scratch[kMoeScratchBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t moe_scratch(hipStream_t stream, int32_t** ptr) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fp8bs
