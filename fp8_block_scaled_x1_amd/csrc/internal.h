// Launchers behind the C ABI of libfp8bs (shapes and pointers are validated by
// the ABI layer before any of these is called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// pow2: power-of-two scales (the E8M0-compatible variant) instead of amax / 448
hipError_t launch_quant_act_1x128(const void* x, bool bf16, bool pow2, int64_t M, int64_t K, uint8_t* q,
                                  float* s, hipStream_t stream);
hipError_t launch_quant_w_128x128(const void* w, bool bf16, bool pow2, int64_t N, int64_t K, uint8_t* q,
                                  float* s, uint8_t* qT, float* sT, hipStream_t stream);
hipError_t launch_quant_act_128x1_T(const void* x, bool bf16, bool pow2, int64_t M, int64_t C, uint8_t* qT,
                                    float* sT, hipStream_t stream);
hipError_t launch_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                   const float* sB, int row_mode, uint16_t* C, int64_t M,
                                   int64_t N, int64_t K, hipStream_t stream);
// the output tile (rows, columns) launch_gemm_blockscaled picks for a shape
void gemm_blockscaled_tile(int64_t M, int64_t N, int64_t K, int row_mode, int* bm, int* bn, int* depth,
                           int* tail);
// sA and sB hold powers of two; the MFMA applies them as E8M0 block scales
hipError_t launch_gemm_blockscaled_pow2(const uint8_t* A, const float* sA, const uint8_t* B,
                                        const float* sB, int row_mode, uint16_t* C, int64_t M,
                                        int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_gemm_blockscaled_q1x128(const uint8_t* A, const float* sA, const uint8_t* B,
                                          const float* sB, int row_mode, uint8_t* Q, float* sQ,
                                          int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_grouped_gemm_wgrad(const uint8_t* A, const float* sA, const uint8_t* B,
                                     const float* sB, uint16_t* C, const int32_t* offsets, int E,
                                     int64_t M_total, int64_t N, int64_t K, int64_t ld,
                                     hipStream_t stream);
hipError_t launch_quant_act_128x1_T_grouped(const void* x, bool bf16, int64_t M_total, int64_t C,
                                            const int32_t* offsets, int E, int64_t ld, uint8_t* qT,
                                            float* sT, hipStream_t stream);
// both 1x128 (q, s) and 128x1 transposed (qT, sT) quantizations in one pass;
// offsets == nullptr: plain (ld = M), else grouped as the call above
hipError_t launch_quant_act_dual(const void* x, bool bf16, int64_t M, int64_t C, uint8_t* q, float* s,
                                 uint8_t* qT, float* sT, const int32_t* offsets, int E, int64_t ld,
                                 hipStream_t stream);
hipError_t launch_gemm_blockscaled_q1x128_q128x1T(const uint8_t* A, const float* sA, const uint8_t* B,
                                                  const float* sB, int row_mode, uint8_t* Q, float* sQ,
                                                  uint8_t* QT, float* sQT, int64_t M, int64_t N, int64_t K,
                                                  hipStream_t stream);
hipError_t launch_grouped_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                           const float* sB, uint16_t* C, const int32_t* offsets,
                                           int E, int64_t M_total, int64_t N, int64_t K,
                                           hipStream_t stream);

int64_t moe_route_blocks(int64_t pairs);
// the no-allocation dispatch's routing workspace: a device array of this many
// bytes per GPU; moe_scratch gives its device address on the stream's GPU
constexpr int64_t kMoeScratchBytes = (int64_t)1 << 20;
hipError_t moe_scratch(hipStream_t stream, int32_t** ptr);
int moe_max_experts();
hipError_t launch_moe_dispatch(const void* x, bool bf16, int64_t T, int64_t K, const int32_t* ids, int topk,
                               int E, uint8_t* q, float* s, int32_t* offsets, int32_t* pos, int32_t* src,
                               int32_t* ws, hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* Y, const int32_t* pos, const float* w, int64_t T, int topk,
                              int64_t N, uint16_t* out, hipStream_t stream);

}  // namespace fp8bs
