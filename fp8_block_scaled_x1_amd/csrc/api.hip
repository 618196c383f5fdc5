// C ABI of libfp8bs: host-side argument validation, then one launch on the
// caller's stream. Declarations and the meaning of every argument are in
// include/fp8bs.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8bs.h"
#include "internal.h"

namespace {

constexpr int64_t kG = 128;
constexpr int64_t kI32 = (int64_t)1 << 31;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

int status_of(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH; }

bool valid_dtype(int d) { return d == FP8BS_F32 || d == FP8BS_BF16; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int quant_act_1x128(const void* x, int dtype, bool pow2, int64_t M, int64_t K, uint8_t* q, float* s,
                    void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (M < 0 || K < 0 || K % kG) return FP8BS_ERR_SHAPE;
  // grid: x over groups of 4 chunks, (y, z) over blocks of 8 rows
  if (K >= kI32 || (M + 7) / 8 >= (int64_t)1 << 27 || (K / kG + 3) / 4 > 65535) return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || K == 0) return FP8BS_OK;
  if (!x || !q || !s) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(q) || misaligned(s)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_quant_act_1x128(x, dtype == FP8BS_BF16, pow2, M, K, q, s, as_stream(stream)));
}

int quant_w_128x128(const void* w, int dtype, bool pow2, int64_t N, int64_t K, uint8_t* q, float* s,
                    uint8_t* qT, float* sT, void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if ((qT == nullptr) != (sT == nullptr)) return FP8BS_ERR_MODE;
  if (N < 0 || K < 0 || N % kG || K % kG) return FP8BS_ERR_SHAPE;
  if (N >= kI32 || K >= kI32 || N * K >= kI32 * 4) return FP8BS_ERR_TOO_LARGE;
  if (N == 0 || K == 0) return FP8BS_OK;
  if (!w || !q || !s) return FP8BS_ERR_NULL_PTR;
  if (misaligned(w) || misaligned(q) || misaligned(s) || misaligned(qT) || misaligned(sT))
    return FP8BS_ERR_ALIGN;
  if (K / kG > 65535 * 1024 || N / kG > 65535) return FP8BS_ERR_TOO_LARGE;
  return status_of(fp8bs::launch_quant_w_128x128(w, dtype == FP8BS_BF16, pow2, N, K, q, s, qT, sT,
                                                 as_stream(stream)));
}

int quant_act_128x1_T(const void* x, int dtype, bool pow2, int64_t M, int64_t C, uint8_t* qT, float* sT,
                      void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (M < 0 || C < 0 || M % kG) return FP8BS_ERR_SHAPE;
  if (M >= kI32 || C >= kI32 || M / kG > 65535) return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || C == 0) return FP8BS_OK;
  if (!x || !qT || !sT) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(qT) || misaligned(sT)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_quant_act_128x1_T(x, dtype == FP8BS_BF16, pow2, M, C, qT, sT,
                                                   as_stream(stream)));
}

int gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB, int b_scale_mode,
                     uint16_t* C, int64_t M, int64_t N, int64_t K, bool pow2, void* stream) {
  if (b_scale_mode != FP8BS_SCALE_BLOCK128 && b_scale_mode != FP8BS_SCALE_ROW) return FP8BS_ERR_MODE;
  if (M < 0 || N < 0 || K <= 0 || K % kG || N % kG) return FP8BS_ERR_SHAPE;
  if (M * K >= kI32 || N * K >= kI32 || M * N >= kI32) return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!A || !sA || !B || !sB || !C) return FP8BS_ERR_NULL_PTR;
  if (misaligned(A) || misaligned(sA) || misaligned(B) || misaligned(sB) || misaligned(C))
    return FP8BS_ERR_ALIGN;
  if (pow2)
    return status_of(fp8bs::launch_gemm_blockscaled_pow2(A, sA, B, sB, b_scale_mode, C, M, N, K,
                                                         as_stream(stream)));
  return status_of(fp8bs::launch_gemm_blockscaled(A, sA, B, sB, b_scale_mode, C, M, N, K,
                                                  as_stream(stream)));
}

}  // namespace

extern "C" {

int fp8bs_abi_version(void) { return FP8BS_ABI_VERSION; }

const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL_PTR: return "null pointer";
    case FP8BS_ERR_SHAPE: return "invalid shape (negative, or not a multiple of 128 where required)";
    case FP8BS_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FP8BS_ERR_DTYPE: return "unknown input dtype";
    case FP8BS_ERR_MODE: return "unknown scale mode, or transposed outputs given one-sided";
    case FP8BS_ERR_LAUNCH: return "kernel launch failed";
    case FP8BS_ERR_TOO_LARGE: return "size exceeds the supported 32-bit index range";
    case FP8BS_ERR_SCRATCH: return "the problem needs more scratch memory than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int fp8_quant_act_1x128(const void* x, int dtype, int64_t M, int64_t K, uint8_t* q, float* s,
                        void* stream) {
  return quant_act_1x128(x, dtype, false, M, K, q, s, stream);
}

int fp8_quant_act_1x128_pow2(const void* x, int dtype, int64_t M, int64_t K, uint8_t* q, float* s,
                             void* stream) {
  return quant_act_1x128(x, dtype, true, M, K, q, s, stream);
}

int fp8_quant_w_128x128(const void* w, int dtype, int64_t N, int64_t K, uint8_t* q, float* s,
                        uint8_t* qT, float* sT, void* stream) {
  return quant_w_128x128(w, dtype, false, N, K, q, s, qT, sT, stream);
}

int fp8_quant_w_128x128_pow2(const void* w, int dtype, int64_t N, int64_t K, uint8_t* q, float* s,
                             uint8_t* qT, float* sT, void* stream) {
  return quant_w_128x128(w, dtype, true, N, K, q, s, qT, sT, stream);
}

int fp8_quant_act_128x1_T(const void* x, int dtype, int64_t M, int64_t C, uint8_t* qT, float* sT,
                          void* stream) {
  return quant_act_128x1_T(x, dtype, false, M, C, qT, sT, stream);
}

int fp8_quant_act_128x1_T_pow2(const void* x, int dtype, int64_t M, int64_t C, uint8_t* qT, float* sT,
                               void* stream) {
  return quant_act_128x1_T(x, dtype, true, M, C, qT, sT, stream);
}

int fp8_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                         int b_scale_mode, uint16_t* C, int64_t M, int64_t N, int64_t K,
                         void* stream) {
  return gemm_blockscaled(A, sA, B, sB, b_scale_mode, C, M, N, K, false, stream);
}

int fp8_gemm_blockscaled_tile(int64_t M, int64_t N, int64_t K, int b_scale_mode, int* bm, int* bn, int* depth,
                              int* tail_tiles) {
  if (!bm || !bn) return FP8BS_ERR_NULL_PTR;
  if (b_scale_mode != FP8BS_SCALE_BLOCK128 && b_scale_mode != FP8BS_SCALE_ROW) return FP8BS_ERR_MODE;
  if (M < 0 || N < 0 || K <= 0 || K % kG || N % kG) return FP8BS_ERR_SHAPE;
  fp8bs::gemm_blockscaled_tile(M, N, K, b_scale_mode, bm, bn, depth, tail_tiles);
  return FP8BS_OK;
}

int fp8_gemm_blockscaled_pow2(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                              int b_scale_mode, uint16_t* C, int64_t M, int64_t N, int64_t K,
                              void* stream) {
  return gemm_blockscaled(A, sA, B, sB, b_scale_mode, C, M, N, K, true, stream);
}

int fp8_gemm_blockscaled_q1x128(const uint8_t* A, const float* sA, const uint8_t* B,
                                const float* sB, int b_scale_mode, uint8_t* Q, float* sQ, int64_t M,
                                int64_t N, int64_t K, void* stream) {
  if (b_scale_mode != FP8BS_SCALE_BLOCK128 && b_scale_mode != FP8BS_SCALE_ROW) return FP8BS_ERR_MODE;
  if (M < 0 || N < 0 || K <= 0 || K % kG || N % kG) return FP8BS_ERR_SHAPE;
  if (M * K >= kI32 || N * K >= kI32 || M * N >= kI32) return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!A || !sA || !B || !sB || !Q || !sQ) return FP8BS_ERR_NULL_PTR;
  if (misaligned(A) || misaligned(sA) || misaligned(B) || misaligned(sB) || misaligned(Q) ||
      misaligned(sQ))
    return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_gemm_blockscaled_q1x128(A, sA, B, sB, b_scale_mode, Q, sQ, M, N, K,
                                                         as_stream(stream)));
}

int fp8_gemm_blockscaled_q1x128_q128x1T(const uint8_t* A, const float* sA, const uint8_t* B,
                                        const float* sB, int b_scale_mode, uint8_t* Q, float* sQ,
                                        uint8_t* QT, float* sQT, int64_t M, int64_t N, int64_t K,
                                        void* stream) {
  if (b_scale_mode != FP8BS_SCALE_BLOCK128 && b_scale_mode != FP8BS_SCALE_ROW) return FP8BS_ERR_MODE;
  if (M < 0 || N < 0 || K <= 0 || K % kG || N % kG || M % kG) return FP8BS_ERR_SHAPE;
  if (M * K >= kI32 || N * K >= kI32 || M * N >= kI32) return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!A || !sA || !B || !sB || !Q || !sQ || !QT || !sQT) return FP8BS_ERR_NULL_PTR;
  if (misaligned(A) || misaligned(sA) || misaligned(B) || misaligned(sB) || misaligned(Q) ||
      misaligned(sQ) || misaligned(QT) || misaligned(sQT))
    return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_gemm_blockscaled_q1x128_q128x1T(A, sA, B, sB, b_scale_mode, Q, sQ, QT, sQT,
                                                                 M, N, K, as_stream(stream)));
}

int fp8_grouped_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                                 const float* sB, uint16_t* C, const int32_t* group_offsets, int E,
                                 int64_t M_total, int64_t N, int64_t K, void* stream) {
  if (E < 0 || M_total < 0 || N < 0 || K <= 0 || K % kG || N % kG) return FP8BS_ERR_SHAPE;
  if (M_total * K >= kI32 || M_total * N >= kI32 || N * K >= kI32 || (int64_t)E * N * K >= kI32 * 4)
    return FP8BS_ERR_TOO_LARGE;
  if (E == 0 && M_total > 0) return FP8BS_ERR_SHAPE;   // rows with no expert
  if (M_total == 0 || N == 0) return FP8BS_OK;
  if (!A || !sA || !B || !sB || !C || !group_offsets) return FP8BS_ERR_NULL_PTR;
  if (misaligned(A) || misaligned(sA) || misaligned(B) || misaligned(sB) || misaligned(C) ||
      misaligned4(group_offsets))
    return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_grouped_gemm_blockscaled(A, sA, B, sB, C, group_offsets, E,
                                                          M_total, N, K, as_stream(stream)));
}

int fp8_quant_act_128x1_T_grouped(const void* x, int dtype, int64_t M_total, int64_t C,
                                  const int32_t* group_offsets, int E, int64_t ld, uint8_t* qT,
                                  float* sT, void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (E < 0 || M_total < 0 || C < 0 || C % kG || ld < 0 || ld % kG) return FP8BS_ERR_SHAPE;
  if (E == 0 && M_total > 0) return FP8BS_ERR_SHAPE;     // rows with no expert
  if (ld < M_total + (kG - 1) * E) return FP8BS_ERR_SHAPE;
  if (M_total >= kI32 || C >= kI32 || ld / kG > 65535) return FP8BS_ERR_TOO_LARGE;
  if (M_total == 0 || C == 0) return FP8BS_OK;
  if (!x || !qT || !sT || !group_offsets) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(qT) || misaligned(sT) || misaligned4(group_offsets)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_quant_act_128x1_T_grouped(x, dtype == FP8BS_BF16, M_total, C, group_offsets,
                                                           E, ld, qT, sT, as_stream(stream)));
}

int fp8_quant_act_1x128_128x1_T(const void* x, int dtype, int64_t M, int64_t C, uint8_t* q, float* s,
                                uint8_t* qT, float* sT, void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (M < 0 || C < 0 || M % kG || C % kG) return FP8BS_ERR_SHAPE;
  if (M >= kI32 || C >= kI32 || M / kG > 65535 || (C / kG + 3) / 4 > 65535 || (M + 7) / 8 >= (int64_t)1 << 27)
    return FP8BS_ERR_TOO_LARGE;
  if (M == 0 || C == 0) return FP8BS_OK;
  if (!x || !q || !s || !qT || !sT) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(q) || misaligned(s) || misaligned(qT) || misaligned(sT)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_quant_act_dual(x, dtype == FP8BS_BF16, M, C, q, s, qT, sT, nullptr, 0, M,
                                                as_stream(stream)));
}

int fp8_quant_act_1x128_128x1_T_grouped(const void* x, int dtype, int64_t M_total, int64_t C,
                                        const int32_t* group_offsets, int E, int64_t ld, uint8_t* q, float* s,
                                        uint8_t* qT, float* sT, void* stream) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (E < 0 || M_total < 0 || C < 0 || C % kG || ld < 0 || ld % kG) return FP8BS_ERR_SHAPE;
  if (E == 0 && M_total > 0) return FP8BS_ERR_SHAPE;     // rows with no expert
  if (ld < M_total + (kG - 1) * E) return FP8BS_ERR_SHAPE;
  if (M_total >= kI32 || C >= kI32 || ld / kG > 65535 || (C / kG + 3) / 4 > 65535 ||
      (M_total + 7) / 8 >= (int64_t)1 << 27)
    return FP8BS_ERR_TOO_LARGE;
  if (M_total == 0 || C == 0) return FP8BS_OK;
  if (!x || !q || !s || !qT || !sT || !group_offsets) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(q) || misaligned(s) || misaligned(qT) || misaligned(sT) ||
      misaligned4(group_offsets))
    return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_quant_act_dual(x, dtype == FP8BS_BF16, M_total, C, q, s, qT, sT, group_offsets,
                                                E, ld, as_stream(stream)));
}

int fp8_grouped_gemm_wgrad(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                           uint16_t* C, const int32_t* group_offsets, int E, int64_t M_total,
                           int64_t N, int64_t K, int64_t ld, void* stream) {
  if (E < 0 || M_total < 0 || N < 0 || K < 0 || N % kG || K % kG || ld < 0 || ld % kG)
    return FP8BS_ERR_SHAPE;
  if (E == 0 && M_total > 0) return FP8BS_ERR_SHAPE;
  if (ld < M_total + (kG - 1) * E) return FP8BS_ERR_SHAPE;
  if (M_total >= kI32 || N * ld >= kI32 || K * ld >= kI32 || (int64_t)E * (N / kG) * (K / kG) >= kI32)
    return FP8BS_ERR_TOO_LARGE;
  if (E == 0 || N == 0 || K == 0) return FP8BS_OK;
  if (!A || !sA || !B || !sB || !C || !group_offsets) return FP8BS_ERR_NULL_PTR;
  if (misaligned(A) || misaligned(sA) || misaligned(B) || misaligned(sB) || misaligned(C) ||
      misaligned4(group_offsets))
    return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_grouped_gemm_wgrad(A, sA, B, sB, C, group_offsets, E, M_total, N, K, ld,
                                                    as_stream(stream)));
}

int64_t fp8_moe_dispatch_workspace_bytes(int64_t T, int topk, int E) {
  if (T < 0 || topk < 1 || topk > 64 || E < 1 || E > fp8bs::moe_max_experts()) return FP8BS_ERR_SHAPE;
  if (T * topk >= kI32) return FP8BS_ERR_TOO_LARGE;
  return 4 * (int64_t)E * fp8bs::moe_route_blocks(T * topk);
}

namespace {
// argument checks shared by both dispatch entry points (workspace aside)
int dispatch_checks(const void* x, int dtype, int64_t T, int64_t K, const int32_t* topk_ids, int topk, int E,
                    uint8_t* q, float* s, int32_t* offsets, int32_t* pos, int32_t* src_row) {
  if (!valid_dtype(dtype)) return FP8BS_ERR_DTYPE;
  if (T < 0 || K < 0 || K % kG || topk < 1 || topk > 64 || E < 1 || E > fp8bs::moe_max_experts())
    return FP8BS_ERR_SHAPE;
  const int64_t P = T * topk;
  if (P >= kI32 || K >= kI32 || (K / kG + 3) / 4 > 65535 || (T + 7) / 8 >= (int64_t)1 << 27)
    return FP8BS_ERR_TOO_LARGE;
  if (!offsets) return FP8BS_ERR_NULL_PTR;
  if (P > 0 && (!topk_ids || !pos || !src_row)) return FP8BS_ERR_NULL_PTR;
  if (P > 0 && K > 0 && (!x || !q || !s)) return FP8BS_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(q) || misaligned(s)) return FP8BS_ERR_ALIGN;
  if (misaligned4(topk_ids) || misaligned4(offsets) || misaligned4(pos) || misaligned4(src_row))
    return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}
}  // namespace

int fp8_moe_dispatch_noalloc(const void* x, int dtype, int64_t T, int64_t K, const int32_t* topk_ids, int topk,
                             int E, uint8_t* q, float* s, int32_t* offsets, int32_t* pos, int32_t* src_row,
                             void* stream) {
  const int st = dispatch_checks(x, dtype, T, K, topk_ids, topk, E, q, s, offsets, pos, src_row);
  if (st != FP8BS_OK) return st;
  if (4 * (int64_t)E * fp8bs::moe_route_blocks(T * topk) > fp8bs::kMoeScratchBytes) return FP8BS_ERR_SCRATCH;
  int32_t* ws = nullptr;
  const hipError_t e = fp8bs::moe_scratch(as_stream(stream), &ws);
  if (e != hipSuccess) return FP8BS_ERR_LAUNCH;
  return status_of(fp8bs::launch_moe_dispatch(x, dtype == FP8BS_BF16, T, K, topk_ids, topk, E, q, s, offsets,
                                              pos, src_row, ws, as_stream(stream)));
}

int fp8_moe_dispatch(const void* x, int dtype, int64_t T, int64_t K, const int32_t* topk_ids, int topk, int E,
                     uint8_t* q, float* s, int32_t* offsets, int32_t* pos, int32_t* src_row, void* workspace,
                     void* stream) {
  const int st = dispatch_checks(x, dtype, T, K, topk_ids, topk, E, q, s, offsets, pos, src_row);
  if (st != FP8BS_OK) return st;
  if (T * topk > 0 && !workspace) return FP8BS_ERR_NULL_PTR;
  if (misaligned4(workspace)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_moe_dispatch(x, dtype == FP8BS_BF16, T, K, topk_ids, topk, E, q, s, offsets,
                                              pos, src_row, static_cast<int32_t*>(workspace),
                                              as_stream(stream)));
}

int fp8_moe_combine(const uint16_t* Y, const int32_t* pos, const float* w, int64_t T, int topk, int64_t N,
                    uint16_t* out, void* stream) {
  if (T < 0 || N < 0 || N % 8 || topk < 1 || topk > 64) return FP8BS_ERR_SHAPE;
  if (T * topk >= kI32 || N >= kI32 || T * (N / 8) >= kI32 * 64) return FP8BS_ERR_TOO_LARGE;
  if (T == 0 || N == 0) return FP8BS_OK;
  if (!Y || !pos || !w || !out) return FP8BS_ERR_NULL_PTR;
  if (misaligned(Y) || misaligned(out)) return FP8BS_ERR_ALIGN;
  if (misaligned4(pos) || misaligned4(w)) return FP8BS_ERR_ALIGN;
  return status_of(fp8bs::launch_moe_combine(Y, pos, w, T, topk, N, out, as_stream(stream)));
}

}  // extern "C"
