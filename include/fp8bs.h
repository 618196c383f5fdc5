/*
 * fp8bs.h -- C ABI of the MI355X (gfx950) fine-grained FP8 block-scaled GEMM
 * library, libfp8bs.so.
 *
 * What the library computes is the FP8 GEMM of the DeepSeek-V3 technical
 * report, section 3.3.2 "Improved Precision from Quantization and
 * Multiplication", as paraphrased on the innerforce.co.kr and
 * why-be.why-be.co.kr pages (and again on the page headed "Deepseek : The
 * Ultimate Convenience!"):
 *   - tensors are quantized to E4M3 (4-bit exponent, 3-bit mantissa) in small
 *     groups, each group sharing one scaling factor, for all of Fprop, Dgrad
 *     and Wgrad;
 *   - the groups lie along the inner (K) dimension of the GEMM;
 *   - the FP8 product is formed one K interval at a time, each interval's
 *     partial result is promoted to FP32 and accumulated there in full FP32
 *     precision (report Figure 7(b)).
 * Readings where the pages are silent: OCP E4M3FN codes (bias 7, max 448, no
 * infinities), scale = amax/448 as an FP32 (1.0 for an all-zero group),
 * codes = E4M3_RNE_saturating(x / scale) with IEEE FP32 division, groups of
 * 1x128 (activations), 128x128 (weights) and 128x1 (Wgrad operands, written
 * transposed), promotion interval 128, BF16 output rounded to nearest even.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to caller-allocated, contiguous,
 *     row-major memory, 16-byte aligned. The library allocates nothing, keeps
 *     no state between calls and is safe to call from several host threads.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; nothing synchronizes inside the library.
 *   - Return value: FP8BS_OK (0) or a negative fp8bs_status. Arguments are
 *     validated on the host before anything is enqueued; on an error nothing
 *     is enqueued and the outputs are untouched. FP8BS_ERR_LAUNCH reports a
 *     launch failure from the HIP runtime. Faults inside a kernel (e.g. from
 *     device offsets that break their precondition) surface at the caller's
 *     next synchronization.
 *   - E4M3 codes are stored as uint8; BF16 as its uint16 bit pattern;
 *     scales as float32. `dtype` selects the high-precision input type.
 *   - Inputs must be finite; the result for NaN/Inf inputs is unspecified.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_ABI_VERSION 11

#ifndef FP8BS_API
#define FP8BS_API __attribute__((visibility("default")))
#endif

/* High-precision input type of the quantizers. */
enum fp8bs_dtype { FP8BS_F32 = 0, FP8BS_BF16 = 1 };

/* How the GEMM reads the B operand's scales (see fp8_gemm_blockscaled). */
enum fp8bs_scale_mode { FP8BS_SCALE_BLOCK128 = 0, FP8BS_SCALE_ROW = 1 };

enum fp8bs_status {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL_PTR = -1, /* a required pointer is NULL                      */
  FP8BS_ERR_SHAPE = -2,    /* negative size or a size not a multiple of 128   */
  FP8BS_ERR_ALIGN = -3,    /* a pointer is not 16-byte aligned                */
  FP8BS_ERR_DTYPE = -4,    /* unknown dtype                                   */
  FP8BS_ERR_MODE = -5,     /* unknown scale mode, or qT/sT given one-sided    */
  FP8BS_ERR_LAUNCH = -6,   /* the HIP runtime rejected a kernel launch        */
  FP8BS_ERR_TOO_LARGE = -7, /* a size exceeds the 32-bit index range supported */
  FP8BS_ERR_SCRATCH = -8    /* more scratch memory needed than a no-allocation
                               entry point holds                             */
};

/*
 * Activation quantization, one group per (row m, 128-wide K chunk kb):
 * report section 3.3.2 (fine-grained grouping along K), innerforce.co.kr page.
 *   x  [M][K]      F32 or BF16 (dtype)
 *   q  [M][K]      uint8 E4M3 codes
 *   s  [K/128][M]  float32, s[kb][m] = amax(group)/448, 1.0 for a zero group
 * K must be a multiple of 128; any M >= 0 (M == 0 or K == 0: no-op).
 * FP8BS_ERR_TOO_LARGE if M >= 2^30 - 8, K >= 2^31 or K/128 > 262140.
 */
FP8BS_API int fp8_quant_act_1x128(const void* x, int dtype, int64_t M, int64_t K,
                        uint8_t* q, float* s, void* stream);

/*
 * Weight quantization, one group per 128x128 block (nb, kb): report section
 * 3.3.2, innerforce.co.kr page. Optionally also writes the transposed copy
 * used by Dgrad (the pages call a transposition fused into the GEMM
 * cumbersome, report section 3.5.2, "Deepseek : The Ultimate Convenience!").
 *   w   [N][K]           F32 or BF16 (dtype)
 *   q   [N][K]           uint8 codes
 *   s   [N/128][K/128]   float32
 *   qT  [K][N]           uint8, qT = q^T        (NULL: not written)
 *   sT  [K/128][N/128]   float32, sT = s^T      (NULL: not written)
 * qT and sT must be both given or both NULL. N and K multiples of 128.
 */
FP8BS_API int fp8_quant_w_128x128(const void* w, int dtype, int64_t N, int64_t K,
                        uint8_t* q, float* s, uint8_t* qT, float* sT,
                        void* stream);

/*
 * Wgrad-operand quantization, one group per (token chunk tb, channel c):
 * 128 consecutive tokens of one channel, so that the Wgrad GEMM, which
 * contracts over tokens, again has its groups along its inner dimension
 * (report sections 3.3.1-3.3.2: the FP8 Wgrad GEMM). The codes are written
 * transposed so that the GEMM reads K-contiguous rows.
 *   x   [M][C]       F32 or BF16 (dtype); M = tokens, C = channels
 *   qT  [C][M]       uint8 codes, qT[c][t] encodes x[t][c]
 *   sT  [M/128][C]   float32
 * M must be a multiple of 128; any C >= 0.
 */
FP8BS_API int fp8_quant_act_128x1_T(const void* x, int dtype, int64_t M, int64_t C,
                          uint8_t* qT, float* sT, void* stream);

/*
 * Block-scaled FP8 GEMM with per-chunk FP32 promotion (report section 3.3.2
 * and Figure 7(b); why-be.why-be.co.kr and innerforce.co.kr pages):
 *   C[m][n] = bf16( sum_kb sA[kb][m] * sb(kb,n) * sum_{k in kb} A[m][k]*B[n][k] )
 * where each inner sum is an FP8 product accumulated in FP32 over one 128-wide
 * chunk, then promoted: scaled and added to an FP32 accumulator.
 *   A   [M][K]  uint8 codes (K contiguous)      sA [K/128][M] float32
 *   B   [N][K]  uint8 codes (K contiguous)      sB see mode
 *   b_scale_mode FP8BS_SCALE_BLOCK128: sB[N/128][K/128], sb(kb,n) = sB[n/128][kb]
 *                  (Fprop with W; Dgrad with the transposed weight copy)
 *                FP8BS_SCALE_ROW:      sB[K/128][N],     sb(kb,n) = sB[kb][n]
 *                  (Wgrad with both operands from fp8_quant_act_128x1_T)
 *   C   [M][N]  BF16 bits, round to nearest even
 * K and N multiples of 128; any M >= 0. M*K, N*K and M*N below 2^31.
 */
FP8BS_API int fp8_gemm_blockscaled(const uint8_t* A, const float* sA, const uint8_t* B,
                         const float* sB, int b_scale_mode, uint16_t* C,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The kernel fp8_gemm_blockscaled uses for an M x N x K problem in the given
 * scale mode on the current device: *bm rows by *bn columns of output per
 * workgroup; *depth, the K chunks its deeper operand ring holds (its loads
 * run depth - 1 chunks ahead); *tail_tiles, how many of its last tiles a
 * second launch computes as 64 x 64 subtiles spread over every compute unit
 * (0: none). The kernel is chosen per shape from an estimate of its time:
 * large tiles in whole rounds of the device's compute units on large
 * problems, with a short last round as subtiles, smaller tiles spread over
 * all units for problems with few tiles. depth and tail_tiles may be NULL.
 * A query only: it launches nothing. Returns FP8BS_ERR_NULL_PTR if bm or bn
 * is NULL, FP8BS_ERR_MODE for an unknown mode, FP8BS_ERR_SHAPE for sizes
 * fp8_gemm_blockscaled rejects.
 */
FP8BS_API int fp8_gemm_blockscaled_tile(int64_t M, int64_t N, int64_t K, int b_scale_mode,
                         int* bm, int* bn, int* depth, int* tail_tiles);

/*
 * Power-of-two scale variant (report section 3.5.2 on the innerforce.co.kr
 * page wishes for dequantization inside the matrix unit; gfx950's MFMA can
 * apply E8M0 block scales, i.e. powers of two, to its operands itself). The
 * quantizers below are fp8_quant_act_1x128, fp8_quant_w_128x128 and
 * fp8_quant_act_128x1_T with one change: each group's scale is the smallest
 * power of two not below amax/448 (the FP32 quotient), and not below 2^-126;
 * 1.0 for a zero group. Codes are E4M3(x / s), exact scaling by a power of
 * two. Layouts, arguments and errors as for the corresponding entry point.
 */
FP8BS_API int fp8_quant_act_1x128_pow2(const void* x, int dtype, int64_t M, int64_t K,
                        uint8_t* q, float* s, void* stream);
FP8BS_API int fp8_quant_w_128x128_pow2(const void* w, int dtype, int64_t N, int64_t K,
                        uint8_t* q, float* s, uint8_t* qT, float* sT,
                        void* stream);
FP8BS_API int fp8_quant_act_128x1_T_pow2(const void* x, int dtype, int64_t M, int64_t C,
                          uint8_t* qT, float* sT, void* stream);

/*
 * fp8_gemm_blockscaled for power-of-two scales: the same result definition,
 * but the MFMA applies sA and sB itself as E8M0 operand scales and
 * accumulates each chunk straight into the FP32 accumulator (no promotion FMA
 * on the vector ALUs). Every sA and sB value must be a power of two in
 * [2^-126, 2^127] (the _pow2 quantizers give such scales); only the exponent
 * field of each value is used. Arguments, layouts and errors as for
 * fp8_gemm_blockscaled.
 */
FP8BS_API int fp8_gemm_blockscaled_pow2(const uint8_t* A, const float* sA, const uint8_t* B,
                         const float* sB, int b_scale_mode, uint16_t* C,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The same GEMM with a quantizing epilogue: instead of the BF16 result it
 * writes that result's 1x128 quantization, the FP8 codes and FP32 scales the
 * next layer's GEMM reads (report section 3.5.2 on the innerforce.co.kr page:
 * FP8 conversion fused with the movement of activations). Q and sQ are
 * exactly what fp8_quant_act_1x128 (BF16 input) would produce from the C that
 * fp8_gemm_blockscaled writes, so C never goes to memory.
 *   A, sA, B, sB, b_scale_mode  as for fp8_gemm_blockscaled
 *   Q   [M][N]      uint8 E4M3 codes
 *   sQ  [N/128][M]  float32, sQ[g][m] = amax(C[m][128g .. 128g+127]) / 448,
 *                   1.0 for a zero group
 * Shapes, sizes, ownership and errors as for fp8_gemm_blockscaled.
 */
FP8BS_API int fp8_gemm_blockscaled_q1x128(const uint8_t* A, const float* sA, const uint8_t* B,
                         const float* sB, int b_scale_mode, uint8_t* Q, float* sQ,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The quantizing epilogue with both layouts the next layer needs: the 1x128
 * quantization (Q, sQ, as fp8_gemm_blockscaled_q1x128 writes it) and the
 * 128x1 quantization written transposed (QT, sQT: exactly what
 * fp8_quant_act_128x1_T, BF16 input, gives for the same BF16 result), the
 * copy the next layer's Wgrad GEMM reads (report sections 3.3.1-3.3.2: the
 * FP8 Wgrad GEMM lets activations be cached in FP8 for the backward pass,
 * innerforce.co.kr page).
 *   Q   [M][N] uint8,  sQ  [N/128][M] float32
 *   QT  [N][M] uint8,  sQT [M/128][N] float32
 * M must be a multiple of 128 (whole 128-row groups); otherwise as for
 * fp8_gemm_blockscaled_q1x128.
 */
FP8BS_API int fp8_gemm_blockscaled_q1x128_q128x1T(const uint8_t* A, const float* sA, const uint8_t* B,
                         const float* sB, int b_scale_mode, uint8_t* Q, float* sQ,
                         uint8_t* QT, float* sQT, int64_t M, int64_t N, int64_t K,
                         void* stream);

/*
 * Grouped (per-expert) form for MoE experts (report sections 3.3.2 and
 * 3.4.2; per-expert token batches, small in decoding, on the page headed
 * "Deepseek : The Ultimate Convenience!"): the rows [off[e], off[e+1]) of A
 * are multiplied by expert e's weights, block scale mode.
 *   A   [M_total][K]         uint8     sA [K/128][M_total] float32
 *   B   [E][N][K]            uint8     sB [E][N/128][K/128] float32
 *   C   [M_total][N]         BF16 bits
 *   group_offsets  DEVICE int32[E+1], 4-byte aligned, off[0] = 0,
 *                  non-decreasing, off[E] = M_total (precondition, not checked
 *                  on the host; the kernels clamp every row index into
 *                  [0, M_total)).
 * K and N multiples of 128; E >= 0; M_total >= 0.
 */
FP8BS_API int fp8_grouped_gemm_blockscaled(const uint8_t* A, const float* sA,
                                 const uint8_t* B, const float* sB,
                                 uint16_t* C, const int32_t* group_offsets,
                                 int E, int64_t M_total, int64_t N, int64_t K,
                                 void* stream);

/*
 * Wgrad-operand quantization per expert (128x1 groups as in
 * fp8_quant_act_128x1_T, report sections 3.3.1-3.3.2 on the innerforce.co.kr
 * page, applied to the per-expert token batches of the grouped form, report
 * section 3.4.2 on "Deepseek : The Ultimate Convenience!"). Expert e owns the
 * rows [off[e], off[e+1]) of x; its tokens are cut into groups of 128 from
 * its first row, and its last group is padded with zero tokens (+0 codes).
 * Groups are numbered expert-major: with P_e = sum_{e' < e} ceil(M_e' / 128),
 * group P_e + j holds rows off[e] + 128 j .. of expert e and lands in the qT
 * columns 128 (P_e + j) .. 128 (P_e + j) + 127 and in row P_e + j of sT.
 *   x    [M_total][C]    F32 or BF16 (dtype), rows grouped by expert
 *   qT   [C][ld]         uint8 codes; columns 128 * P_E .. ld-1 are not written
 *   sT   [ld/128][C]     float32; rows P_E .. are not written
 *   group_offsets  DEVICE int32[E+1], 4-byte aligned, off[0] = 0,
 *                  non-decreasing, off[E] = M_total (precondition as for the
 *                  grouped GEMM)
 * C a multiple of 128; ld a multiple of 128 with ld >= M_total + 127 E (room
 * for every expert's padding); E >= 0, M_total >= 0 (M_total == 0: no-op).
 * FP8BS_ERR_TOO_LARGE if M_total >= 2^31 or ld / 128 > 65535.
 */
FP8BS_API int fp8_quant_act_128x1_T_grouped(const void* x, int dtype, int64_t M_total, int64_t C,
                          const int32_t* group_offsets, int E, int64_t ld,
                          uint8_t* qT, float* sT, void* stream);

/*
 * Both quantizations of one activation in a single pass over it: the 1x128
 * groups of fp8_quant_act_1x128 (groups along each row's C values) and the
 * 128x1 groups of fp8_quant_act_128x1_T (groups along 128 rows of one
 * column, written transposed). The backward pass quantizes the output
 * gradient dY both ways, 1x128 for the Dgrad GEMM and 128x1 for the Wgrad
 * GEMM (FP8 for Fprop, Dgrad and Wgrad, report section 3.3.1, and the
 * per-group scaling along the inner dimension of each, report section 3.3.2,
 * on the innerforce.co.kr page); reading dY once halves the pass's input
 * traffic. Outputs bit-identical to the two calls:
 *   x    [M][C]        F32 or BF16 (dtype)
 *   q    [M][C]        uint8,  s  [C/128][M] float32   (fp8_quant_act_1x128, K = C)
 *   qT   [C][M]        uint8,  sT [M/128][C] float32   (fp8_quant_act_128x1_T)
 * M and C multiples of 128; M == 0 or C == 0: no-op. One pass for BF16
 * inputs with C a multiple of 256; otherwise the two passes, one after the
 * other, on the same stream. FP8BS_ERR_TOO_LARGE beyond the limits of either
 * call.
 */
FP8BS_API int fp8_quant_act_1x128_128x1_T(const void* x, int dtype, int64_t M, int64_t C,
                          uint8_t* q, float* s, uint8_t* qT, float* sT, void* stream);

/*
 * The same in the grouped (per-expert) form: q and s as fp8_quant_act_1x128
 * over all M_total rows, qT and sT as fp8_quant_act_128x1_T_grouped with the
 * same group_offsets, E and ld (the MoE backward needs the experts' dY both
 * ways: 1x128 for the grouped Dgrad, 128x1 per expert for the grouped Wgrad).
 *   x    [M_total][C]   q [M_total][C], s [C/128][M_total]
 *   qT   [C][ld]        sT [ld/128][C]   (columns and rows past the last group not written)
 * C a multiple of 128; ld a multiple of 128 with ld >= M_total + 127 E;
 * group_offsets 4-byte aligned, with the precondition of the grouped GEMM.
 */
FP8BS_API int fp8_quant_act_1x128_128x1_T_grouped(const void* x, int dtype, int64_t M_total, int64_t C,
                          const int32_t* group_offsets, int E, int64_t ld,
                          uint8_t* q, float* s, uint8_t* qT, float* sT, void* stream);

/*
 * Per-expert Wgrad GEMM (the FP8 Wgrad GEMM of report sections 3.3.1-3.3.2,
 * innerforce.co.kr page, in the grouped form of the MoE experts): for every
 * expert e, with the groups of fp8_quant_act_128x1_T_grouped,
 *   C[e][n][k] = bf16( sum_{g of e} sA[g][n] * sB[g][k] * sum_{t in g} A[n][t]*B[k][t] )
 * i.e. dW_e = dY_e^T X_e over expert e's tokens (row-mode scales on both
 * operands, per-group FP32 promotion as in fp8_gemm_blockscaled).
 *   A  [N][ld]  uint8, sA [ld/128][N]  fp8_quant_act_128x1_T_grouped of dY[M_total][N]
 *   B  [K][ld]  uint8, sB [ld/128][K]  fp8_quant_act_128x1_T_grouped of X[M_total][K]
 *   C  [E][N][K]  BF16 bits; an expert without tokens gets zeros
 *   group_offsets, E, M_total, ld  exactly as given to both quantizer calls
 * N and K multiples of 128; N*ld and K*ld below 2^31.
 */
FP8BS_API int fp8_grouped_gemm_wgrad(const uint8_t* A, const float* sA, const uint8_t* B,
                          const float* sB, uint16_t* C, const int32_t* group_offsets,
                          int E, int64_t M_total, int64_t N, int64_t K, int64_t ld,
                          void* stream);

/*
 * MoE dispatch with the payload in FP8 (report section 3.3.3: activations are
 * quantized to FP8 before they are dispatched to the experts, innerforce.co.kr
 * page). Routes every (token t, slot j) pair to expert topk_ids[t][j], sorts
 * the pairs by expert (stable: by t, then j, inside an expert) and writes, in
 * that row order, the 1x128 quantization of each pair's token row: exactly
 * the codes and scales fp8_quant_act_1x128 gives for x[t], ready for
 * fp8_grouped_gemm_blockscaled (A = q, sA = s, group_offsets = offsets,
 * M_total = T*topk). Each token row is read once.
 *   x         [T][K]        F32 or BF16 (dtype)
 *   topk_ids  [T][topk]     int32, DEVICE; experts in [0, E) (precondition;
 *                           others are treated as the nearest valid id)
 *   q         [T*topk][K]   uint8 codes, row r = copy of token src_row[r]
 *   s         [K/128][T*topk] float32
 *   offsets   [E+1]         int32, expert e owns rows [offsets[e], offsets[e+1])
 *   pos       [T][topk]     int32, the row of each pair
 *   src_row   [T*topk]      int32, the token of each row
 *   workspace DEVICE, at least fp8_moe_dispatch_workspace_bytes(T, topk, E)
 *             bytes; its contents on entry do not matter
 * 1 <= E <= 1024, 1 <= topk <= 64, K a multiple of 128, T >= 0 (T == 0 writes
 * offsets = 0 only). x, q and s 16-byte aligned; the int32 buffers 4-byte.
 */
FP8BS_API int fp8_moe_dispatch(const void* x, int dtype, int64_t T, int64_t K,
                          const int32_t* topk_ids, int topk, int E,
                          uint8_t* q, float* s, int32_t* offsets, int32_t* pos,
                          int32_t* src_row, void* workspace, void* stream);

/* Workspace bytes fp8_moe_dispatch needs (negative: invalid sizes). */
FP8BS_API int64_t fp8_moe_dispatch_workspace_bytes(int64_t T, int topk, int E);

/*
 * fp8_moe_dispatch for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same routing, payload and outputs, bit for bit, without the workspace
 * argument. The routing workspace is a device array inside the library, 1 MiB
 * on each GPU it runs on, held until the process ends; the call allocates
 * nothing. Problems whose workspace (fp8_moe_dispatch_workspace_bytes) exceeds
 * 1 MiB, i.e. 4 * E * ceil(T*topk / 1024) > 2^20, return FP8BS_ERR_SCRATCH
 * before anything is enqueued. Every call on one GPU uses that GPU's array:
 * calls that may run at the same time on one GPU (on different streams) race
 * and must be ordered by the caller. Other arguments, layouts and errors as
 * for fp8_moe_dispatch.
 */
FP8BS_API int fp8_moe_dispatch_noalloc(const void* x, int dtype, int64_t T, int64_t K,
                          const int32_t* topk_ids, int topk, int E,
                          uint8_t* q, float* s, int32_t* offsets, int32_t* pos,
                          int32_t* src_row, void* stream);

/*
 * MoE combine in BF16 (report section 3.3.3: the combine is kept in BF16,
 * why-be.why-be.co.kr page): every token's expert outputs are weighted and
 * summed back,
 *   out[t][n] = bf16( sum_{j < topk} w[t][j] * Y[pos[t][j]][n] )
 * with FP32 fused multiply-adds in slot order j = 0, 1, ... from zero, then
 * round to nearest even.
 *   Y    [T*topk][N]  BF16 bits (rows in the order fp8_moe_dispatch gave)
 *   pos  [T][topk]    int32 from fp8_moe_dispatch
 *   w    [T][topk]    float32 routing weights
 *   out  [T][N]       BF16 bits
 * N a multiple of 8; 1 <= topk <= 64; T >= 0.
 */
FP8BS_API int fp8_moe_combine(const uint16_t* Y, const int32_t* pos, const float* w,
                          int64_t T, int topk, int64_t N, uint16_t* out, void* stream);

/* Human-readable name of a status code (static string). */
FP8BS_API const char* fp8bs_status_string(int status);

/* FP8BS_ABI_VERSION of the loaded library. */
FP8BS_API int fp8bs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
