"""Fine-grained FP8 (E4M3, block-scaled) GEMM library for AMD MI355X (gfx950).

The compute path is libfp8bs.so (hand-written HIP kernels behind a C ABI,
declared in include/fp8bs.h); this package is its thin Python binding. Build
the library with ``python -m fp8_block_scaled_x1_amd.build``.
"""

from ._lib import (ABI_VERSION, BF16, F32, LIB_PATH, SCALE_BLOCK128, SCALE_ROW, Fp8bsError,
                   fp8_gemm_blockscaled, fp8_gemm_blockscaled_q1x128, fp8_gemm_blockscaled_tile, fp8_gemm_blockscaled_q1x128_q128x1T,
                   fp8_grouped_gemm_blockscaled,
                   fp8_grouped_gemm_wgrad, fp8_moe_combine, fp8_moe_dispatch, fp8_moe_dispatch_noalloc, fp8_quant_act_128x1_T,
                   fp8_quant_act_128x1_T_grouped, fp8_quant_act_1x128_128x1_T,
                   fp8_quant_act_1x128_128x1_T_grouped,
                   fp8_quant_act_1x128, fp8_quant_w_128x128, grouped_ld, lib, status_string)

__all__ = [
    "ABI_VERSION", "BF16", "F32", "LIB_PATH", "SCALE_BLOCK128", "SCALE_ROW", "Fp8bsError",
    "fp8_gemm_blockscaled", "fp8_gemm_blockscaled_q1x128", "fp8_gemm_blockscaled_tile", "fp8_gemm_blockscaled_q1x128_q128x1T",
    "fp8_grouped_gemm_blockscaled",
    "fp8_grouped_gemm_wgrad", "fp8_moe_combine", "fp8_moe_dispatch", "fp8_moe_dispatch_noalloc", "fp8_quant_act_128x1_T",
    "fp8_quant_act_128x1_T_grouped",
    "fp8_quant_act_1x128_128x1_T",
    "fp8_quant_act_1x128_128x1_T_grouped",
    "fp8_quant_act_1x128", "fp8_quant_w_128x128", "grouped_ld", "lib", "status_string",
]
