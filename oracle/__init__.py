"""CPU oracle for the fine-grained FP8 block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
shares no code, tables or helpers with the HIP library; it is a plain, slow,
obviously correct restatement of what the method computes, in numpy with
float64 arithmetic where the method does not fix the precision.

Sources (the DeepSeek-V3 technical report as paraphrased on the pages):
  * innerforce.co.kr page, report section 3.3.2 "Improved Precision from
    Quantization and Multiplication": elements are quantized in small groups
    that share a scale; E4M3 (4-bit exponent, 3-bit mantissa) is used for all
    tensors (Fprop, Dgrad, Wgrad); per-group scaling factors lie along the inner
    dimension of the GEMM; the FP8 Wgrad GEMM is what lets activations be kept
    in FP8.
  * why-be.why-be.co.kr page, same section, Figure 7(b): partial MMA results
    are promoted to FP32 registers at a fixed interval of the inner dimension
    and accumulated there in full FP32 precision.
  * the page headed "Deepseek : The Ultimate Convenience!", report sections
    3.3.2 and 3.5.2: per-group scaling along the inner dimension again, and the
    remark that fusing a transposition into the GEMM is cumbersome; report
    section 3.4.2: every MoE expert works on its own batch of tokens (the
    grouped forms).

Where the pages leave a step open (group geometry 1x128 / 128x128 / 128x1,
the OCP E4M3FN variant with max 448, scale = amax/448 in FP32, RNE, the
promotion interval of 128) the plainest reading is taken; each reading is
named in the function that uses it.

Every function here is pinned by the ``-m "not gpu"`` tests against closed
forms, brute force and independent library routines (torch's float8 cast and
integer matmul), never against this package itself.
"""

from .e4m3 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_finite_values)
from .quant import (GROUP, bf16_bits_to_f32, group_scale, pow2_scale, quant_act_1x128,
                    quant_act_128x1_T, quant_w_128x128)
from .gemm import gemm_ref, grouped_gemm_ref, gemm_ref_rows
from .grouped import grouped_wgrad_ref, padded_group_starts, quant_act_128x1_T_grouped
from .dispatch import check_combine, combine_ref, dispatch_quant, route
from .tolerance import bf16_ulp, check_gemm, bf16_bits_to_f64

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_finite_values", "GROUP",
    "bf16_bits_to_f32", "group_scale", "pow2_scale", "quant_act_1x128", "quant_act_128x1_T",
    "quant_w_128x128", "gemm_ref", "grouped_gemm_ref", "gemm_ref_rows",
    "bf16_ulp", "check_gemm", "bf16_bits_to_f64", "grouped_wgrad_ref", "padded_group_starts",
    "quant_act_128x1_T_grouped", "check_combine", "combine_ref", "dispatch_quant", "route",
]
