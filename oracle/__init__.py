"""CPU oracle for the packed Q1 path.  Test infrastructure only: the library
never imports it; tests, the smoke check and the benchmark's CPU baseline do."""
from .q1_oracle import *  # noqa: F401,F403
from .q1_oracle import (GROUP, bf16_to_f32, f16_to_f32, meta_to_f32, f32_to_bf16_rne, f32_to_f16_rne, round_to,
                        out_to_f64, unpack_bits, group_scale_bias, dequant_f32, dequantize, embed_rows, qmm_ref,
                        tolerance, dense_rounding_bound, output_half_ulp, check_within, check_close, qmm_exact, silu, silu_grad, ffn_ref, h_perturbation_bound,
                        ffn_h_bound, ffn_y_bound,
                        symmetric_mismatches, pack_signs)
