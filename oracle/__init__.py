"""CPU oracle (TEST INFRASTRUCTURE): plain NumPy restatement of the method.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library and its binding never do.
"""
from .w4_oracle import (  # noqa: F401
    widen_bf16, to_bf16, as_f32, split_groups, group_range, scale_zero,
    quantize_codes, pack_nibbles, unpack_nibbles, quantize_pack_int4,
    dequant_f32, dequant, dequant_f64, act_quant_int8, matmul_w4a16_f64,
    matmul_w4a8_f64, max_rel_err, SYM_OFFSET, group_absmax, scale_sym,
    quantize_codes_sym, quantize_pack_int4_sym, store_scale, percentile_position,
    calib_percentile_range, quantize_pack_int4_sym_percentile, mse_candidates,
    calib_mse_step, quantize_pack_int4_sym_mse, MSE_SKIP_BELOW, MSE_NONE,
)
