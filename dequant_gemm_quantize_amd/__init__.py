"""MI355X-native group-wise INT4 weight quantization and fused dequantize-matmul.

The work runs in HIP kernels for gfx950 behind the C ABI of ``libw4.so``
(declared in include/w4.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    W4Error, load, quantize_pack_int4, quantize_pack_int4_sym, quantize_pack_int4_sym_percentile,
    quantize_pack_int4_sym_mse, dequant_int4, quantize_act_int8,
    gptq_hessian, gptq_inverse_cholesky, gptq_quantize_pack_int4,
    w4a16_matmul, w4a16_matmul_workspace_size, w4a8_matmul, w4a8_matmul_workspace_size, version,
    LIB_PATH,
    W4_F32, W4_F16, W4_BF16, W4_OK, W4_EINVAL, W4_EUNSUPPORTED, W4_EHIP,
)
from .layer import QuantizedLinear, replace_linears  # noqa: F401
