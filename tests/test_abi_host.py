"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/w4.h declares, and
reject invalid arguments with W4_EINVAL *before* touching the HIP runtime.
On a machine without a GPU any HIP call would fail, so a W4_EINVAL status
with the expected message shows the check ran first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")
LIB = os.path.join(ROOT, "dequant_gemm_quantize_amd", "libw4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libw4.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import dequant_gemm_quantize_amd as w4
    return w4.load()


def test_header_declares_the_abi():
    names = declared_functions()
    for want in ("quantize_pack_int4", "quantize_pack_int4_sym", "dequant_int4", "quantize_act_int8",
                 "w4a16_matmul", "w4a8_matmul", "w4_status_string", "w4_last_error", "w4_version"):
        assert want in names, names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_binding_covers_the_header():
    from dequant_gemm_quantize_amd import _lib
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == declared_functions()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, 7):
        assert lib.w4_status_string(code)
    assert b"W4_EINVAL" in lib.w4_status_string(-1)
    assert lib.w4_version().startswith(b"w4 ")


# pointer values used for validation only; they are never dereferenced
A = 0x10000  # 16-byte aligned
U = 0x10004  # misaligned


def _err(lib):
    return lib.w4_last_error().decode()


@pytest.mark.parametrize("args,msg", [
    ((A, 2, 4, 100, 32, A, A, A, 1, None), "not a multiple of group_size"),
    ((A, 2, 4, 128, 48, A, A, A, 1, None), "multiple of 32"),
    ((A, 2, 4, 128, 0, A, A, A, 1, None), "multiple of 32"),
    ((A, 2, 4, 0, 32, A, A, A, 1, None), "k = 0"),
    ((A, 2, -1, 128, 32, A, A, A, 1, None), "n = -1"),
    ((A, 1, 4, 128, 32, A, A, A, 1, None), "w dtype"),
    ((A, 2, 4, 128, 32, A, A, A, 2, None), "scale dtype"),
    ((None, 2, 4, 128, 32, A, A, A, 1, None), "w is NULL"),
    ((U, 2, 4, 128, 32, A, A, A, 1, None), "w is not 16-byte aligned"),
    ((A, 2, 4, 128, 32, A, U, A, 1, None), "scales is not 16-byte aligned"),
    ((A, 2, 4, 128, 32, A, A, None, 1, None), "zeros is NULL"),
    ((A, 2, 1 << 30, 1 << 20, 32, A, A, A, 1, None), "too large"),
    ((A, 2, 1 << 14, 1 << 23, 32, A, A, A, 1, None), "n * k"),
    ((A, 2, 4, (1 << 23) + 32, 32, A, A, A, 1, None), "k = 8388640 is too large"),
])
@pytest.mark.parametrize("name", ["quantize_pack_int4", "quantize_pack_int4_sym"])
def test_quantize_pack_rejects(lib, name, args, msg):
    assert getattr(lib, name)(*args) == -1
    assert msg in _err(lib), _err(lib)
    assert _err(lib).startswith(name + ":"), _err(lib)


@pytest.mark.parametrize("pct,g,msg", [(0.0, 128, "percentile 0 must lie in (0, 100]"),
                                       (100.5, 128, "must lie in (0, 100]"),
                                       (float("nan"), 128, "must lie in (0, 100]"),
                                       (99.9, 2048, "above the calibrators' limit of 1024"),
                                       (99.9, 48, "multiple of 32")])
def test_percentile_rejects(lib, pct, g, msg):
    assert lib.quantize_pack_int4_sym_percentile(A, 2, 4, 4096, g, pct, A, A, A, 1, None) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("cand,g,msg", [(1, 128, "candidates = 1 must lie in [2, 65536]"),
                                        (65537, 128, "must lie in [2, 65536]"),
                                        (1000, 2048, "limit of 1024"),
                                        (1000, 128, "zeros is NULL")])
def test_mse_rejects(lib, cand, g, msg):
    zeros = None if "zeros" in msg else A
    assert lib.quantize_pack_int4_sym_mse(A, 2, 4, 4096, g, cand, A, A, zeros, 1, None) == -1
    assert msg in _err(lib), _err(lib)


def test_empty_calls_are_noops(lib):
    assert lib.quantize_pack_int4(None, 2, 0, 128, 32, None, None, None, 1, None) == 0
    assert lib.quantize_pack_int4_sym(None, 2, 0, 128, 32, None, None, None, 1, None) == 0
    assert lib.quantize_pack_int4_sym_percentile(None, 2, 0, 128, 32, 99.9, None, None, None, 1, None) == 0
    assert lib.quantize_pack_int4_sym_mse(None, 2, 0, 128, 32, 1000, None, None, None, 1, None) == 0
    assert lib.dequant_int4(None, None, None, 1, 0, 128, 32, None, 2, None) == 0
    assert lib.quantize_act_int8(None, 2, 0, 128, None, None, None) == 0
    assert lib.w4a16_matmul(None, 2, 0, 128, None, None, None, 1, 64, 128, None, 2, None) == 0
    assert lib.w4a16_matmul(None, 2, 3, 128, None, None, None, 1, 0, 128, None, 2, None) == 0
    assert lib.w4a8_matmul(None, None, 0, 128, None, None, None, 1, 64, 128, None, 2, None) == 0


@pytest.mark.parametrize("args,msg", [
    ((A, 2, 1, 100, A, A, A, 1, 64, 32, A, 2, None), "not a multiple of group_size"),
    ((A, 1, 1, 128, A, A, A, 1, 64, 32, A, 2, None), "x dtype"),
    ((A, 2, 1, 128, A, A, A, 1, 64, 32, A, 1, None), "y dtype"),
    ((A, 2, -2, 128, A, A, A, 1, 64, 32, A, 2, None), "m = -2"),
    ((U, 2, 1, 128, A, A, A, 1, 64, 32, A, 2, None), "x is not 16-byte aligned"),
    ((A, 2, 1, 128, None, A, A, 1, 64, 32, A, 2, None), "packed is NULL"),
    ((A, 2, 1, 128, A, A, A, 1, 64, 32, U, 2, None), "y is not 16-byte aligned"),
    ((A, 2, 1, 128, A, A, A, 5, 64, 32, A, 2, None), "scale dtype"),
    ((A, 2, 1 << 30, 32, A, A, A, 1, 128, 32, A, 2, None), "m * n is too large"),
    ((A, 2, 1 << 29, 1 << 8, A, A, A, 1, 64, 32, A, 2, None), "m * k is too large"),
])
def test_w4a16_rejects(lib, args, msg):
    assert lib.w4a16_matmul(*args) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("args,msg", [
    ((A, A, 1, 100, A, A, A, 1, 64, 32, A, 2, None), "not a multiple of group_size"),
    ((A, None, 1, 128, A, A, A, 1, 64, 32, A, 2, None), "x_scale is NULL"),
    ((A, A + 2, 1, 128, A, A, A, 1, 64, 32, A, 2, None), "x_scale is not 4-byte aligned"),
    ((A, A, 1, 128, A, A, A, 1, 64, 32, A, 1, None), "y dtype"),
    ((None, A, 1, 128, A, A, A, 1, 64, 32, A, 2, None), "xq is NULL"),
])
def test_w4a8_rejects(lib, args, msg):
    assert lib.w4a8_matmul(*args) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("args,msg", [
    ((A, 2, 4, 100, A, A, None), "multiple of 8"),
    ((A, 1, 4, 128, A, A, None), "x dtype"),
    ((A, 2, 4, 128, A, None, None), "x_scale is NULL"),
    ((U, 2, 4, 128, A, A, None), "x is not 16-byte aligned"),
])
def test_act_quant_rejects(lib, args, msg):
    assert lib.quantize_act_int8(*args) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("args,msg", [
    ((A, A, A, 1, 4, 128, 32, A, 7, None), "out dtype"),
    ((A, A, A, 1, 4, 128, 32, U, 2, None), "w_out is not 16-byte aligned"),
])
def test_dequant_rejects(lib, args, msg):
    assert lib.dequant_int4(*args) == -1
    assert msg in _err(lib), _err(lib)


def test_binding_refuses_cpu_tensors():
    import torch
    import dequant_gemm_quantize_amd as w4
    with pytest.raises(ValueError, match="GPU only"):
        w4.quantize_pack_int4(torch.zeros(4, 128), 32)
    with pytest.raises(ValueError, match="GPU only"):
        w4.quantize_pack_int4_sym(torch.zeros(4, 128), 32)


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "dequant_gemm_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("no oracle", ""), f


def test_layer_arguments_without_gpu():
    """QuantizedLinear validates its shape arguments and refuses a biased
    Linear or an unknown mode before any GPU work."""
    import torch
    import dequant_gemm_quantize_amd as w4
    with pytest.raises(ValueError, match="multiple of group_size"):
        w4.QuantizedLinear(200, 64, group_size=128)
    with pytest.raises(ValueError, match="has one"):
        w4.QuantizedLinear.from_linear(torch.nn.Linear(256, 64, bias=True))
    with pytest.raises(ValueError, match="mode must be one of"):
        w4.QuantizedLinear.from_weight(torch.zeros(64, 256), mode="awq")
    with pytest.raises(ValueError, match="calibration rows"):
        w4.QuantizedLinear.from_weight(torch.zeros(64, 256), mode="gptq")
    layer = w4.QuantizedLinear(256, 64, group_size=128)
    assert tuple(layer.packed.shape) == (64, 128) and tuple(layer.scales.shape) == (64, 2)
    with pytest.raises(ValueError, match="features"):
        layer(torch.zeros(2, 128))


@pytest.mark.parametrize("args,msg", [
    ((A, 0, 64, A, None), "t = 0 calibration rows"),
    ((A, 8, 0, A, None), "k = 0 must lie in [1, 65536]"),
    ((A, 8, 65537, A, None), "must lie in [1, 65536]"),
    ((U, 8, 64, A, None), "x is not 16-byte aligned"),
    ((A, 8, 64, None, None), "h is NULL"),
    ((A, 1 << 40, 64, A, None), "t * k is too large"),
])
def test_gptq_hessian_rejects(lib, args, msg):
    assert lib.gptq_hessian(*args) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("args,msg", [
    ((A, 0, A + 256, A, None), "k = 0 must lie"),
    ((A, 64, A + 256, None, None), "info is NULL"),
    ((A, 64, A + 256, A + 2, None), "info is not 4-byte aligned"),
    ((A, 64, A, A, None), "h and u must be distinct"),
    ((U, 64, A, A, None), "h is not 16-byte aligned"),
])
def test_gptq_inverse_cholesky_rejects(lib, args, msg):
    assert lib.gptq_inverse_cholesky(*args) == -1
    assert msg in _err(lib), _err(lib)


@pytest.mark.parametrize("args,msg", [
    ((A, A, 4, 384, 96, 0, A, A, A, 1, None), "must be 32, 64 or a multiple of 128"),
    ((A, A, 4, 384, 160, 0, A, A, A, 1, None), "not a multiple of group_size"),
    ((A, A, 4, 131072, 128, 0, A, A, A, 1, None), "must be at most 65536"),
    ((A, None, 4, 256, 128, 1, A, A, A, 1, None), "u is NULL"),
    ((A, A, 4, 256, 128, 1, A, A, A, 7, None), "scale dtype"),
])
def test_gptq_quantize_rejects(lib, args, msg):
    assert lib.gptq_quantize_pack_int4(*args) == -1
    assert msg in _err(lib), _err(lib)


def test_gptq_empty_sweep_is_noop(lib):
    assert lib.gptq_quantize_pack_int4(None, None, 0, 256, 128, 0, None, None, None, 1, None) == 0


def _cpu_weights(n=8, k=256, g=128, sz=None, zsz=None):
    import torch
    sz = sz or torch.float16
    return (torch.zeros(n, k // 2, dtype=torch.uint8), torch.ones(n, k // g, dtype=sz),
            torch.zeros(n, k // g, dtype=zsz or sz))


def test_binding_checks_shapes_and_dtypes():
    """The wrappers refuse tensors whose shape or dtype does not match the
    call before anything reaches the library (the C ABI cannot see sizes, so
    such a call would read or write out of bounds there)."""
    import torch
    import dequant_gemm_quantize_amd as w4
    bf = torch.bfloat16
    p, s, z = _cpu_weights()
    x = torch.zeros(3, 256, dtype=bf)
    cases = [
        # w4a16_matmul
        (lambda: w4.w4a16_matmul(x, p, s, z, 128, out=torch.zeros(3, 9, dtype=bf)), "out has shape"),
        (lambda: w4.w4a16_matmul(x, p, s, z, 128, out=torch.zeros(3, 8, dtype=torch.float16)), "out has dtype"),
        (lambda: w4.w4a16_matmul(x, p, s[:, :1], z, 128), "scales has shape"),
        (lambda: w4.w4a16_matmul(x, p, s, z, 64), "scales has shape"),
        (lambda: w4.w4a16_matmul(x, p, s, z.float(), 128), "zeros has dtype"),
        (lambda: w4.w4a16_matmul(x, p, s.to(bf), z.to(bf), 128), "scales has dtype"),
        (lambda: w4.w4a16_matmul(x, p.to(torch.int8), s, z, 128), "packed has dtype"),
        (lambda: w4.w4a16_matmul(x, p, s, z, 96), "not a multiple of group_size"),
        (lambda: w4.w4a16_matmul(x.to(torch.float16), p, s, z, 128), "x has dtype"),
        (lambda: w4.w4a16_matmul(x[0], p, s, z, 128), "x must be a 2-D"),
        # w4a8_matmul
        (lambda: w4.w4a8_matmul(torch.zeros(3, 256, dtype=torch.uint8), torch.ones(3), p, s, z, 128),
         "xq has dtype"),
        (lambda: w4.w4a8_matmul(torch.zeros(3, 256, dtype=torch.int8), torch.ones(2), p, s, z, 128),
         "x_scale has shape"),
        (lambda: w4.w4a8_matmul(torch.zeros(3, 256, dtype=torch.int8), torch.ones(3, dtype=torch.float64),
                                p, s, z, 128), "x_scale has dtype"),
        (lambda: w4.w4a8_matmul(torch.zeros(3, 256, dtype=torch.int8), torch.ones(3), p, s, z, 128,
                                out=torch.zeros(8, 3, dtype=bf)), "out has shape"),
        # dequant_int4
        (lambda: w4.dequant_int4(p, s, z, 128, out=torch.zeros(8, 128, dtype=bf)), "out has shape"),
        (lambda: w4.dequant_int4(p, s, z.float(), 128), "zeros has dtype"),
        # quantizers
        (lambda: w4.quantize_pack_int4(torch.zeros(8, 256), 128, out=(p, s, z[:4])), "zeros has shape"),
        (lambda: w4.quantize_pack_int4(torch.zeros(8, 256), 128, out=(p[:, :64], s, z)), "packed has shape"),
        (lambda: w4.quantize_pack_int4(torch.zeros(8, 256), 100), "not a multiple of group_size"),
        (lambda: w4.quantize_pack_int4(torch.zeros(8, 256, dtype=torch.float16), 128), "w has dtype"),
        (lambda: w4.quantize_pack_int4(torch.zeros(8, 256), 128, torch.bfloat16), "sz_dtype must be"),
        (lambda: w4.quantize_pack_int4_sym_mse(torch.zeros(8, 256), 128, 10, out=(p, s, z.float())),
         "zeros has dtype"),
        # activations
        (lambda: w4.quantize_act_int8(x, out=(torch.zeros(3, 256, dtype=torch.int8), torch.zeros(4))),
         "x_scale has shape"),
        (lambda: w4.quantize_act_int8(x, out=(torch.zeros(3, 128, dtype=torch.int8), torch.zeros(3))),
         "xq has shape"),
        # GPTQ
        (lambda: w4.gptq_hessian(torch.zeros(5, 64), out=torch.zeros(64, 64)), "out has dtype"),
        (lambda: w4.gptq_hessian(torch.zeros(5, 64), out=torch.zeros(64, 32, dtype=torch.float64)),
         "out has shape"),
        (lambda: w4.gptq_inverse_cholesky(torch.eye(64, dtype=torch.float64),
                                          out=torch.zeros(63, 63, dtype=torch.float64)), "out has shape"),
        (lambda: w4.gptq_quantize_pack_int4(torch.zeros(8, 256), torch.eye(256, dtype=torch.float64), 128,
                                            out=(p, s[:, :1], z)), "scales has shape"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()
    # well-formed CPU tensors pass every check and are then refused for the device
    with pytest.raises(ValueError, match="GPU only"):
        w4.w4a16_matmul(x, p, s, z, 128)
    with pytest.raises(ValueError, match="GPU only"):
        w4.w4a8_matmul(torch.zeros(3, 256, dtype=torch.int8), torch.ones(3), p, s, z, 128)


PEAKS_HEADER = os.path.join(ROOT, "include", "w4_peaks.h")
PEAKS_LIB = os.path.join(ROOT, "dequant_gemm_quantize_amd", "libw4peaks.so")


@pytest.mark.skipif(not os.path.exists(PEAKS_LIB), reason="libw4peaks.so not built")
def test_peaks_library_exports_and_rejects():
    """The measurement library exports what include/w4_peaks.h declares and
    rejects bad arguments before any HIP call."""
    text = re.sub(r"/\*.*?\*/", "", open(PEAKS_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"^int\s+([a-z0-9_]+)\s*\(", text, flags=re.M)))
    assert names == ["w4_peak_mfma_loop", "w4_peak_stream_read"]
    raw = ctypes.CDLL(PEAKS_LIB)
    for n in names:
        assert hasattr(raw, n), n
    sr = raw.w4_peak_stream_read
    sr.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    mf = raw.w4_peak_mfma_loop
    mf.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                   ctypes.c_void_p]
    for args in ((None, 1024, 8, A, None), (A, 1000, 8, A, None), (A, 1024, 3, A, None),
                 (U, 1024, 8, A, None), (A, 0, 8, A, None), (A, 1024, 8, None, None)):
        assert sr(*args) == -1, args
    for args in ((2, A, 512, 10, A, None), (0, None, 512, 10, A, None), (0, A, 0, 10, A, None),
                 (1, A, 512, 0, A, None), (0, U, 512, 10, A, None)):
        assert mf(*args) == -1, args


def test_workspace_size_query(lib):
    """w4a16_matmul_workspace_size is host-only: split K for the down
    projection [4096, 11008] below 513 tokens (32 MiB at most), none for the
    M = 2048 prefill, decode shapes or invalid arguments."""
    import dequant_gemm_quantize_amd as w4
    assert w4.w4a16_matmul_workspace_size(256, 11008, 4096, 128) == 32 << 20
    assert 0 < w4.w4a16_matmul_workspace_size(129, 11008, 4096, 128) <= 32 << 20
    assert w4.w4a16_matmul_workspace_size(2048, 11008, 4096, 128) == 0
    assert w4.w4a16_matmul_workspace_size(2048, 4096, 11008, 128) == 0
    assert w4.w4a16_matmul_workspace_size(1, 4096, 11008, 128) == 0
    assert w4.w4a16_matmul_workspace_size(64, 11008, 4096, 128) == 0      # GEMV path
    assert w4.w4a16_matmul_workspace_size(256, 11008, 4096, 100) == 0     # invalid group
    assert w4.w4a16_matmul_workspace_size(256, 11008, 4096, 128, torch_float32()) == 0  # fp32 x: general kernel


def test_w4a8_workspace_size_query(lib):
    """w4a8_matmul_workspace_size is host-only: split K for one GPU's 8-way
    column shard [3584, 8192] from 17 tokens on (32 MiB at most), none for the
    whole [28672, 8192] projection at 512 tokens, the GEMV token counts or
    invalid arguments."""
    import dequant_gemm_quantize_amd as w4
    for m in (17, 128, 129, 512):
        assert 0 < w4.w4a8_matmul_workspace_size(m, 8192, 3584, 128) <= 32 << 20, m
    assert w4.w4a8_matmul_workspace_size(512, 8192, 28672, 128) == 0
    assert w4.w4a8_matmul_workspace_size(2048, 8192, 3584, 128) == 0
    for m in (1, 4, 16):                                                  # GEMV paths
        assert w4.w4a8_matmul_workspace_size(m, 8192, 3584, 128) == 0, m
    assert w4.w4a8_matmul_workspace_size(512, 8192, 3584, 96) == 0       # not a multiple of 128: general kernel
    assert w4.w4a8_matmul_workspace_size(512, 8192, 3584, 100) == 0      # invalid group
    assert w4.w4a8_matmul_workspace_size(0, 8192, 3584, 128) == 0


def torch_float32():
    import torch
    return torch.float32


def test_noalloc_validates_before_any_hip_call(lib):
    """The allocation-free entry point checks every argument before it looks
    up its scratch (a HIP call): on a machine without a GPU an invalid call
    still reports W4_EINVAL with the argument's message."""
    assert lib.w4a16_matmul_noalloc(A, 2, 256, 11008, A, A, A, 1, 4096, 128, None, 2, None) == -1
    assert "y is NULL" in _err(lib)
    assert lib.w4a16_matmul_noalloc(A, 2, 256, 11008, A, A, A, 1, 4096, 100, A, 2, None) == -1
    assert "group_size" in _err(lib)
    assert lib.w4a16_matmul_noalloc(None, 2, 0, 11008, None, None, None, 1, 4096, 128, None, 2, None) == 0
