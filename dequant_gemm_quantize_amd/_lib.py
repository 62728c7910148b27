"""ctypes binding of libw4.so.

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/w4.h.  PyTorch supplies device memory and the
current stream.  There is no CPU fallback: if the library is missing or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("W4_LIB", os.path.join(HERE, "libw4.so"))

W4_F32, W4_F16, W4_BF16 = 0, 1, 2
W4_OK, W4_EINVAL, W4_EUNSUPPORTED, W4_EHIP = 0, -1, -2, -3

_DT = {torch.float32: W4_F32, torch.float16: W4_F16, torch.bfloat16: W4_BF16}

# (name, restype, argtypes) of every exported function, in header order.
_VP, _I, _I64, _I32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32
SIGNATURES = [
    ("quantize_pack_int4", _I, [_VP, _I, _I64, _I64, _I32, _VP, _VP, _VP, _I, _VP]),
    ("quantize_pack_int4_sym", _I, [_VP, _I, _I64, _I64, _I32, _VP, _VP, _VP, _I, _VP]),
    ("quantize_pack_int4_sym_percentile", _I,
     [_VP, _I, _I64, _I64, _I32, ctypes.c_double, _VP, _VP, _VP, _I, _VP]),
    ("quantize_pack_int4_sym_mse", _I, [_VP, _I, _I64, _I64, _I32, _I32, _VP, _VP, _VP, _I, _VP]),
    ("dequant_int4", _I, [_VP, _VP, _VP, _I, _I64, _I64, _I32, _VP, _I, _VP]),
    ("quantize_act_int8", _I, [_VP, _I, _I64, _I64, _VP, _VP, _VP]),
    ("w4a16_matmul", _I, [_VP, _I, _I64, _I64, _VP, _VP, _VP, _I, _I64, _I32, _VP, _I, _VP]),
    ("w4a16_matmul_workspace_size", ctypes.c_size_t, [_I64, _I64, _I64, _I32, _I]),
    ("w4a16_matmul_ws", _I, [_VP, _I, _I64, _I64, _VP, _VP, _VP, _I, _I64, _I32, _VP, _I, _VP,
                             ctypes.c_size_t, _VP]),
    ("w4a16_matmul_noalloc", _I, [_VP, _I, _I64, _I64, _VP, _VP, _VP, _I, _I64, _I32, _VP, _I, _VP]),
    ("w4a8_matmul", _I, [_VP, _VP, _I64, _I64, _VP, _VP, _VP, _I, _I64, _I32, _VP, _I, _VP]),
    ("w4a8_matmul_workspace_size", ctypes.c_size_t, [_I64, _I64, _I64, _I32]),
    ("w4a8_matmul_ws", _I, [_VP, _VP, _I64, _I64, _VP, _VP, _VP, _I, _I64, _I32, _VP, _I, _VP,
                            ctypes.c_size_t, _VP]),
    ("gptq_hessian", _I, [_VP, _I64, _I64, _VP, _VP]),
    ("gptq_inverse_cholesky", _I, [_VP, _I64, _VP, _VP, _VP]),
    ("gptq_quantize_pack_int4", _I, [_VP, _VP, _I64, _I64, _I32, _I32, _VP, _VP, _VP, _I, _VP]),
    ("w4_status_string", ctypes.c_char_p, [_I]),
    ("w4_last_error", ctypes.c_char_p, []),
    ("w4_version", ctypes.c_char_p, []),
]

_lib = None


class W4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libw4.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"libw4.so not found at {p}: build it first "
            "(python -m dequant_gemm_quantize_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != W4_OK:
        lib = load()
        msg = lib.w4_last_error().decode() or lib.w4_status_string(status).decode()
        raise W4Error(status, msg)


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _gpu(*ts: torch.Tensor) -> torch.device:
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libw4 runs on the GPU only: every tensor must be on a cuda (HIP) device")
        if not t.is_contiguous():
            raise ValueError("libw4 expects contiguous row-major tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    return _DT[dt]


# Shape and dtype checks.  The C ABI sees only pointers and sizes, so a
# tensor of the wrong shape or dtype would be read or written out of bounds
# there; the wrappers, which know every tensor's size, refuse such calls
# before anything reaches the library.
def _expect(t: torch.Tensor, name: str, shape, dtypes) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} has dtype {str(t.dtype).replace('torch.', '')}, expected {names}")


def _matrix(t: torch.Tensor, name: str) -> Tuple[int, int]:
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor, got {t.dim()} dimensions")
    return int(t.shape[0]), int(t.shape[1])


def _ngroups(k: int, group_size: int) -> int:
    if group_size <= 0 or k % group_size:
        raise ValueError(f"K = {k} is not a multiple of group_size = {group_size}")
    return k // group_size


SZ_DTYPES = (torch.float16, torch.float32)


def _check_weights(packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, k: int,
                   group_size: int) -> int:
    """packed uint8 [N, K/2], scales and zeros [N, K/g] of one dtype; returns N."""
    n = _matrix(packed, "packed")[0]
    _expect(packed, "packed", (n, k // 2), (torch.uint8,))
    ng = _ngroups(k, group_size)
    _expect(scales, "scales", (n, ng), SZ_DTYPES)
    _expect(zeros, "zeros", (n, ng), (scales.dtype,))
    return n


# ---------------------------------------------------------------------------
# Public wrappers (same names as the C ABI)
# ---------------------------------------------------------------------------
def quantize_pack_int4(w: torch.Tensor, group_size: int, sz_dtype: torch.dtype = torch.float16,
                       out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """W [N, K] (fp32 or bf16) -> (packed uint8 [N, K/2], scales [N, K/g], zeros [N, K/g])."""
    return _quantize_pack(load().quantize_pack_int4, w, group_size, sz_dtype, out)


def quantize_pack_int4_sym(w: torch.Tensor, group_size: int, sz_dtype: torch.dtype = torch.float16,
                           out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Symmetric variant: same arguments and outputs; every zero-point is 8."""
    return _quantize_pack(load().quantize_pack_int4_sym, w, group_size, sz_dtype, out)


def quantize_pack_int4_sym_percentile(w: torch.Tensor, group_size: int, percentile: float = 99.9,
                                      sz_dtype: torch.dtype = torch.float16,
                                      out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Symmetric format, scale = (percentile of |w| per group) / 7."""
    fn = load().quantize_pack_int4_sym_percentile
    return _quantize_pack(lambda w_, d, n, k, g, *rest: fn(w_, d, n, k, g, float(percentile), *rest),
                          w, group_size, sz_dtype, out)


def quantize_pack_int4_sym_mse(w: torch.Tensor, group_size: int, candidates: int = 1000,
                               sz_dtype: torch.dtype = torch.float16,
                               out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Symmetric format, step chosen per group by the MSE search over `candidates` steps."""
    fn = load().quantize_pack_int4_sym_mse
    return _quantize_pack(lambda w_, d, n, k, g, *rest: fn(w_, d, n, k, g, int(candidates), *rest),
                          w, group_size, sz_dtype, out)


def gptq_hessian(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H = X^T X / T + 1e-4 mean(diag) I (float64 [K, K]) from float32 calibration rows X [T, K]."""
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a float32 [T, K] tensor")
    t, k = x.shape
    if out is not None:
        _expect(out, "out", (k, k), (torch.float64,))
    dev = _gpu(x)
    h = torch.empty((k, k), dtype=torch.float64, device=dev) if out is None else out
    _gpu(h)
    _check(load().gptq_hessian(_ptr(x), t, k, _ptr(h), _stream(dev)))
    return h


def gptq_inverse_cholesky(h: torch.Tensor, out: Optional[torch.Tensor] = None, overwrite_h: bool = False,
                          check: bool = True):
    """U (float64 [K, K], upper triangular, U^T U = H^-1).  h is used as the
    factorization's workspace: it is copied first unless overwrite_h.  With
    check, waits for the device status and raises if H is not positive
    definite; otherwise returns (u, info) with info a device int32 tensor."""
    if h.dtype != torch.float64 or h.dim() != 2 or h.shape[0] != h.shape[1]:
        raise ValueError("h must be a square float64 tensor")
    k = h.shape[0]
    if out is not None:
        _expect(out, "out", (k, k), (torch.float64,))
    dev = _gpu(h)
    work = h if overwrite_h else h.clone()
    u = torch.empty((k, k), dtype=torch.float64, device=dev) if out is None else out
    _gpu(u)
    info = torch.empty((1,), dtype=torch.int32, device=dev)
    _check(load().gptq_inverse_cholesky(_ptr(work), k, _ptr(u), _ptr(info), _stream(dev)))
    if not check:
        return u, info
    bad = int(info.item())
    if bad:
        raise ValueError(f"gptq_inverse_cholesky: H is not positive definite (pivot of column {bad - 1})")
    return u


def gptq_quantize_pack_int4(w: torch.Tensor, u: torch.Tensor, group_size: int, symmetric: bool = False,
                            sz_dtype: torch.dtype = torch.float16, overwrite_w: bool = False,
                            out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """GPTQ column sweep of W [N, K] (float32) with U from gptq_inverse_cholesky;
    returns (packed, scales, zeros) in the library's format.  W is copied
    first unless overwrite_w (the sweep uses it as working storage)."""
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a float32 [N, K] tensor")
    if u.dtype != torch.float64 or tuple(u.shape) != (w.shape[1], w.shape[1]):
        raise ValueError("u must be a float64 [K, K] tensor")
    n, k = w.shape
    ng = _ngroups(k, group_size)
    if out is not None:
        _check_out3(out, n, k, ng)
    dev = _gpu(w, u)
    work = w if overwrite_w else w.clone()
    if out is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, k // group_size), dtype=sz_dtype, device=dev)
        zeros = torch.empty((n, k // group_size), dtype=sz_dtype, device=dev)
    else:
        packed, scales, zeros = out
        _gpu(packed, scales, zeros)
    _check(load().gptq_quantize_pack_int4(_ptr(work), _ptr(u), n, k, group_size, int(bool(symmetric)),
                                          _ptr(packed), _ptr(scales), _ptr(zeros),
                                          _dtype_code(scales.dtype), _stream(dev)))
    return packed, scales, zeros


def _check_out3(out, n: int, k: int, ng: int) -> None:
    packed, scales, zeros = out
    _expect(packed, "packed", (n, k // 2), (torch.uint8,))
    _expect(scales, "scales", (n, ng), SZ_DTYPES)
    _expect(zeros, "zeros", (n, ng), (scales.dtype,))


def _quantize_pack(fn, w, group_size, sz_dtype, out):
    n, k = _matrix(w, "w")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"w has dtype {w.dtype}, expected float32 or bfloat16")
    ng = _ngroups(k, group_size)
    if out is not None:
        _check_out3(out, n, k, ng)
    elif sz_dtype not in SZ_DTYPES:
        raise ValueError(f"sz_dtype must be float16 or float32, got {sz_dtype}")
    dev = _gpu(w)
    if out is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, k // group_size), dtype=sz_dtype, device=dev)
        zeros = torch.empty((n, k // group_size), dtype=sz_dtype, device=dev)
    else:
        packed, scales, zeros = out
        _gpu(packed, scales, zeros)
    _check(fn(_ptr(w), _dtype_code(w.dtype), n, k, group_size, _ptr(packed), _ptr(scales),
              _ptr(zeros), _dtype_code(scales.dtype), _stream(dev)))
    return packed, scales, zeros


def dequant_int4(packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, group_size: int,
                 out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """(packed, scales, zeros) -> dequantized W [N, K] in out_dtype."""
    lib = load()
    n, half = _matrix(packed, "packed")
    k = 2 * half
    _check_weights(packed, scales, zeros, k, group_size)
    if out is not None:
        _expect(out, "out", (n, k), tuple(_DT))
    dev = _gpu(packed, scales, zeros)
    w = torch.empty((n, k), dtype=out_dtype, device=dev) if out is None else out
    _gpu(w)
    _check(lib.dequant_int4(_ptr(packed), _ptr(scales), _ptr(zeros), _dtype_code(scales.dtype), n, k,
                            group_size, _ptr(w), _dtype_code(w.dtype), _stream(dev)))
    return w


def quantize_act_int8(x: torch.Tensor, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """x [M, K] (fp32 or bf16) -> (xq int8 [M, K], x_scale float32 [M])."""
    lib = load()
    m, k = _matrix(x, "x")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x has dtype {x.dtype}, expected float32 or bfloat16")
    if out is not None:
        _expect(out[0], "xq", (m, k), (torch.int8,))
        _expect(out[1], "x_scale", (m,), (torch.float32,))
    dev = _gpu(x)
    if out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xs = torch.empty((m,), dtype=torch.float32, device=dev)
    else:
        xq, xs = out
        _gpu(xq, xs)
    _check(lib.quantize_act_int8(_ptr(x), _dtype_code(x.dtype), m, k, _ptr(xq), _ptr(xs), _stream(dev)))
    return xq, xs


def w4a16_matmul_workspace_size(m: int, k: int, n: int, group_size: int,
                                x_dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of workspace with which w4a16_matmul splits K for this shape (0: none)."""
    return int(load().w4a16_matmul_workspace_size(m, k, n, group_size, _dtype_code(x_dtype)))


def w4a16_matmul(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 group_size: int, out_dtype: Optional[torch.dtype] = None,
                 out: Optional[torch.Tensor] = None, workspace="auto"):
    """y [M, N] = x [M, K] . dequant(W)^T; out_dtype defaults to x's dtype.

    workspace: "auto" (default) allocates, through torch, the workspace the
    library asks for on this shape (none for most shapes) and calls
    w4a16_matmul_ws; a uint8 device tensor is used as given; None calls
    w4a16_matmul, which uses none."""
    lib = load()
    m, k = _matrix(x, "x")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x has dtype {x.dtype}, expected float32 or bfloat16")
    if _matrix(packed, "packed")[1] * 2 != k:
        raise ValueError(f"packed has {packed.shape[1] * 2} columns of codes, x has K={k}")
    n = _check_weights(packed, scales, zeros, k, group_size)
    if out is not None:
        _expect(out, "out", (m, n), (torch.float32, torch.bfloat16))
    dev = _gpu(x, packed, scales, zeros)
    y = torch.empty((m, n), dtype=out_dtype or x.dtype, device=dev) if out is None else out
    _gpu(y)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 tensor')
        nbytes = int(lib.w4a16_matmul_workspace_size(m, k, n, group_size, _dtype_code(x.dtype)))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev) if nbytes else None
    args = (_ptr(x), _dtype_code(x.dtype), m, k, _ptr(packed), _ptr(scales), _ptr(zeros),
            _dtype_code(scales.dtype), n, group_size, _ptr(y), _dtype_code(y.dtype))
    if workspace is None:
        _check(lib.w4a16_matmul(*args, _stream(dev)))
    else:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        _gpu(workspace)
        _check(lib.w4a16_matmul_ws(*args, _ptr(workspace), workspace.numel(), _stream(dev)))
    return y


def w4a8_matmul_workspace_size(m: int, k: int, n: int, group_size: int) -> int:
    """Bytes of workspace with which w4a8_matmul splits K for this shape (0: none)."""
    return int(load().w4a8_matmul_workspace_size(m, k, n, group_size))


def w4a8_matmul(xq: torch.Tensor, x_scale: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                zeros: torch.Tensor, group_size: int, out_dtype: torch.dtype = torch.bfloat16,
                out: Optional[torch.Tensor] = None, workspace="auto"):
    """y [M, N] = x_scale[m] * (xq [M, K] . dequant(W)^T).

    workspace: "auto" (default) allocates, through torch, the workspace the
    library asks for on this shape (none for most shapes) and calls
    w4a8_matmul_ws; a uint8 device tensor is used as given; None calls
    w4a8_matmul, which uses none."""
    lib = load()
    m, k = _matrix(xq, "xq")
    _expect(xq, "xq", (m, k), (torch.int8,))
    _expect(x_scale, "x_scale", (m,), (torch.float32,))
    if _matrix(packed, "packed")[1] * 2 != k:
        raise ValueError(f"packed has {packed.shape[1] * 2} columns of codes, xq has K={k}")
    n = _check_weights(packed, scales, zeros, k, group_size)
    if out is not None:
        _expect(out, "out", (m, n), (torch.float32, torch.bfloat16))
    dev = _gpu(xq, x_scale, packed, scales, zeros)
    y = torch.empty((m, n), dtype=out_dtype, device=dev) if out is None else out
    _gpu(y)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 tensor')
        nbytes = int(lib.w4a8_matmul_workspace_size(m, k, n, group_size))
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev) if nbytes else None
    args = (_ptr(xq), _ptr(x_scale), m, k, _ptr(packed), _ptr(scales), _ptr(zeros),
            _dtype_code(scales.dtype), n, group_size, _ptr(y), _dtype_code(y.dtype))
    if workspace is None:
        _check(lib.w4a8_matmul(*args, _stream(dev)))
    else:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        _gpu(workspace)
        _check(lib.w4a8_matmul_ws(*args, _ptr(workspace), workspace.numel(), _stream(dev)))
    return y


def version() -> str:
    return load().w4_version().decode()
