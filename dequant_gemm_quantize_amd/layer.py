"""PyTorch layer over the library: a drop-in for a bias-free nn.Linear whose
weight is stored as group-wise INT4 codes and multiplied by the fused
dequantize-matmul ("Building a From-Scratch Group-Wise INT4 Quantization
Layer for LLaMA Weights", Step 3: the quantized linear layer; Step 5: the
replacement pass over a model).

Every numeric step runs in the HIP kernels behind libw4.so: quantization at
construction (asymmetric, symmetric, symmetric with a percentile or MSE
calibrated scale, or GPTQ with calibration activations), the product in forward (W4A16, or W4A8 with per-token
INT8 activations).  This module only reshapes tensors and keeps the buffers.
"""
from __future__ import annotations

from typing import Callable, Optional

import torch

from . import _lib

QUANTIZERS = {
    "asym": lambda w, g, sz, p: _lib.quantize_pack_int4(w, g, sz),
    "sym": lambda w, g, sz, p: _lib.quantize_pack_int4_sym(w, g, sz),
    "percentile": lambda w, g, sz, p: _lib.quantize_pack_int4_sym_percentile(w, g, 99.9 if p is None else p, sz),
    "mse": lambda w, g, sz, p: _lib.quantize_pack_int4_sym_mse(w, g, 1000 if p is None else int(p), sz),
    "gptq": lambda w, g, sz, p: _gptq(w, g, sz, p, False),
    "gptq_sym": lambda w, g, sz, p: _gptq(w, g, sz, p, True),
}


def _gptq(w: torch.Tensor, g: int, sz: torch.dtype, x: Optional[torch.Tensor], symmetric: bool):
    """GPTQ ([P4] Step 3) with calibration rows x [T, in_features] (float32,
    on the weight's GPU): Hessian, inverse Cholesky factor, column sweep."""
    if x is None:
        raise ValueError("GPTQ modes need the calibration rows X [T, in_features] as param")
    h = _lib.gptq_hessian(x.reshape(-1, x.shape[-1]).to(torch.float32).contiguous())
    u = _lib.gptq_inverse_cholesky(h, overwrite_h=True)
    # The sweep uses its weight argument as working storage.  A float32
    # contiguous weight converts to itself, so the sweep may take it over
    # only when the conversion made a copy; otherwise the wrapper copies it
    # and the caller's weight (possibly a tied parameter) is left unchanged.
    wf = w.to(torch.float32).contiguous()
    owned = wf.data_ptr() != w.data_ptr()
    return _lib.gptq_quantize_pack_int4(wf, u, g, symmetric, sz, overwrite_w=owned)


class QuantizedLinear(torch.nn.Module):
    """y = x . dequant(Wq)^T with W [out_features, in_features] held as packed
    INT4 codes [N, K/2], scales and zero-points [N, K/g].

    forward(x): x [..., in_features] in bf16 or fp32 on the weight's GPU;
    returns [..., out_features] in ``out_dtype`` (default: x's dtype).  With
    ``act_int8=True`` the activations are quantized per token to INT8 first
    and the W4A8 product is used (bf16 output)."""

    def __init__(self, in_features: int, out_features: int, group_size: int = 128,
                 scale_dtype: torch.dtype = torch.float16, act_int8: bool = False,
                 out_dtype: Optional[torch.dtype] = None, device=None):
        super().__init__()
        if in_features % group_size or group_size % 32:
            raise ValueError("in_features must be a multiple of group_size, itself a multiple of 32")
        self.in_features = in_features
        self.out_features = out_features
        self.group_size = group_size
        self.act_int8 = act_int8
        self.out_dtype = out_dtype
        ng = in_features // group_size
        self.register_buffer("packed", torch.zeros((out_features, in_features // 2), dtype=torch.uint8,
                                                   device=device))
        self.register_buffer("scales", torch.ones((out_features, ng), dtype=scale_dtype, device=device))
        self.register_buffer("zeros", torch.zeros((out_features, ng), dtype=scale_dtype, device=device))

    @classmethod
    def from_weight(cls, weight: torch.Tensor, group_size: int = 128, mode: str = "asym",
                    param=None, scale_dtype: torch.dtype = torch.float16, act_int8: bool = False,
                    out_dtype: Optional[torch.dtype] = None) -> "QuantizedLinear":
        """Quantize W [out, in] (bf16 or fp32, on the GPU) with ``mode`` in
        asym / sym / percentile (param: p, default 99.9) / mse (param:
        candidates, default 1000) / gptq or gptq_sym (param: calibration
        rows X [T, in], required)."""
        if mode not in QUANTIZERS:
            raise ValueError(f"mode must be one of {sorted(QUANTIZERS)}")
        n, k = weight.shape
        layer = cls(k, n, group_size, scale_dtype, act_int8, out_dtype, device=weight.device)
        w = weight.detach()
        if w.dtype not in (torch.bfloat16, torch.float32):
            w = w.to(torch.float32)
        p, s, z = QUANTIZERS[mode](w.contiguous(), group_size, scale_dtype, param)
        layer.packed.copy_(p)
        layer.scales.copy_(s)
        layer.zeros.copy_(z)
        return layer

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, **kw) -> "QuantizedLinear":
        if linear.bias is not None:
            raise ValueError("QuantizedLinear has no bias; the linear layer has one")
        return cls.from_weight(linear.weight, **kw)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"x has {x.shape[-1]} features, the layer takes {self.in_features}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        if self.act_int8:
            xq, xs = _lib.quantize_act_int8(x2)
            y = _lib.w4a8_matmul(xq, xs, self.packed, self.scales, self.zeros, self.group_size,
                                 out_dtype=self.out_dtype or torch.bfloat16)
        else:
            y = _lib.w4a16_matmul(x2, self.packed, self.scales, self.zeros, self.group_size,
                                  out_dtype=self.out_dtype or x.dtype)
        return y.reshape(*lead, self.out_features)

    def dequantize(self, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
        """The dense weight (q - zp) * scale, for inspection."""
        return _lib.dequant_int4(self.packed, self.scales, self.zeros, self.group_size, out_dtype=dtype)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"group_size={self.group_size}, act_int8={self.act_int8}")


def replace_linears(module: torch.nn.Module, group_size: int = 128, mode: str = "asym",
                    skip: Optional[Callable[[str, torch.nn.Linear], bool]] = None, **kw) -> torch.nn.Module:
    """Replace, in place and recursively, every bias-free nn.Linear whose
    in_features is a multiple of group_size by a QuantizedLinear of its
    weight.  ``skip(name, layer)`` can keep chosen layers dense."""
    for name, child in list(module.named_children()):
        if isinstance(child, torch.nn.Linear):
            if child.bias is None and child.in_features % group_size == 0 and not (skip and skip(name, child)):
                setattr(module, name, QuantizedLinear.from_linear(child, group_size=group_size, mode=mode, **kw))
        else:
            replace_linears(child, group_size, mode, skip, **kw)
    return module
