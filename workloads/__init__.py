"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws random numbers and rounds them to the storage dtype of
the workload; it holds none of the quantization or matmul arithmetic, so both
the oracle and the HIP path can take their inputs from here without sharing
any of the method's code.

Recipe (the pages measure on no public dataset; the Llama-7B / 70B-MLP
shapes stand in for the real checkpoints named on "Building a From-Scratch
Group-Wise INT4 Quantization Layer for LLaMA Weights", Running and Testing It):

* every tensor is drawn with ``numpy.random.default_rng(seed)`` (PCG64), as the
  demos on "Build a GPTQ INT4 Quantization Engine in Python/NumPy" (The demo)
  and "Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
  Per-channel Scales" (Step 1) do;
* normal draws are taken in float64 with ``rng.normal(0, sigma, shape)`` and
  cast to float32, then rounded to bfloat16 (round-to-nearest-even) where the
  workload is bf16;
* "outliers" replace ``round(0.001 * N * K)`` distinct weights, picked with
  ``rng.choice(N*K, count, replace=False)``, by +-0.5 with a sign drawn from
  ``rng.integers(0, 2, count)``;
* heavy-tailed activation channels multiply 5% of the K columns (the same
  columns for every token, ``rng.choice(K, round(0.05*K), replace=False)``)
  by 20 before the bf16 rounding.

bf16 tensors are carried as ``uint16`` bit patterns in NumPy (NumPy has no
bfloat16); ``Tensor.kind`` says how to read them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "Tensor", "weight", "activation", "CONFIGS", "WEIGHTS", "config_cases",
    "bf16_round_bits", "bits_as_f32",
]


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Used only to put synthetic draws into the workload's storage dtype.
    Inputs here are finite draws, so NaN handling is not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bits_as_f32(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A synthetic tensor: ``data`` holds float32 values or bf16 bits."""
    data: np.ndarray
    kind: str          # "f32" or "bf16"

    @property
    def shape(self) -> Tuple[int, ...]:
        return tuple(self.data.shape)

    def as_f32(self) -> np.ndarray:
        """Exact float32 view of the stored values."""
        if self.kind == "f32":
            return self.data
        return bits_as_f32(self.data)


# --------------------------------------------------------------------------
# Weights.  name -> (seed, N, K, sigma, outliers, kind)
# --------------------------------------------------------------------------
WEIGHTS: Dict[str, Tuple[int, int, int, float, bool, str]] = {
    # 256x256 fp32 single layer; the activation is drawn from the same stream.
    "W1": (0, 256, 256, 0.02, False, "f32"),
    # Llama-7B attention projection [4096, 4096].
    "Wa": (1, 4096, 4096, 0.02, True, "bf16"),
    # Llama-7B MLP up/gate projection [11008, 4096].
    "Wb": (2, 11008, 4096, 0.02, True, "bf16"),
    # Llama-7B MLP down projection [4096, 11008].
    "Wd": (3, 4096, 11008, 0.02, True, "bf16"),
    # 70B-class MLP projection [28672, 8192].
    "We": (4, 28672, 8192, 0.015, False, "bf16"),
}


def _draw_weight(rng: np.random.Generator, n: int, k: int, sigma: float, outliers: bool) -> np.ndarray:
    w = rng.normal(0.0, sigma, size=(n, k)).astype(np.float32)
    if outliers:
        count = int(round(0.001 * n * k))
        pos = rng.choice(n * k, size=count, replace=False)
        sign = 2 * rng.integers(0, 2, size=count) - 1
        w.reshape(-1)[pos] = (0.5 * sign).astype(np.float32)
    return w


_CACHE: Dict[str, Tensor] = {}


def weight(name: str, rows: int | None = None, cache: bool = False) -> Tensor:
    """The named synthetic weight ``[N, K]``.

    ``rows`` keeps only the first ``rows`` rows (the stream is still drawn in
    full so the values equal those of the whole tensor).
    """
    if cache and name in _CACHE and rows is None:
        return _CACHE[name]
    seed, n, k, sigma, outl, kind = WEIGHTS[name]
    rng = np.random.default_rng(seed)
    w = _draw_weight(rng, n, k, sigma, outl)
    if rows is not None:
        w = np.ascontiguousarray(w[:rows])
    t = Tensor(w if kind == "f32" else bf16_round_bits(w), kind)
    if cache and rows is None:
        _CACHE[name] = t
    return t


def activation(cfg: int, m: int, k: int) -> Tensor:
    """Activation ``x [M, K]`` for workload ``cfg`` (1..5).

    cfg 1: x ~ N(0,1) fp32, drawn from the weight's own rng(0) stream after W.
    cfg 2/3: x ~ N(0,1) bf16 from rng(100 + M).
    cfg 4: x ~ N(0,1) bf16 from rng(2048) for K=4096, rng(2049) for K=11008.
    cfg 5: x ~ N(0,1), 5% of columns x20, bf16, from rng(500 + M).
    """
    if cfg == 1:
        seed, n, kk, sigma, outl, _ = WEIGHTS["W1"]
        assert k == kk
        rng = np.random.default_rng(seed)
        _draw_weight(rng, n, kk, sigma, outl)
        x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
        return Tensor(x, "f32")
    if cfg in (2, 3):
        rng = np.random.default_rng(100 + m)
        x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
        return Tensor(bf16_round_bits(x), "bf16")
    if cfg == 4:
        rng = np.random.default_rng(2048 if k == 4096 else 2049)
        x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
        return Tensor(bf16_round_bits(x), "bf16")
    if cfg == 5:
        rng = np.random.default_rng(500 + m)
        x = rng.normal(0.0, 1.0, size=(m, k)).astype(np.float32)
        cols = rng.choice(k, size=int(round(0.05 * k)), replace=False)
        x[:, cols] *= np.float32(20.0)
        return Tensor(bf16_round_bits(x), "bf16")
    raise ValueError(f"unknown workload {cfg}")


# --------------------------------------------------------------------------
# The five workloads: (weight names, M values, group size, scale dtype,
# activation/output dtype, path).
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(weights=["W1"], ms=[1], group=32, sz="f32", xy="f32", path="w4a16",
            desc="single 256x256 fp32 layer, g=32, fp32 x and y"),
    2: dict(weights=["Wa", "Wb"], ms=[1], group=128, sz="f16", xy="bf16", path="w4a16",
            desc="Llama-7B decode GEMV, M=1"),
    3: dict(weights=["Wa", "Wb"], ms=[4, 8, 16, 32], group=128, sz="f16", xy="bf16", path="w4a16",
            desc="Llama-7B small batch, GEMV/MFMA switch"),
    4: dict(weights=["Wb", "Wd"], ms=[2048], group=128, sz="f16", xy="bf16", path="w4a16",
            desc="Llama-7B prefill GEMM, M=2048"),
    5: dict(weights=["We"], ms=[1, 512], group=128, sz="f16", xy="bf16", path="w4a8",
            desc="W4A8 70B-MLP projection, per-token int8 activations"),
}


def config_cases(cfg: int):
    """Yield (weight_name, M, K, N) for every matmul of workload ``cfg``."""
    c = CONFIGS[cfg]
    for wname in c["weights"]:
        _, n, k, _, _, _ = WEIGHTS[wname]
        for m in c["ms"]:
            yield wname, m, k, n
