"""Helpers for the GPU parity tests: host <-> device copies and canaries.

Nothing here computes any part of the method; it only moves data.
"""
from __future__ import annotations

import numpy as np
import torch

TORCH_SZ = {"f16": torch.float16, "f32": torch.float32}


def to_dev(a: np.ndarray, kind: str) -> torch.Tensor:
    """NumPy array (bf16 given as uint16 bits) -> contiguous cuda tensor."""
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).cuda()
    if kind == "f16":
        return torch.from_numpy(a.astype(np.float16, copy=False)).cuda()
    if kind in ("u8", "i8"):
        return torch.from_numpy(a).cuda()
    raise ValueError(kind)


def to_host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> NumPy (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit view for bit-exact comparisons."""
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def y_as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Canary:
    """A device buffer with guard bytes before and after the region handed to
    a kernel; check() asserts the guards are untouched."""

    PAD = 256
    FILL = 0xA5

    def __init__(self, shape, dtype):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((nbytes + 2 * self.PAD,), self.FILL, dtype=torch.uint8, device="cuda")
        self.nbytes = nbytes
        self.tensor = self.raw[self.PAD:self.PAD + nbytes].view(dtype).view(*shape)

    def check(self):
        torch.cuda.synchronize()
        head = self.raw[:self.PAD].cpu().numpy()
        tail = self.raw[self.PAD + self.nbytes:].cpu().numpy()
        assert (head == self.FILL).all(), "write before the output buffer"
        assert (tail == self.FILL).all(), "write past the output buffer"
