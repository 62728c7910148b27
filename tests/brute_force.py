"""Brute-force per-element twins of the oracle, for tiny inputs only.

Written independently of oracle/w4_oracle.py: Python loops over single
elements, each arithmetic step a NumPy float32 *scalar* operation (IEEE
single precision, round to nearest even) and Python's round() (ties to even)
for the integer decisions.  The vectorised oracle must agree bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

from tests import page_calibrators as PC

f32 = np.float32


def _rint(v) -> int:
    # Python's round() on a float rounds half to even; float(v) of a float32
    # is exact, so this is the float32 value's nearest-even integer.
    return int(round(float(v)))


def _clamp(i: int, lo: int, hi: int) -> int:
    return lo if i < lo else hi if i > hi else i


def quantize_group(vals, sz: str):
    """One group: list of float32 values -> (stored scale, zp int, codes)."""
    mn = vals[0]
    mx = vals[0]
    for v in vals[1:]:
        if v < mn:
            mn = v
        if v > mx:
            mx = v
    s32 = f32(f32(mx - mn) / f32(15.0))
    stored = np.float16(s32) if sz == "f16" else f32(s32)
    if float(stored) == 0.0:
        stored = np.float16(1.0) if sz == "f16" else f32(1.0)
    s = f32(stored)
    zp = _clamp(_rint(f32(f32(-mn) / s)), 0, 15)
    codes = []
    for v in vals:
        t = f32(f32(v / s) + f32(zp))
        codes.append(_clamp(_rint(t), 0, 15))
    return stored, zp, codes


def quantize_pack(w32: np.ndarray, g: int, sz: str):
    """W [N,K] float32 -> (packed bytes, scales, zeros) by per-element loops."""
    n, k = w32.shape
    ng = k // g
    sdt = np.float16 if sz == "f16" else np.float32
    packed = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, ng), sdt)
    zeros = np.zeros((n, ng), sdt)
    for r in range(n):
        codes_row = []
        for gi in range(ng):
            vals = [f32(w32[r, gi * g + t]) for t in range(g)]
            st, zp, codes = quantize_group(vals, sz)
            scales[r, gi] = st
            zeros[r, gi] = zp
            codes_row.extend(codes)
        for j in range(k // 2):
            packed[r, j] = codes_row[2 * j] + 16 * codes_row[2 * j + 1]
    return packed, scales, zeros


def quantize_group_sym(vals, sz: str):
    """One group, symmetric: list of float32 values -> (stored scale, codes
    0..15 holding the signed code + 8)."""
    amax = f32(0.0)
    for v in vals:
        a = f32(abs(v))
        if a > amax:
            amax = a
    s32 = f32(amax / f32(7.0))
    stored = np.float16(s32) if sz == "f16" else f32(s32)
    if float(stored) == 0.0:
        stored = np.float16(1.0) if sz == "f16" else f32(1.0)
    s = f32(stored)
    return stored, [_clamp(_rint(f32(v / s)), -8, 7) + 8 for v in vals]


def quantize_pack_sym(w32: np.ndarray, g: int, sz: str):
    """Symmetric W [N,K] float32 -> (packed bytes, scales, zeros = 8)."""
    n, k = w32.shape
    ng = k // g
    sdt = np.float16 if sz == "f16" else np.float32
    packed = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, ng), sdt)
    zeros = np.zeros((n, ng), sdt)
    for r in range(n):
        codes_row = []
        for gi in range(ng):
            st, codes = quantize_group_sym([f32(w32[r, gi * g + t]) for t in range(g)], sz)
            scales[r, gi] = st
            zeros[r, gi] = 8
            codes_row.extend(codes)
        for j in range(k // 2):
            packed[r, j] = codes_row[2 * j] + 16 * codes_row[2 * j + 1]
    return packed, scales, zeros


def quantize_pack_calibrated(w32: np.ndarray, g: int, sz: str, method: str, param):
    """Symmetric codes with a calibrated scale ("percentile" range / 7, or the
    "mse" step), element by element; the range or step of each group comes
    from the page's own torch calls, one group at a time."""
    n, k = w32.shape
    ng = k // g
    sdt = np.float16 if sz == "f16" else np.float32
    packed = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, ng), sdt)
    zeros = np.full((n, ng), 8, sdt)
    for r in range(n):
        codes_row = []
        for gi in range(ng):
            vals = [f32(w32[r, gi * g + t]) for t in range(g)]
            if method == "percentile":
                step = f32(PC.percentile(vals, param) / f32(7.0))
            else:
                step = PC.mse_search(vals, param)
            stored = sdt(step)
            if float(stored) == 0.0:
                stored = sdt(1.0)
            s = f32(stored)
            scales[r, gi] = stored
            codes_row.extend(_clamp(_rint(f32(v / s)), -8, 7) + 8 for v in vals)
        for j in range(k // 2):
            packed[r, j] = codes_row[2 * j] + 16 * codes_row[2 * j + 1]
    return packed, scales, zeros


def dequant(packed, scales, zeros, g: int) -> np.ndarray:
    """w_hat[r, c] = fl32((code - zp) * scale), element by element."""
    n, half = packed.shape
    k = 2 * half
    out = np.zeros((n, k), np.float32)
    for r in range(n):
        for c in range(k):
            byte = int(packed[r, c // 2])
            code = byte % 16 if c % 2 == 0 else byte // 16
            zp = int(float(zeros[r, c // g]))
            s = f32(scales[r, c // g])
            out[r, c] = f32(f32(code - zp) * s)
    return out


def act_quant(x32: np.ndarray):
    m, k = x32.shape
    xq = np.zeros((m, k), np.int8)
    sa = np.zeros(m, np.float32)
    for r in range(m):
        amax = f32(0.0)
        for c in range(k):
            a = f32(abs(x32[r, c]))
            if a > amax:
                amax = a
        floor = f32(1e-8)
        s = f32((amax if amax > floor else floor) / f32(127.0))
        sa[r] = s
        for c in range(k):
            xq[r, c] = _clamp(_rint(f32(x32[r, c] / s)), -128, 127)
    return xq, sa


def dot_exact(xrow, wrow) -> float:
    """Correctly rounded float64 dot product (math.fsum of exact products)."""
    return math.fsum(float(a) * float(b) for a, b in zip(xrow, wrow))
