"""CPU oracle for GPTQ-style second-order INT4 quantization.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path never calls
it and shares no code with it.

Page: [P4] "Build a GPTQ INT4 Quantization Engine in Python/NumPy", Step 3
("GPTQ-style second-order calibration"), with its tests section for the
comparison against round-to-nearest.

What Step 3 fixes, and the readings taken where its listing is garbled (the
listing sweeps weight *rows* with an in_features x in_features matrix, which
only type-checks for square weights; the prose says columns):
  * Hessian H = X^T X / T over T calibration rows of X [T, K], plus a damping
    of 1e-4 * mean(diag(X^T X / T)) on the diagonal.  The prose's factor 2 is
    dropped, as in the listing: it scales H, the damping scales with it, and
    the updates below are invariant to the scale of H.
  * U is the upper-triangular Cholesky factor of H^-1 (U^T U = H^-1, positive
    diagonal): "the upper-triangular form" of the Cholesky of the inverse.
  * Columns are processed left to right.  Column i is quantized; its error
    e = (w_i - w_hat_i) / U[i, i] is propagated into every later column j of
    the same row as w_j -= e * U[i, j].  Rows are independent.
  * Group parameters: a group (g consecutive columns of a row, the format of
    the rest of the library) takes its scale and zero-point when the sweep
    reaches its first column, from the group's current (error-compensated)
    values, with the same formulas as round-to-nearest: asymmetric
    (max - min)/15 with zero-point, or symmetric absmax/7 with codes +-8
    stored with the +8 offset.  This replaces the listing's final "re-quantize
    per group" pass, which re-rounds codes that were already integers.
  * Precision: the working values and the error propagation are float64;
    each integer decision (code, zero-point) is taken in float32 on the
    float32 rounding of the working value, with the same IEEE float32 steps
    as the plain quantizer.  The dequantized value used for the error is
    (q - zp) * scale, exact in float64.

Parity pins: tests/gptq_pins.py (closed form of the compensated values,
U H U^T = I, brute-force Hessian, reduction to round-to-nearest for a
diagonal Hessian, the page's comparison against round-to-nearest); none of
these functions is "parity unpinned".

``gptq_quantize`` also serves as the checker of another implementation's
output: given its codes and group parameters as a ``guide``, it replays the
sweep, accepts a differing decision only where its own float64 decision
variable lies within ``tol`` of the rounding boundary between the two (or a
scale within ``scale_rtol``), continues with the guide's choice, and counts
such acceptances (codes, zero-points; a float32 scale is continuous in the
values, so scales are only held to the tolerance); any other difference
raises.
"""
from __future__ import annotations

import numpy as np

from . import w4_oracle as W

F32 = np.float32
F64 = np.float64
DAMP = 1e-4


def gptq_hessian(x) -> np.ndarray:
    """H = X^T X / T + 1e-4 * mean(diag(X^T X / T)) * I in float64, from
    float32 calibration rows X [T, K] ([P4] Step 3, compute_hessian)."""
    x64 = np.asarray(x, F32).astype(F64)
    t = x64.shape[0]
    h = (x64.T @ x64) / t
    h = h + DAMP * np.mean(np.diag(h)) * np.eye(h.shape[0])
    return h


def gptq_inverse_cholesky(h) -> np.ndarray:
    """U upper triangular with U^T U = H^-1 ([P4] Step 3): the inverse, then
    its Cholesky factor L (L L^T = H^-1), and U = L^T."""
    hinv = np.linalg.inv(np.asarray(h, F64))
    hinv = (hinv + hinv.T) / 2          # symmetric to the last bit for cholesky
    return np.linalg.cholesky(hinv).T


def group_params(vals32: np.ndarray, symmetric: bool, sz: str):
    """Scale (storage dtype) and zero-point (int) of one group per row, from
    its float32 values [R, g]: the round-to-nearest formulas of the library's
    format (asymmetric or symmetric)."""
    if symmetric:
        s_st = W.scale_sym(np.abs(vals32).max(axis=1), sz)
        return s_st, np.full(s_st.shape, W.SYM_OFFSET, np.int32)
    return W.scale_zero(vals32.min(axis=1), vals32.max(axis=1), sz)


def _decide(v32, s, zp, symmetric):
    """float32 decision variable and stored code of one column."""
    if symmetric:
        t = v32 / s
        return t, (np.clip(np.rint(t), -8, 7) + W.SYM_OFFSET).astype(np.int32)
    t = v32 / s + zp.astype(F32)
    return t, np.clip(np.rint(t), 0, 15).astype(np.int32)


def gptq_quantize(w, u, g: int, sz: str, symmetric: bool, guide=None, tol: float = 1e-3,
                  scale_rtol=None, trace: bool = False):
    """The column sweep over W [N, K] (float32 values) with U [K, K].

    Returns (codes uint8 [N, K], scales [N, K/g] sz dtype, zeros [N, K/g] sz
    dtype, stats, trace) where trace[i] (if asked) holds the float64 working
    values of column i just before it is quantized."""
    w64 = np.asarray(w, F32).astype(F64).copy()
    u = np.asarray(u, F64)
    n, k = w64.shape
    if k % g:
        raise ValueError("K must be a multiple of g")
    sd = W.SZ_DTYPES[sz]
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // g), sd)
    zeros = np.zeros((n, k // g), np.int32)
    stats = {"codes_accepted": 0, "zeros_accepted": 0, "scales_differing": 0}
    if scale_rtol is None:                 # about one unit in the last place of the stored scale
        scale_rtol = 2e-3 if sz == "f16" else 1e-5
    tr = np.zeros((n, k)) if trace else None
    s = zp = None
    if guide is not None:
        g_codes = W.unpack_nibbles(guide[0]).astype(np.int32)
        g_s = np.asarray(guide[1])
        g_z = np.asarray(guide[2]).astype(F32).astype(np.int32)
    for i in range(k):
        if i % g == 0:
            j = i // g
            vals32 = w64[:, i:i + g].astype(F32)
            s_st, zpo = group_params(vals32, symmetric, sz)
            if guide is not None:
                s_st, zpo = _accept_params(vals32, w64[:, i:i + g], s_st, zpo, g_s[:, j], g_z[:, j],
                                           symmetric, sz, tol, scale_rtol, stats, i)
            scales[:, j] = s_st
            zeros[:, j] = zpo
            s = s_st.astype(F32)
            zp = zpo
        if trace:
            tr[:, i] = w64[:, i]
        v32 = w64[:, i].astype(F32)
        t, q = _decide(v32, s, zp, symmetric)
        if guide is not None:
            q = _accept_codes(w64[:, i], s, zp, q, g_codes[:, i], symmetric, tol, stats, i)
        codes[:, i] = q
        zq = zp if not symmetric else np.full(n, W.SYM_OFFSET)
        dq = (q.astype(F64) - zq.astype(F64)) * s.astype(F64)
        err = (w64[:, i] - dq) / u[i, i]
        w64[:, i + 1:] -= err[:, None] * u[i, i + 1:][None, :]
    return codes, scales, zeros.astype(sd), stats, tr


def _accept_codes(w_col64, s, zp, q, qg, symmetric, tol, stats, i):
    bad = np.nonzero(q != qg)[0]
    if bad.size == 0:
        return q
    t64 = w_col64[bad] / s[bad].astype(F64)
    if not symmetric:
        t64 = t64 + zp[bad]
    else:
        t64 = t64 + W.SYM_OFFSET
    bound = (q[bad] + qg[bad]) / 2.0
    ok = (np.abs(q[bad] - qg[bad]) == 1) & (np.abs(t64 - bound) <= tol)
    if not ok.all():
        r = bad[~ok][0]
        raise AssertionError(f"column {i} row {r}: code {qg[r]} where {q[r]} is due "
                             f"(decision variable {w_col64[r] / float(s[r]):.6f})")
    stats["codes_accepted"] += int(bad.size)
    q = q.copy()
    q[bad] = qg[bad]
    return q


def _accept_params(vals32, vals64, s_st, zpo, s_g, z_g, symmetric, sz, tol, rtol, stats, i):
    sd = W.SZ_DTYPES[sz]
    s_g = s_g.astype(sd)
    diff_s = s_st != s_g
    if diff_s.any():
        a = s_st[diff_s].astype(F64)
        b = s_g[diff_s].astype(F64)
        if not (np.abs(a - b) <= rtol * np.abs(a)).all():
            raise AssertionError(f"group at column {i}: scale outside tolerance")
        stats["scales_differing"] += int(diff_s.sum())
    s32 = s_g.astype(F32)
    if symmetric:
        if not (z_g == W.SYM_OFFSET).all():
            raise AssertionError(f"group at column {i}: symmetric zero-point is not 8")
        return s_g, z_g
    mn64 = vals64.min(axis=1)
    zp_due = np.clip(np.rint(-vals32.min(axis=1) / s32), 0, 15).astype(np.int32)
    bad = np.nonzero(zp_due != z_g)[0]
    if bad.size:
        t64 = -mn64[bad] / s32[bad].astype(F64)
        bound = (zp_due[bad] + z_g[bad]) / 2.0
        if not ((np.abs(zp_due[bad] - z_g[bad]) == 1) & (np.abs(t64 - bound) <= tol)).all():
            raise AssertionError(f"group at column {i}: zero-point outside tolerance")
        stats["zeros_accepted"] += int(bad.size)
    return s_g, z_g


def gptq_quantize_pack_int4(w, kind: str, u, g: int, sz: str, symmetric: bool = False):
    """GPTQ quantize + pack of W [N, K] with U from gptq_inverse_cholesky:
    (packed uint8 [N, K/2], scales, zeros) in the library's format."""
    codes, scales, zeros, _, _ = gptq_quantize(W.as_f32(w, kind), u, g, sz, symmetric)
    return W.pack_nibbles(codes), scales, zeros


def proxy_loss(w, w_hat, h) -> float:
    """sum over rows of (w - w_hat) H (w - w_hat)^T: the layer-output error
    ||X W^T - X W_hat^T||^2 / T that the sweep minimizes greedily."""
    d = np.asarray(w, F64) - np.asarray(w_hat, F64)
    return float(np.einsum("nk,kl,nl->", d, np.asarray(h, F64), d))
