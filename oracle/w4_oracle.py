"""CPU oracle for group-wise asymmetric INT4 quantization and dequantize-matmul.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Plain NumPy, written to be checked against the pages by eye.  Every
quantization step is a single IEEE-754 float32 operation with
round-to-nearest-even, so that the integer decisions (codes, zero-points)
are taken in the same precision as the GPU kernels; the matmul references
are exact-input float64.

Pages cited (martinuke0.github.io posts):
  [P1] "Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
       Per-channel Scales"
  [P2] "From-scratch INT4 Weight-only Quantizer with Per-group Scales and
       Zero-points for LLMs"
  [P3] "Building a From-Scratch Group-Wise INT4 Quantization Layer for LLaMA
       Weights"
  [P4] "Build a GPTQ INT4 Quantization Engine in Python/NumPy"
  [P5] "From Scratch: Building a GPTQ INT4 Quantizer in Pure Python"

Readings taken where the pages disagree or are silent (each is pinned by a
test in tests/test_oracle_pins.py):
  * groups are runs of ``g`` consecutive columns (in_features) of one row
    ([P1] Architecture Overview; [P2] Architecture Overview, "Group Divisor");
  * scale = (max - min) / 15 and zero-point = clamp(round(-min/scale), 0, 15)
    ([P2] Architecture Overview and Step 6), computed with the scale as
    stored (fp16 or fp32), a stored scale of 0 replaced by 1 ([P4] Step 2);
  * code q = clamp(round(w/scale + zp), 0, 15) ([P5] Step 2), round half to
    even; dequantized weight (q - zp) * scale ([P5] Step 4);
  * two codes per byte, the even column in the low nibble ([P4] Step 4;
    [P3] Step 1);
  * symmetric variant: scale = absmax/7 and code clamp(round(w/scale), -8, 7)
    ([P4] Step 2), stored with the +8 offset of [P4] Step 4, i.e. a fixed
    zero-point of 8; same stored-scale and zero-guard readings as above;
  * calibrated symmetric scales ([P3] Step 4): the range is the p-th
    percentile of |w| as torch.quantile computes it in float32, or the step
    is the one the MSE search picks among torch.linspace(min|w|, max|w|, n)
    (codes round(w / c) in float32 clamped to +-7 during the search, the
    mean of the squared errors, first minimum wins); the codes are then the
    symmetric ones with the stored scale;
  * per-token activation scale max(max|x|, 1e-8)/127 and
    clamp(round(x/s), -128, 127) ([P1] Step 3);
  * matmul y = x . dequant(W)^T ([P3] Step 2; [P4] Step 5), and for the
    INT8-activation variant y = s_a * (x_int8 . dequant(W)^T) ([P1] Step 5).

Parity pins: every function here is pinned (see tests/test_oracle_pins.py);
none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F16 = np.float16

SZ_DTYPES = {"f32": np.float32, "f16": np.float16}


# --------------------------------------------------------------------------
# Representations.  bf16 has no NumPy dtype, so bf16 tensors are uint16 bits.
# --------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32: a bf16 number is the top half of an fp32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (finite input).

    Drops the low 16 bits of the fp32 pattern after adding half an ulp of the
    result (0x7FFF plus the result's lowest kept bit, which breaks ties
    towards an even result).
    """
    u = np.ascontiguousarray(a, dtype=F32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)


def as_f32(w: np.ndarray, kind: str) -> np.ndarray:
    """Input tensor as exact float32 values ([P5] Step 1 works in float32)."""
    if kind == "bf16":
        return widen_bf16(w)
    if kind == "f32":
        return np.asarray(w, F32)
    if kind == "f16":
        return np.asarray(w, F16).astype(F32)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Quantization ([P2] Architecture Overview, Steps 5-6; [P5] Step 2)
# --------------------------------------------------------------------------
def split_groups(w32: np.ndarray, g: int) -> np.ndarray:
    """[N, K] -> [N, K/g, g]: each row cut into runs of g consecutive columns."""
    n, k = w32.shape
    if k % g:
        raise ValueError("K must be a multiple of the group size")
    return w32.reshape(n, k // g, g)


def group_range(w32: np.ndarray, g: int):
    """Per-group minimum and maximum ([P2] Step 5)."""
    wg = split_groups(w32, g)
    return wg.min(axis=2), wg.max(axis=2)


def scale_zero(mn: np.ndarray, mx: np.ndarray, sz: str):
    """Scale and zero-point per group ([P2] Architecture Overview, Step 6).

    scale = fl32(fl32(max - min) / 15), rounded to the storage dtype; a stored
    scale of zero (constant group) becomes 1 ([P4] Step 2 uses the same
    guard).  The zero-point uses the stored scale:
    zp = clamp(rint(fl32(-min / scale)), 0, 15), an integer.
    Returns (scale_stored [sz dtype], zero_point [int32]).
    """
    sd = SZ_DTYPES[sz]
    s32 = (mx.astype(F32) - mn.astype(F32)) / F32(15.0)
    s_st = s32.astype(sd)
    s_st = np.where(s_st == 0, sd(1.0), s_st).astype(sd)
    s = s_st.astype(F32)
    zp = np.clip(np.rint(-mn.astype(F32) / s), 0, 15).astype(np.int32)
    return s_st, zp


def quantize_codes(w32: np.ndarray, s_st: np.ndarray, zp: np.ndarray, g: int) -> np.ndarray:
    """q = clamp(rint(fl32(fl32(w / scale) + zp)), 0, 15)  ([P5] Step 2)."""
    wg = split_groups(w32, g)
    s = s_st.astype(F32)[..., None]
    z = zp.astype(F32)[..., None]
    q = np.clip(np.rint(wg / s + z), 0, 15).astype(np.uint8)
    return q.reshape(w32.shape)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two codes per byte; column 2j in the low nibble, 2j+1 in the high one
    ([P4] Step 4 states this order; [P3] Step 1 builds bytes the same way)."""
    q = np.asarray(q, np.uint8)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    return (q[..., 0::2] | (q[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: [N, K/2] bytes -> [N, K] codes 0..15."""
    p = np.asarray(packed, np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    q[..., 0::2] = p & np.uint8(0x0F)
    q[..., 1::2] = p >> np.uint8(4)
    return q


def quantize_pack_int4(w: np.ndarray, kind: str, g: int, sz: str):
    """Full quantize + pack of W [N, K].

    Returns (packed uint8 [N, K/2], scales [N, K/g] in sz dtype,
    zeros [N, K/g] in sz dtype holding the integers 0..15).
    """
    w32 = as_f32(w, kind)
    mn, mx = group_range(w32, g)
    s_st, zp = scale_zero(mn, mx, sz)
    q = quantize_codes(w32, s_st, zp, g)
    return pack_nibbles(q), s_st, zp.astype(SZ_DTYPES[sz])


# --------------------------------------------------------------------------
# Symmetric variant ([P4] Step 2 for scale and codes, Step 4 for the +8
# offset).  The codes and scales it stores feed the same dequantization and
# matmuls as the asymmetric ones, with every zero-point equal to 8.
# --------------------------------------------------------------------------
SYM_OFFSET = 8


def group_absmax(w32: np.ndarray, g: int) -> np.ndarray:
    """Per-group maximum of |w| ([P4] Step 2)."""
    return np.abs(split_groups(w32, g)).max(axis=2)


def scale_sym(amax: np.ndarray, sz: str) -> np.ndarray:
    """scale = fl32(absmax / 7), rounded to the storage dtype; a stored scale
    of zero becomes 1 ([P4] Step 2).  Like the asymmetric scale, the guard is
    applied to the stored value."""
    sd = SZ_DTYPES[sz]
    s_st = (amax.astype(F32) / F32(7.0)).astype(sd)
    return np.where(s_st == 0, sd(1.0), s_st).astype(sd)


def quantize_codes_sym(w32: np.ndarray, s_st: np.ndarray, g: int) -> np.ndarray:
    """Signed code clamp(rint(fl32(w / scale)), -8, 7) ([P4] Step 2), stored
    unsigned as code + 8 ([P4] Step 4).  The offset is added to the rounded
    integer, not before rounding."""
    wg = split_groups(w32, g)
    s = s_st.astype(F32)[..., None]
    q = np.clip(np.rint(wg / s), -8, 7).astype(np.int32)
    return (q + SYM_OFFSET).astype(np.uint8).reshape(w32.shape)


def quantize_pack_int4_sym(w: np.ndarray, kind: str, g: int, sz: str):
    """Symmetric quantize + pack of W [N, K].

    Returns (packed uint8 [N, K/2], scales [N, K/g] in sz dtype, zeros
    [N, K/g] in sz dtype, all equal to 8), so that (q - zp) * scale is the
    symmetric dequantization.
    """
    w32 = as_f32(w, kind)
    s_st = scale_sym(group_absmax(w32, g), sz)
    q = quantize_codes_sym(w32, s_st, g)
    zeros = np.full(s_st.shape, SYM_OFFSET, SZ_DTYPES[sz])
    return pack_nibbles(q), s_st, zeros


# --------------------------------------------------------------------------
# Range-clipping calibrators for the symmetric variant ([P3] Step 4): they
# choose each group's scale differently; the codes are then the symmetric
# ones, clamp(rint(w / scale), -8, 7) + 8 with the stored scale.
#
# The page's calibrators are PyTorch calls on a float32 group:
# torch.quantile(|w|, p / 100) and a search over torch.linspace(min|w|,
# max|w|, n) with torch's float32 division, round, clamp and mse_loss.  The
# functions below write out the float32 values those calls return (the
# readings are pinned bit for bit against torch itself in the tests).
# --------------------------------------------------------------------------
def store_scale(s32: np.ndarray, sz: str) -> np.ndarray:
    """fp32 step -> storage dtype (nearest even); a stored 0 becomes 1."""
    sd = SZ_DTYPES[sz]
    s_st = np.asarray(s32, F32).astype(sd)
    return np.where(s_st == 0, sd(1.0), s_st).astype(sd)


def fma32(a, b, c) -> np.ndarray:
    """a * b + c with ONE rounding to float32 (a fused multiply-add),
    elementwise, for float32 a, b, c.

    a * b of two float32 numbers is exact in float64.  The float64 sum with c
    is then rounded to odd: when Knuth's TwoSum shows the sum was inexact and
    the float64 result has an even last bit, it is moved one step towards the
    exact value.  Rounding that value to float32 gives the correctly rounded
    a * b + c, because float64 carries more than float32's 24 + 2 bits
    (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd", IEEE Trans. Computers 2008)."""
    a64 = np.asarray(a, F32).astype(np.float64)
    b64 = np.asarray(b, F32).astype(np.float64)
    c64 = np.asarray(c, F32).astype(np.float64)
    prod = a64 * b64                          # exact: 24 + 24 significant bits
    s = prod + c64
    bv = s - prod                             # TwoSum: err = exact sum - s
    err = (prod - (s - bv)) + (c64 - bv)
    even = (np.ascontiguousarray(s).view(np.int64) & 1) == 0
    s = np.where((err != 0) & even, np.nextafter(s, np.where(err > 0, np.inf, -np.inf)), s)
    return s.astype(F32)


def percentile_position(g: int, p: float):
    """Where torch.quantile(v, p / 100) of g values reads the sorted values:
    q = fl32(p / 100) (the fraction becomes a float32 tensor), rank =
    fl32(q * (g - 1)); returns (i0, i1, f) with i0 = floor(rank), i1 =
    ceil(rank) and the interpolation weight f = rank - i0 (exact)."""
    q = F32(p / 100.0)
    rank = F32(q * F32(g - 1))
    i0 = int(np.floor(rank))
    return i0, int(np.ceil(rank)), F32(rank - F32(i0))


def calib_percentile_range(w32: np.ndarray, g: int, p: float) -> np.ndarray:
    """[P3] Step 4, "percentile": torch.quantile(|w|, p / 100) per group
    (linear interpolation).  With a the group's |w| in ascending order and
    (i0, i1, f) from percentile_position, d = fl32(a[i1] - a[i0]); the value
    is taken from the nearer end with one rounding: a[i0] + f d when f < 1/2,
    else a[i1] - (1 - f) d, i.e. fma(f, d, a[i0]) or fma(f - 1, d, a[i1])."""
    a = np.sort(np.abs(split_groups(w32, g)), axis=2)
    i0, i1, f = percentile_position(g, p)
    lo = a[..., i0].astype(F32)
    hi = a[..., i1].astype(F32)
    d = (hi - lo).astype(F32)
    if f < F32(0.5):
        return fma32(f, d, lo)
    return fma32(F32(f - F32(1.0)), d, hi)


def quantize_pack_int4_sym_percentile(w: np.ndarray, kind: str, g: int, sz: str, p: float):
    """Symmetric quantize + pack with range = the p-th percentile of |w|
    (scale = range / 7, as scale_sym does with the maximum)."""
    w32 = as_f32(w, kind)
    s_st = scale_sym(calib_percentile_range(w32, g, p), sz)
    q = quantize_codes_sym(w32, s_st, g)
    return pack_nibbles(q), s_st, np.full(s_st.shape, SYM_OFFSET, SZ_DTYPES[sz])


def mse_candidates(lo: np.ndarray, hi: np.ndarray, n: int) -> np.ndarray:
    """torch.linspace(lo, hi, n) in float32 ([P3] Step 4 "mse_search"): the
    step d = fl32(fl32(hi - lo) / (n - 1)); the first n // 2 values are
    counted up from lo, the rest down from hi, each with one rounding:
    c_i = fma(d, i, lo) for i < n // 2, fma(-d, n - 1 - i, hi) otherwise.
    So c_0 = lo and c_(n-1) = hi exactly."""
    lo = np.asarray(lo, F32)[..., None]
    hi = np.asarray(hi, F32)[..., None]
    d = ((hi - lo) / F32(n - 1)).astype(F32)
    i = np.arange(n)
    up = fma32(d, i.astype(F32), lo)
    down = fma32(-d, (n - 1 - i).astype(F32), hi)
    return np.where(i < n // 2, up, down).astype(F32)


MSE_SKIP_BELOW = F32(1e-10)
MSE_NONE = F32(1e-8)


def mse_codes(w: np.ndarray, c: np.ndarray) -> np.ndarray:
    """The search's codes for the candidate step c: clamp(rint(fl32(w / c)),
    -7, 7) -- a float32 division, rounded half to even, clamped to +-7."""
    return np.clip(np.rint((np.asarray(w, F32) / np.asarray(c, F32)).astype(F32)), -7, 7).astype(F32)


def calib_mse_step(w32: np.ndarray, g: int, n: int) -> np.ndarray:
    """[P3] Step 4, "mse_search", per group: candidate steps c =
    mse_candidates(min|w|, max|w|, n); a c below 1e-10 is skipped; for the
    others the codes are q = clamp(rint(fl32(w / c)), -7, 7) and the error
    is the mean over the group of fl32(fl32(q * c) - w)^2: the float32 sum in
    column order, divided by g in float32.  The first candidate with the
    least mean is the step; 1e-8 when every candidate is skipped."""
    wg = split_groups(w32, g)
    a = np.abs(wg)
    c = mse_candidates(a.min(axis=2), a.max(axis=2), n)
    valid = c >= MSE_SKIP_BELOW
    csafe = np.where(valid, c, F32(1.0))
    E = np.zeros(c.shape, F32)
    for k in range(g):
        wk = wg[..., k][..., None]
        q = mse_codes(wk, csafe)
        e = ((q * csafe).astype(F32) - wk).astype(F32)
        E = (E + (e * e).astype(F32)).astype(F32)
    mean = (E / F32(g)).astype(F32)
    mean = np.where(valid, mean, np.inf)
    best = np.argmin(mean, axis=2)  # first occurrence of the minimum
    step = np.take_along_axis(c, best[..., None], 2)[..., 0]
    return np.where(valid.any(axis=2), step, MSE_NONE).astype(F32)


def quantize_pack_int4_sym_mse(w: np.ndarray, kind: str, g: int, sz: str, n: int):
    """Symmetric quantize + pack with the step chosen by the MSE search."""
    w32 = as_f32(w, kind)
    s_st = store_scale(calib_mse_step(w32, g, n), sz)
    q = quantize_codes_sym(w32, s_st, g)
    return pack_nibbles(q), s_st, np.full(s_st.shape, SYM_OFFSET, SZ_DTYPES[sz])


# --------------------------------------------------------------------------
# Dequantization ([P5] Step 4)
# --------------------------------------------------------------------------
def dequant_f32(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g: int) -> np.ndarray:
    """w_hat = fl32((q - zp) * scale) as float32 [N, K]."""
    q = unpack_nibbles(packed).astype(np.int32)
    n, k = q.shape
    zp = np.asarray(zeros).astype(np.int32)
    s = np.asarray(scales).astype(F32)
    d = (q.reshape(n, k // g, g) - zp[..., None]).astype(F32)
    return (d * s[..., None]).reshape(n, k)


def dequant(packed, scales, zeros, g: int, out: str) -> np.ndarray:
    """dequant_f32 rounded (nearest-even) to the output dtype: "f32" gives
    float32, "f16" float16, "bf16" bf16 bits."""
    w = dequant_f32(packed, scales, zeros, g)
    if out == "f32":
        return w
    if out == "f16":
        return w.astype(F16)
    if out == "bf16":
        return to_bf16(w)
    raise ValueError(out)


def dequant_f64(packed, scales, zeros, g: int, rows=None) -> np.ndarray:
    """Exact (q - zp) * scale in float64 for the matmul references."""
    p = np.asarray(packed) if rows is None else np.asarray(packed)[rows]
    s = np.asarray(scales) if rows is None else np.asarray(scales)[rows]
    z = np.asarray(zeros) if rows is None else np.asarray(zeros)[rows]
    q = unpack_nibbles(p).astype(np.float64)
    n, k = q.shape
    d = q.reshape(n, k // g, g) - z.astype(np.float64)[..., None]
    return (d * s.astype(np.float64)[..., None]).reshape(n, k)


# --------------------------------------------------------------------------
# Per-token INT8 activations ([P1] Architecture Overview, Step 3)
# --------------------------------------------------------------------------
def act_quant_int8(x32: np.ndarray):
    """s_a = fl32(max(max_k |x|, 1e-8) / 127); xq = clamp(rint(fl32(x/s_a)), -128, 127).

    The 1e-8 floor is applied before the division, as on the page.
    Returns (xq int8 [M, K], s_a float32 [M]).
    """
    x32 = np.asarray(x32, F32)
    amax = np.max(np.abs(x32), axis=1)
    s = np.maximum(amax, F32(1e-8)) / F32(127.0)
    xq = np.clip(np.rint(x32 / s[:, None]), -128, 127).astype(np.int8)
    return xq, s.astype(F32)


# --------------------------------------------------------------------------
# Matmul references ([P3] Step 2; [P4] Step 5; [P1] Step 5)
# --------------------------------------------------------------------------
def _chunks(n: int, step: int):
    for i in range(0, n, step):
        yield slice(i, min(n, i + step))


def matmul_w4a16_f64(x32: np.ndarray, packed, scales, zeros, g: int, chunk: int = 2048) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w_hat[n, k] in float64 (x widened exactly).

    Done chunk by chunk over output rows of W so the fp64 weight never exists
    whole; the matmul itself is NumPy's (a library primitive).
    """
    x64 = np.asarray(x32, F32).astype(np.float64)
    n = np.asarray(packed).shape[0]
    y = np.empty((x64.shape[0], n), np.float64)
    for sl in _chunks(n, chunk):
        w64 = dequant_f64(packed, scales, zeros, g, rows=sl)
        y[:, sl] = x64 @ w64.T
    return y


def matmul_w4a8_f64(xq: np.ndarray, s_a: np.ndarray, packed, scales, zeros, g: int,
                    chunk: int = 2048) -> np.ndarray:
    """y[m, n] = s_a[m] * sum_k xq[m, k] * w_hat[n, k] in float64."""
    x64 = np.asarray(xq).astype(np.float64)
    sa = np.asarray(s_a, F32).astype(np.float64)
    n = np.asarray(packed).shape[0]
    y = np.empty((x64.shape[0], n), np.float64)
    for sl in _chunks(n, chunk):
        w64 = dequant_f64(packed, scales, zeros, g, rows=sl)
        y[:, sl] = x64 @ w64.T
    return y * sa[:, None]


# --------------------------------------------------------------------------
# Comparison metric for matmul outputs
# --------------------------------------------------------------------------
def max_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max |ref|  (infinity-norm relative error)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
