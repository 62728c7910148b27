"""Planted mistakes in the oracle must be caught by its pins.

Each mutation replaces one oracle function (on the CPU, via monkeypatch) with
a plausible wrong version: a dropped term, a wrong sign, a wrong rounding, a
transposed operand, the other nibble order.  The pin suite must then fail at
least one check.  This is evidence that the pins constrain the oracle, not a
test of the GPU path.
"""
import numpy as np
import pytest

import oracle.w4_oracle as O
from tests import oracle_pins as P

F32 = np.float32
_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _pack_high_even(q):
    q = np.asarray(q, np.uint8)
    return ((q[..., 0::2] << np.uint8(4)) | q[..., 1::2]).astype(np.uint8)


def _unpack_high_even(p):
    p = np.asarray(p, np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    q[..., 0::2] = p >> np.uint8(4)
    q[..., 1::2] = p & np.uint8(0x0F)
    return q


def _unpack_swapped_only(p):
    return _unpack_high_even(p)


def _codes_round_half_up(w32, s_st, zp, g):
    wg = O.split_groups(w32, g)
    t = wg / s_st.astype(F32)[..., None] + zp.astype(F32)[..., None]
    return np.clip(np.floor(t + F32(0.5)), 0, 15).astype(np.uint8).reshape(w32.shape)


def _codes_round_then_shift(w32, s_st, zp, g):
    wg = O.split_groups(w32, g)
    t = np.rint(wg / s_st.astype(F32)[..., None]) + zp.astype(F32)[..., None]
    return np.clip(t, 0, 15).astype(np.uint8).reshape(w32.shape)


def _codes_with_unrounded_scale_factory():
    # quantize with the fp32 scale although the fp16 one is stored
    def scale_zero(mn, mx, sz):
        sd = O.SZ_DTYPES[sz]
        s32 = (mx.astype(F32) - mn.astype(F32)) / F32(15.0)
        s32 = np.where(s32 == 0, F32(1.0), s32)
        zp = np.clip(np.rint(-mn.astype(F32) / s32), 0, 15).astype(np.int32)
        _state["s32"] = s32
        return s32.astype(sd), zp

    def quantize_codes(w32, s_st, zp, g):
        return _orig["quantize_codes"](w32, _state["s32"], zp, g)

    return scale_zero, quantize_codes


_state = {}


def _scale_zero_sign_flip(mn, mx, sz):
    s_st, zp = _orig["scale_zero"](mn, mx, sz)
    s = s_st.astype(F32)
    return s_st, np.clip(np.rint(mn.astype(F32) / s), 0, 15).astype(np.int32)


def _scale_zero_div16(mn, mx, sz):
    sd = O.SZ_DTYPES[sz]
    s_st = ((mx - mn) / F32(16.0)).astype(sd)
    s_st = np.where(s_st == 0, sd(1.0), s_st).astype(sd)
    zp = np.clip(np.rint(-mn / s_st.astype(F32)), 0, 15).astype(np.int32)
    return s_st, zp


def _scale_zero_no_guard(mn, mx, sz):
    sd = O.SZ_DTYPES[sz]
    with np.errstate(all="ignore"):
        s_st = ((mx - mn) / F32(15.0)).astype(sd)
        zp = np.clip(np.nan_to_num(np.rint(-mn / s_st.astype(F32))), 0, 15).astype(np.int32)
    return s_st, zp


def _scale_zero_guard_before_rounding(mn, mx, sz):
    sd = O.SZ_DTYPES[sz]
    s32 = (mx - mn) / F32(15.0)
    s32 = np.where(s32 == 0, F32(1.0), s32)
    s_st = s32.astype(sd)
    with np.errstate(all="ignore"):
        zp = np.clip(np.nan_to_num(np.rint(-mn / s_st.astype(F32))), 0, 15).astype(np.int32)
    return s_st, zp


def _dequant_plus_zp(packed, scales, zeros, g):
    q = O.unpack_nibbles(packed).astype(np.int32)
    n, k = q.shape
    d = (q.reshape(n, k // g, g) + np.asarray(zeros).astype(np.int32)[..., None]).astype(F32)
    return (d * np.asarray(scales).astype(F32)[..., None]).reshape(n, k)


def _dequant64_plus_zp(packed, scales, zeros, g, rows=None):
    return _dequant_plus_zp(packed if rows is None else packed[rows],
                            scales if rows is None else scales[rows],
                            zeros if rows is None else zeros[rows], g).astype(np.float64)


def _split_strided(w32, g):
    n, k = w32.shape
    return w32.reshape(n, g, k // g).transpose(0, 2, 1)


def _matmul_untransposed(x32, packed, scales, zeros, g, chunk=2048):
    w64 = O.dequant_f64(packed, scales, zeros, g)
    return np.asarray(x32, F32).astype(np.float64) @ w64


def _act_clip_after(x32):
    amax = np.max(np.abs(x32), axis=1)
    s = np.maximum(amax / F32(127.0), F32(1e-8)).astype(F32)
    xq = np.clip(np.rint(x32 / s[:, None]), -128, 127).astype(np.int8)
    return xq, s


def _act_div128(x32):
    amax = np.max(np.abs(x32), axis=1)
    s = (np.maximum(amax, F32(1e-8)) / F32(128.0)).astype(F32)
    xq = np.clip(np.rint(x32 / s[:, None]), -128, 127).astype(np.int8)
    return xq, s


def _w4a8_no_act_scale(xq, s_a, packed, scales, zeros, g, chunk=2048):
    return _orig["matmul_w4a8_f64"](xq, np.ones_like(s_a), packed, scales, zeros, g, chunk)


def _to_bf16_truncate(a):
    return (np.ascontiguousarray(a, F32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _dequant64_wrong_group(packed, scales, zeros, g, rows=None):
    # scale/zero of the next group (a shifted index)
    s = np.roll(np.asarray(scales), 1, axis=1)
    z = np.roll(np.asarray(zeros), 1, axis=1)
    return _orig["dequant_f64"](packed, s, z, g, rows)


def _sym_scale_over_8(amax, sz):
    sd = O.SZ_DTYPES[sz]
    s_st = (amax.astype(F32) / F32(8.0)).astype(sd)
    return np.where(s_st == 0, sd(1.0), s_st).astype(sd)


def _sym_scale_guard_first(amax, sz):
    sd = O.SZ_DTYPES[sz]
    s32 = amax.astype(F32) / F32(7.0)
    with np.errstate(all="ignore"):
        return np.where(s32 == 0, F32(1.0), s32).astype(sd)


def _sym_offset_before_rounding(w32, s_st, g):
    wg = O.split_groups(w32, g)
    t = np.rint(wg / s_st.astype(F32)[..., None] + F32(8.0))
    return np.clip(t, 0, 15).astype(np.uint8).reshape(w32.shape)


def _sym_codes_of_magnitude(w32, s_st, g):
    # quantizes |w| instead of w
    return _orig["quantize_codes_sym"](np.abs(w32), s_st, g)


def _sym_clamp_7(w32, s_st, g):
    wg = O.split_groups(w32, g)
    q = np.clip(np.rint(wg / s_st.astype(F32)[..., None]), -7, 7).astype(np.int32)
    return (q + 8).astype(np.uint8).reshape(w32.shape)


def _sym_round_half_away(w32, s_st, g):
    wg = O.split_groups(w32, g)
    v = wg / s_st.astype(F32)[..., None]
    q = np.clip(np.sign(v) * np.floor(np.abs(v) + F32(0.5)), -8, 7).astype(np.int32)
    return (q + 8).astype(np.uint8).reshape(w32.shape)


def _sym_quantize_with_unrounded_scale(w, kind, g, sz):
    w32 = O.as_f32(w, kind)
    s32 = O.group_absmax(w32, g).astype(F32) / F32(7.0)
    s32 = np.where(s32 == 0, F32(1.0), s32).astype(F32)
    s_st = s32.astype(O.SZ_DTYPES[sz])
    s_st = np.where(s_st == 0, O.SZ_DTYPES[sz](1.0), s_st)
    q = O.quantize_codes_sym(w32, s32, g)
    return O.pack_nibbles(q), s_st, np.full(s_st.shape, 8, O.SZ_DTYPES[sz])


def _sym_zero_point_7(w, kind, g, sz):
    p, s, z = _orig["quantize_pack_int4_sym"](w, kind, g, sz)
    return p, s, np.full(z.shape, 7, z.dtype)


def _pct_nearest_rank(w32, g, p):
    a = np.sort(np.abs(O.split_groups(w32, g)), axis=2)
    i = int(round((g - 1) * p / 100.0))
    return a[..., i].astype(F32)


def _pct_signed(w32, g, p):
    a = np.sort(O.split_groups(w32, g), axis=2)
    i0, i1, f = O.percentile_position(g, p)
    return (a[..., i0] + f * (a[..., i1] - a[..., i0])).astype(F32)


def _pct_position_from_g(g, p):
    h = g * (p / 100.0)
    i0 = min(int(np.floor(h)), g - 1)
    return i0, min(i0 + 1, g - 1), F32(h - np.floor(h))


def _mse_search_with(w32, g, n, lo_clamp=-7, last=False):
    # calib_mse_step with one of two planted mistakes: codes clamped at
    # lo_clamp instead of -7, or the last (not the first) least mean kept
    wg = O.split_groups(w32, g)
    a = np.abs(wg)
    c = O.mse_candidates(a.min(axis=2), a.max(axis=2), n)
    valid = c >= O.MSE_SKIP_BELOW
    cs = np.where(valid, c, F32(1.0))
    E = np.zeros(c.shape, F32)
    for k in range(g):
        wk = wg[..., k][..., None]
        q = np.clip(np.rint((wk / cs).astype(F32)), lo_clamp, 7).astype(F32)
        e = ((q * cs).astype(F32) - wk).astype(F32)
        E = (E + (e * e).astype(F32)).astype(F32)
    E = np.where(valid, (E / F32(g)).astype(F32), np.inf)
    best = E.shape[2] - 1 - np.argmin(E[..., ::-1], axis=2) if last else np.argmin(E, axis=2)
    step = np.take_along_axis(c, best[..., None], 2)[..., 0]
    return np.where(valid.any(axis=2), step, O.MSE_NONE).astype(F32)


def _mse_last_minimum(w32, g, n):
    return _mse_search_with(w32, g, n, last=True)


def _mse_clamp_8(w32, g, n):
    return _mse_search_with(w32, g, n, lo_clamp=-8)


def _mse_candidates_one_ended(lo, hi, n):
    # every candidate counted up from lo: c_i = fl32(lo + fl32(i * d))
    lo = np.asarray(lo, F32)[..., None]
    hi = np.asarray(hi, F32)[..., None]
    d = ((hi - lo) / F32(n - 1)).astype(F32)
    return (lo + (np.arange(n, dtype=F32) * d).astype(F32)).astype(F32)


def _mse_codes_by_reciprocal(w, c):
    return np.clip(np.rint((np.asarray(w, F32) * (F32(1.0) / np.asarray(c, F32)).astype(F32)).astype(F32)),
                   -7, 7).astype(F32)


def _pct_lower_end_two_roundings(w32, g, p):
    a = np.sort(np.abs(O.split_groups(w32, g)), axis=2)
    i0, i1, f = O.percentile_position(g, p)
    lo = a[..., i0].astype(F32)
    return (lo + (f * (a[..., i1] - lo).astype(F32)).astype(F32)).astype(F32)


def _pct_position_float64(g, p):
    h = (g - 1) * (p / 100.0)
    i0 = int(np.floor(h))
    return i0, min(i0 + 1, g - 1), F32(h - i0)


def _fma32_two_roundings(a, b, c):
    return ((np.asarray(a, F32) * np.asarray(b, F32)).astype(F32) + np.asarray(c, F32)).astype(F32)


def _mse_candidates_from_zero(lo, hi, n):
    return _orig["mse_candidates"](np.zeros_like(lo), hi, n)


def _mse_candidates_n_steps(lo, hi, n):
    d = ((hi.astype(F32) - lo.astype(F32)) / F32(n)).astype(F32)
    i = np.arange(n, dtype=F32)
    return (lo.astype(F32)[..., None] + i * d[..., None]).astype(F32)


def _mse_no_none_default(w32, g, n):
    st = _orig["calib_mse_step"](w32, g, n)
    return np.where(st == O.MSE_NONE, F32(0.0), st).astype(F32)


def _cal_scale_over_8(w, kind, g, sz, p):
    w32 = O.as_f32(w, kind)
    s_st = O.store_scale((O.calib_percentile_range(w32, g, p) / F32(8.0)).astype(F32), sz)
    q = O.quantize_codes_sym(w32, s_st, g)
    return O.pack_nibbles(q), s_st, np.full(s_st.shape, 8, O.SZ_DTYPES[sz])


_uq_sz, _uq_codes = _codes_with_unrounded_scale_factory()

MUTATIONS = {
    "pack_high_nibble_even": {"pack_nibbles": _pack_high_even, "unpack_nibbles": _unpack_high_even},
    "unpack_swapped_only": {"unpack_nibbles": _unpack_swapped_only},
    "round_half_up": {"quantize_codes": _codes_round_half_up},
    "round_before_zero_point": {"quantize_codes": _codes_round_then_shift},
    "zero_point_sign": {"scale_zero": _scale_zero_sign_flip},
    "scale_over_16": {"scale_zero": _scale_zero_div16},
    "no_zero_scale_guard": {"scale_zero": _scale_zero_no_guard},
    "guard_before_fp16_rounding": {"scale_zero": _scale_zero_guard_before_rounding},
    "quantize_with_unrounded_scale": {"scale_zero": _uq_sz, "quantize_codes": _uq_codes},
    "dequant_adds_zero_point": {"dequant_f32": _dequant_plus_zp, "dequant_f64": _dequant64_plus_zp},
    "groups_strided_not_runs": {"split_groups": _split_strided},
    "matmul_untransposed": {"matmul_w4a16_f64": _matmul_untransposed},
    "act_floor_after_divide": {"act_quant_int8": _act_clip_after},
    "act_scale_over_128": {"act_quant_int8": _act_div128},
    "w4a8_drops_act_scale": {"matmul_w4a8_f64": _w4a8_no_act_scale},
    "bf16_truncates": {"to_bf16": _to_bf16_truncate},
    "dequant_shifted_group_index": {"dequant_f64": _dequant64_wrong_group},
    "sym_scale_over_8": {"scale_sym": _sym_scale_over_8},
    "sym_guard_before_fp16_rounding": {"scale_sym": _sym_scale_guard_first},
    "sym_offset_before_rounding": {"quantize_codes_sym": _sym_offset_before_rounding},
    "sym_quantizes_magnitude": {"quantize_codes_sym": _sym_codes_of_magnitude},
    "sym_clamp_to_plus_minus_7": {"quantize_codes_sym": _sym_clamp_7},
    "sym_round_half_away": {"quantize_codes_sym": _sym_round_half_away},
    "sym_quantize_with_unrounded_scale": {"quantize_pack_int4_sym": _sym_quantize_with_unrounded_scale},
    "sym_zero_point_7": {"quantize_pack_int4_sym": _sym_zero_point_7},
    "percentile_nearest_rank": {"calib_percentile_range": _pct_nearest_rank},
    "percentile_of_signed_values": {"calib_percentile_range": _pct_signed},
    "percentile_position_g_not_g_minus_1": {"percentile_position": _pct_position_from_g},
    "percentile_scale_over_8": {"quantize_pack_int4_sym_percentile": _cal_scale_over_8},
    "mse_last_minimum": {"calib_mse_step": _mse_last_minimum},
    "mse_search_clamps_at_minus_8": {"calib_mse_step": _mse_clamp_8},
    "mse_candidates_from_zero": {"mse_candidates": _mse_candidates_from_zero},
    "mse_candidates_spacing_over_n": {"mse_candidates": _mse_candidates_n_steps},
    "mse_no_default_step": {"calib_mse_step": _mse_no_none_default},
    "mse_candidates_one_ended": {"mse_candidates": _mse_candidates_one_ended},
    "mse_codes_by_reciprocal": {"mse_codes": _mse_codes_by_reciprocal},
    "percentile_lower_end_two_roundings": {"calib_percentile_range": _pct_lower_end_two_roundings},
    "percentile_position_float64": {"percentile_position": _pct_position_float64},
    "fma32_two_roundings": {"fma32": _fma32_two_roundings},
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name].items():
        monkeypatch.setattr(O, attr, fn)
    failed = []
    for check in P.ALL_CHECKS:  # the slowest pins come last; stop at the first that fails
        try:
            with np.errstate(all="ignore"):
                check()
        except Exception as exc:  # AssertionError or a shape error: caught either way
            failed.append((check.__name__, type(exc).__name__))
            break
    assert failed, f"planted mistake {name!r} passed every pin"
