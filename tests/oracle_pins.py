"""Checks that pin the oracle to things other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
pages or the mathematics fix: values printed on the pages, hand-derived
worked examples (tests/golden/), closed forms, invariants, library routines
for special cases, and brute force on tiny inputs.  They are plain functions
so that tests/test_oracle_mutations.py can run all of them against an oracle
with a planted mistake and require that at least one fails.

The oracle is reached through the module object ``O`` (never through names
imported from it) so that a planted mistake is seen by every check.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.w4_oracle as O
from tests import brute_force as BF
from tests import page_calibrators as PC

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
f32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------
def check_pack_page_vector():
    """Page vector (GPTQ engine page, 'The tests') under the Step 4 convention."""
    gv = _golden("pack_vector.json")
    codes = np.array([gv["codes"]], np.uint8)
    assert (codes.astype(int) - 8).tolist() == [gv["signed_values"]]
    packed = O.pack_nibbles(codes)
    want = [int(h, 16) for h in gv["packed_bytes_hex"]]
    assert packed.tolist() == [want], (packed.tolist(), want)
    assert O.unpack_nibbles(packed).tolist() == codes.tolist()


def check_pack_exhaustive():
    """All 256 bytes unpack to (low, high) and pack back exactly."""
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = O.unpack_nibbles(b)
    assert q.shape == (1, 512)
    assert np.array_equal(q[0, 0::2], np.arange(256) % 16)
    assert np.array_equal(q[0, 1::2], np.arange(256) // 16)
    assert np.array_equal(O.pack_nibbles(q), b)


# ---------------------------------------------------------------------------
# Worked example: scale, zero-point, ties (tests/golden/worked_example_g32.json)
# ---------------------------------------------------------------------------
def worked_example_group():
    """The 32 values of the worked example, interleaved, plus expected codes."""
    u = 2.0 ** -6
    lv = [((j - 5) * u, j) for j in range(16)]
    mid_codes = _golden("worked_example_g32.json")["expected"]["midpoint_codes"]
    md = [((j - 4.5) * u, mid_codes[j]) for j in range(15)]
    order = [lv[15], md[0], lv[0], md[14]]
    rest_l = lv[1:15]
    rest_m = md[1:14]
    for i in range(max(len(rest_l), len(rest_m))):
        if i < len(rest_l):
            order.append(rest_l[i])
        if i < len(rest_m):
            order.append(rest_m[i])
    order.append(lv[7])
    assert len(order) == 32
    vals = np.array([v for v, _ in order], np.float32)
    codes = np.array([c for _, c in order], np.uint8)
    return vals, codes


def check_worked_example():
    gv = _golden("worked_example_g32.json")
    vals, codes = worked_example_group()
    u = 2.0 ** -6
    for sz in ("f32", "f16"):
        for kind in ("f32", "bf16"):
            w = vals.reshape(1, 32) if kind == "f32" else O.to_bf16(vals).reshape(1, 32)
            p, s, z = O.quantize_pack_int4(w, kind, 32, sz)
            assert float(s[0, 0]) == u, (sz, kind, float(s[0, 0]))
            assert float(z[0, 0]) == gv["expected"]["zero_point"]
            assert np.array_equal(O.unpack_nibbles(p)[0], codes), (O.unpack_nibbles(p)[0], codes)
            wh = O.dequant_f32(p, s, z, 32)[0]
            lv = np.array([abs(v / u - round(v / u)) < 1e-12 for v in vals.astype(float)])
            assert np.array_equal(wh[lv], vals[lv])  # levels reproduce exactly
            assert np.array_equal(wh, ((codes.astype(np.float64) - 5) * u).astype(np.float32))


# ---------------------------------------------------------------------------
# Degenerate, clamped and extreme groups
# ---------------------------------------------------------------------------
def check_degenerate_groups():
    w = np.zeros((2, 64), np.float32)
    w[1, :32] = 3.0
    w[1, 32:] = -3.0
    for sz in ("f32", "f16"):
        p, s, z = O.quantize_pack_int4(w, "f32", 32, sz)
        q = O.unpack_nibbles(p)
        assert float(s[0, 0]) == 1.0 and float(z[0, 0]) == 0.0 and not q[0, :32].any()
        assert float(s[1, 0]) == 1.0 and float(z[1, 0]) == 0.0 and (q[1, :32] == 3).all()
        assert float(s[1, 1]) == 1.0 and float(z[1, 1]) == 3.0 and (q[1, 32:] == 0).all()
        wh = O.dequant_f32(p, s, z, 32)
        assert np.array_equal(wh[:2], w[:2])
        # the stored zero-point of a zero-range group is +0.0, never -0.0
        assert not np.signbit(np.asarray(z, np.float32)).any()


def check_tiny_range_scales():
    """fp16 subnormal scales are kept; a scale that underflows fp16 becomes 1."""
    g = 32
    w = np.zeros((2, g), np.float32)
    w[0] = (np.arange(g) % 16).astype(np.float32) * np.float32(2.0 ** -20)  # range 15*2^-20
    w[1] = (np.arange(g) % 16).astype(np.float32) * np.float32(2.0 ** -27)  # range 15*2^-27
    p, s, z = O.quantize_pack_int4(w, "f32", g, "f16")
    assert float(s[0, 0]) == 2.0 ** -20  # fp16 subnormal, exact
    assert float(z[0, 0]) == 0.0
    assert np.array_equal(O.unpack_nibbles(p)[0], (np.arange(g) % 16).astype(np.uint8))
    assert float(s[1, 0]) == 1.0 and float(z[1, 0]) == 0.0
    assert not O.unpack_nibbles(p)[1].any()
    # with fp32 scales nothing underflows
    p2, s2, z2 = O.quantize_pack_int4(w, "f32", g, "f32")
    assert float(s2[1, 0]) == 2.0 ** -27
    assert np.array_equal(O.unpack_nibbles(p2)[1], (np.arange(g) % 16).astype(np.uint8))


def check_clamped_zero_point():
    """All-positive group: zp clamps to 0 and the top codes saturate at 15;
    all-negative group: zp clamps to 15 and the low codes saturate at 0."""
    g = 32
    w = np.zeros((2, g), np.float32)
    w[0] = np.linspace(1.0, 2.5, g, dtype=np.float32)
    w[1] = -np.linspace(1.0, 2.5, g, dtype=np.float32)
    for sz in ("f32", "f16"):
        p, s, z = O.quantize_pack_int4(w, "f32", g, sz)
        q = O.unpack_nibbles(p)
        assert float(z[0, 0]) == 0.0 and q[0].max() == 15 and q[0, -1] == 15
        assert float(z[1, 0]) == 15.0 and q[1].min() == 0 and q[1, -1] == 0
        sv = float(s[0, 0])
        assert abs(sv - 0.1) < 1e-3
        # codes are the clamped nearest levels
        want = np.clip(np.rint(w[0].astype(np.float64) / sv), 0, 15)
        assert np.array_equal(q[0], want.astype(np.uint8))


# ---------------------------------------------------------------------------
# Group axis, per-group scales: each group is the per-tensor quantizer of
# "From Scratch: Building a GPTQ INT4 Quantizer in Pure Python" (Step 2)
# applied to that run of g columns.
# ---------------------------------------------------------------------------
def check_groups_are_row_runs():
    rng = np.random.default_rng(11)
    n, k, g = 3, 96, 32
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    w[1, 40] = 0.5  # an outlier confined to group (1, 1)
    p, s, z = O.quantize_pack_int4(w, "f32", g, "f16")
    q = O.unpack_nibbles(p)
    for r in range(n):
        for gi in range(k // g):
            vals = [f32(v) for v in w[r, gi * g:(gi + 1) * g]]
            st, zp, codes = BF.quantize_group(vals, "f16")
            assert float(s[r, gi]) == float(st) and float(z[r, gi]) == zp
            assert q[r, gi * g:(gi + 1) * g].tolist() == codes
    big = float(s[1, 1])
    assert all(float(s[r, gi]) < big / 4 for r in range(n) for gi in range(3) if (r, gi) != (1, 1))


# ---------------------------------------------------------------------------
# Brute force on tiny random inputs: bit-exact agreement
# ---------------------------------------------------------------------------
def check_brute_force_quantize():
    rng = np.random.default_rng(5)
    for (n, k, g) in ((4, 64, 32), (3, 64, 64), (8, 32, 32)):
        w = rng.normal(0, 0.05, (n, k)).astype(np.float32)
        w[0, 3] = 0.5
        w[-1, :g] = np.abs(w[-1, :g])  # an all-positive group (clamped zp)
        for sz in ("f32", "f16"):
            for kind in ("f32", "bf16"):
                src = w if kind == "f32" else O.to_bf16(w)
                w32 = w if kind == "f32" else O.widen_bf16(src)
                p, s, z = O.quantize_pack_int4(src, kind, g, sz)
                bp, bs, bz = BF.quantize_pack(w32, g, sz)
                assert np.array_equal(p, bp), (n, k, g, sz, kind)
                assert np.array_equal(s.view(np.uint8), bs.view(np.uint8))
                assert np.array_equal(z.view(np.uint8), bz.view(np.uint8))
                d = O.dequant_f32(p, s, z, g)
                assert np.array_equal(d.view(np.uint32), BF.dequant(p, s, z, g).view(np.uint32))


def check_brute_force_act_quant():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 1, (5, 48)).astype(np.float32)
    x[1] *= 20.0
    x[2] = 0.0
    x[3] = x[3] * np.float32(1e-12)
    xq, sa = O.act_quant_int8(x)
    bq, bs = BF.act_quant(x)
    assert np.array_equal(xq, bq) and np.array_equal(sa.view(np.uint32), bs.view(np.uint32))


def check_brute_force_matmul():
    """fp64 references agree with correctly rounded dot products (fsum)."""
    rng = np.random.default_rng(7)
    n, k, g, m = 6, 64, 32, 3
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    p, s, z = O.quantize_pack_int4(w, "f32", g, "f32")
    wh = BF.dequant(p, s, z, g)  # fl32 values
    w64 = O.dequant_f64(p, s, z, g)
    # the fp64 dequant is the exact (q-zp)*s; its fp32 rounding is the fp32 dequant
    assert np.array_equal(w64.astype(np.float32), wh)
    y = O.matmul_w4a16_f64(x, p, s, z, g)
    for i in range(m):
        for j in range(n):
            ref = BF.dot_exact(x[i], w64[j])
            assert abs(y[i, j] - ref) <= 1e-12 * (1 + abs(ref)), (i, j, y[i, j], ref)
    xq, sa = O.act_quant_int8(x)
    y8 = O.matmul_w4a8_f64(xq, sa, p, s, z, g)
    for i in range(m):
        for j in range(n):
            ref = float(sa[i]) * BF.dot_exact(xq[i], w64[j])
            assert abs(y8[i, j] - ref) <= 1e-12 * (1 + abs(ref))


# ---------------------------------------------------------------------------
# Closed forms: exact matmuls with no tolerance
# ---------------------------------------------------------------------------
def _integer_weights(rng, n, k, g):
    """Integers in [0, 15], every group holding both 0 and 15."""
    w = rng.integers(0, 16, (n, k))
    for r in range(n):
        for gi in range(k // g):
            a, b = rng.choice(g, 2, replace=False)
            w[r, gi * g + a] = 0
            w[r, gi * g + b] = 15
    return w


def check_exact_integer_matmul():
    """W in [0,15] with 0 and 15 in each group quantizes to s=1, zp=0, q=W;
    with integer x the fp64 product equals the integer product exactly."""
    rng = np.random.default_rng(8)
    for (n, k, g, m, sz) in ((64, 64, 32, 3, "f16"), (24, 256, 32, 5, "f32"), (24, 256, 32, 5, "f16")):
        wi = _integer_weights(rng, n, k, g)
        xi = rng.integers(-8, 9, (m, k))
        p, s, z = O.quantize_pack_int4(wi.astype(np.float32), "f32", g, sz)
        assert (np.asarray(s, np.float32) == 1).all() and (np.asarray(z, np.float32) == 0).all()
        assert np.array_equal(O.unpack_nibbles(p), wi.astype(np.uint8))
        y = O.matmul_w4a16_f64(xi.astype(np.float32), p, s, z, g)
        assert y.shape == (m, n)
        assert np.array_equal(y, (xi @ wi.T).astype(np.float64))


def check_codes_nearest_stored_level():
    """Every code is a nearest level of the grid (q - zp) * s_stored, q in
    0..15: neither neighbouring code would reconstruct w more closely (round
    to nearest on the stored grid; exact ties may go either way)."""
    rng = np.random.default_rng(14)
    n, k, g = 64, 512, 128
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    for sz in ("f16", "f32"):
        p, s, z = O.quantize_pack_int4(w, "f32", g, sz)
        q = O.unpack_nibbles(p).astype(np.int64).reshape(n, k // g, g)
        sv = np.asarray(s, np.float64)[..., None]
        zv = np.asarray(z, np.float64)[..., None]
        wv = w.astype(np.float64).reshape(n, k // g, g)
        err = np.abs(wv - (q - zv) * sv)
        for d in (-1, 1):
            qn = q + d
            ok = (qn >= 0) & (qn <= 15)
            errn = np.abs(wv - (qn - zv) * sv)
            # allow only rounding-level differences (fp32 division of w by s)
            assert (err[ok] <= errn[ok] + sv.repeat(g, 2)[ok] * 2.0 ** -20).all(), sz


def check_exact_scaled_matmul():
    """Per-group power-of-two scales and zero-points, exactly representable:
    W[r, group] = 2^e * (Q - Z).  Quantization must return (2^e, Z, Q) for
    every (row, group), and the matmul must equal the exact rational result."""
    rng = np.random.default_rng(9)
    n, k, g, m = 6, 128, 32, 3
    ng = k // g
    Q = _integer_weights(rng, n, k, g)
    E = rng.integers(-9, -3, (n, ng))
    Z = rng.integers(0, 16, (n, ng))
    w = np.zeros((n, k), np.float64)
    for r in range(n):
        for gi in range(ng):
            w[r, gi * g:(gi + 1) * g] = (2.0 ** E[r, gi]) * (Q[r, gi * g:(gi + 1) * g] - Z[r, gi])
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    xi = rng.integers(-127, 128, (m, k))
    for sz in ("f32", "f16"):
        p, s, z = O.quantize_pack_int4(w32, "f32", g, sz)
        assert np.array_equal(np.asarray(s, np.float64), 2.0 ** E)
        assert np.array_equal(np.asarray(z, np.float64), Z.astype(np.float64))
        assert np.array_equal(O.unpack_nibbles(p), Q.astype(np.uint8))
        assert np.array_equal(O.dequant_f32(p, s, z, g), w32)
        y = O.matmul_w4a16_f64(xi.astype(np.float32), p, s, z, g)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(int(xi[i, c])) * Fraction(float(w[j, c])) for c in range(k))
                assert y[i, j] == float(exact)
        # W4A8 with a non-unit activation scale: x = 2^-3 * xi, amax = 127/8
        xs = (xi.astype(np.float64) / 8.0)
        xs[:, 0] = 127.0 / 8.0
        xq, sa = O.act_quant_int8(xs.astype(np.float32))
        assert (sa == np.float32(0.125)).all()
        assert np.array_equal(xq.astype(np.int64), (xs * 8).astype(np.int64))
        y8 = O.matmul_w4a8_f64(xq, sa, p, s, z, g)
        assert np.array_equal(y8, xs @ w.T)


# ---------------------------------------------------------------------------
# Activation quantization closed forms
# ("Hands-on Build Guide: Group-wise INT4 ...", Step 3)
# ---------------------------------------------------------------------------
def check_act_quant_closed_forms():
    k = 64
    x = np.zeros((4, k), np.float32)
    x[0] = np.arange(-32, 32)
    x[0, 5] = 127.0                      # amax 127 -> s = 1, xq = x
    x[1] = 0.0                           # all-zero token: s = fl32(1e-8)/127
    x[2] = (np.arange(k) % 9 - 4 + 0.5) * 0.25  # ties: x/s = j + 0.5 with s = 0.25
    x[2, 0] = 31.75                      # amax 31.75 -> s = 0.25
    x[3] = -x[0]
    xq, sa = O.act_quant_int8(x)
    assert sa[0] == 1.0 and np.array_equal(xq[0].astype(np.float32), x[0])
    assert sa[1] == np.float32(np.float32(1e-8) / np.float32(127.0)) and not xq[1].any()
    assert sa[2] == 0.25
    t = x[2, 1:].astype(np.float64) / 0.25
    # every t is an exact .5 tie: half-even picks the even neighbour
    want = np.array([(math.floor(v) if math.floor(v) % 2 == 0 else math.floor(v) + 1) for v in t])
    assert np.array_equal(xq[2, 1:].astype(np.int64), want)
    assert xq[2, 0] == 127
    assert sa[3] == 1.0 and np.array_equal(xq[3].astype(np.float32), x[3])
    assert xq.min() >= -127


def check_act_quant_invariants():
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1, (16, 512)).astype(np.float32)
    x[:, rng.choice(512, 26, replace=False)] *= 20
    xq, sa = O.act_quant_int8(x)
    assert xq.min() >= -127 and xq.max() <= 127
    assert (np.abs(xq).max(axis=1) == 127).all()
    err = np.abs(x.astype(np.float64) - xq.astype(np.float64) * sa[:, None].astype(np.float64))
    assert (err <= sa[:, None] * 0.5 * (1 + 2.0 ** -16)).all()


# ---------------------------------------------------------------------------
# Invariants on a realistic matrix
# ---------------------------------------------------------------------------
def quant_invariants(w32: np.ndarray, g: int, sz: str, mse_band=None):
    """zp in [0, 15]; |w - w_hat| <= (s/2)(1 + slack) wherever the zero-point
    was not clamped; MSE close to s^2/12.  Returns (max ratio, count above s/2)."""
    src = w32
    p, s, z = O.quantize_pack_int4(src, "f32", g, sz)
    zf = np.asarray(z, np.float32)
    assert (zf >= 0).all() and (zf <= 15).all() and (zf == np.rint(zf)).all()
    wh = O.dequant_f64(p, s, z, g)
    n, k = w32.shape
    sv = np.asarray(s, np.float64)
    err = np.abs(w32.astype(np.float64) - wh).reshape(n, k // g, g)
    mn = w32.reshape(n, k // g, g).min(axis=2)
    raw = np.rint(-mn.astype(np.float32) / np.asarray(s, np.float32))
    free = (raw >= 0) & (raw <= 15)
    slack = 2.0 ** -6 if sz == "f16" else 2.0 ** -16
    ratio = err.max(axis=2) / (sv / 2)
    assert (ratio[free] <= 1 + slack).all(), float(ratio[free].max())
    above = int((err > (sv / 2)[..., None]).sum())
    if mse_band is not None:
        mse_ratio = float((err ** 2).mean() / (sv ** 2 / 12).mean())
        assert mse_band[0] < mse_ratio < mse_band[1], mse_ratio
    return float(ratio[free].max()), above


def check_invariants_small_config():
    """256x256 fp32 single layer, g=32, fp32 scales (the first workload)."""
    from workloads import weight
    w = weight("W1").as_f32()
    quant_invariants(w, 32, "f32", mse_band=(0.95, 1.05))
    quant_invariants(w, 32, "f16", mse_band=(0.95, 1.05))


# ---------------------------------------------------------------------------
# Symmetric variant ("Build a GPTQ INT4 Quantization Engine in Python/NumPy",
# Step 2: scale = absmax/7, code clamp(round(w/scale), -8, 7); Step 4: +8)
# ---------------------------------------------------------------------------
def worked_example_sym_group(kind: str):
    """The 32 values of the symmetric worked example and their stored codes
    (tests/golden/worked_example_sym_g32.json).  The near-tie value is exact
    in fp32 only; the bf16 case has 0 (code 8) in its place."""
    gv = _golden("worked_example_sym_g32.json")
    u = 2.0 ** -6
    vals = [j * u for j in gv["levels_j"]]
    codes = [j + 8 for j in gv["levels_j"]]
    vals += [(j + 0.5) * u for j in gv["midpoints_j"]]
    codes += gv["expected"]["midpoint_codes"]
    vals += [j * u for j in gv["repeated_levels_j"]]
    codes += [j + 8 for j in gv["repeated_levels_j"]]
    if kind == "f32":
        vals.append(float(np.frombuffer(bytes.fromhex(gv["near_tie_value_f32_hex"])[::-1], f32)[0]))
        codes.append(gv["expected"]["near_tie_code"])
    else:
        vals.append(0.0)
        codes.append(8)
    assert len(vals) == 32
    return np.array(vals, f32), np.array(codes, np.uint8)


def check_sym_worked_example():
    gv = _golden("worked_example_sym_g32.json")
    u = 2.0 ** -6
    for sz in ("f32", "f16"):
        for kind in ("f32", "bf16"):
            vals, codes = worked_example_sym_group(kind)
            w = vals.reshape(1, 32) if kind == "f32" else O.to_bf16(vals).reshape(1, 32)
            assert np.array_equal(O.as_f32(w, kind)[0], vals)  # every value exact in the input type
            p, s, z = O.quantize_pack_int4_sym(w, kind, 32, sz)
            assert float(s[0, 0]) == u, (sz, kind, float(s[0, 0]))
            assert float(z[0, 0]) == gv["expected"]["zero_point"]
            assert np.array_equal(O.unpack_nibbles(p)[0], codes), (O.unpack_nibbles(p)[0], codes)
            wh = O.dequant_f32(p, s, z, 32)[0]
            assert np.array_equal(wh, ((codes.astype(np.float64) - 8) * u).astype(np.float32))
            lv = np.r_[0:15, 29:31]  # the levels reproduce exactly
            assert np.array_equal(wh[lv], vals[lv])


def check_sym_special_groups():
    """Zero and signed-zero groups, a scale that underflows fp16, and an
    fp16-subnormal scale coarse enough that the -8 code is reached."""
    g = 32
    t = np.float32(2.0 ** -24)
    w = np.zeros((4, 2 * g), np.float32)
    w[0, g:] = -3.0                                   # constant negative group
    w[1, :5] = np.array([-10, 10, 7.5, -8.5, -7.5], np.float32) * t
    w[1, g:g + 15] = np.arange(-7, 8) * np.float32(2.0 ** -27)
    w[2, ::2] = -0.0
    w[3, :g] = np.arange(-16, 16) * np.float32(1e-30)  # tiny fp32 range
    p16, s16, z16 = O.quantize_pack_int4_sym(w, "f32", g, "f16")
    q16 = O.unpack_nibbles(p16).astype(int)
    assert (np.asarray(z16, np.float32) == 8).all()
    # all-zero and signed-zero groups: scale 1, code 8 (signed 0)
    assert float(s16[0, 0]) == 1.0 and (q16[0, :g] == 8).all()
    assert float(s16[2, 0]) == 1.0 and (q16[2] == 8).all()
    # constant -3: scale fp16(3/7), code -7
    assert float(s16[0, 1]) == float(np.float16(np.float32(3.0) / np.float32(7.0)))
    assert (q16[0, g:] == 1).all()
    # absmax 10 * 2^-24: fp32 scale 10/7 * 2^-24 rounds to the fp16 subnormal
    # 2^-24, so w/s = -10, 10, 7.5, -8.5, -7.5 -> -8, 7, 7, -8, -8 (stored +8)
    assert float(s16[1, 0]) == 2.0 ** -24
    assert q16[1, :5].tolist() == [0, 15, 15, 0, 0]
    # absmax 7 * 2^-27: the scale 2^-27 underflows fp16 -> 1, every code 8
    assert float(s16[1, 1]) == 1.0 and (q16[1, g:] == 8).all()
    assert float(s16[3, 0]) == 1.0 and (q16[3, :g] == 8).all()
    # fp32 scales keep all of these
    p32, s32, z32 = O.quantize_pack_int4_sym(w, "f32", g, "f32")
    q32 = O.unpack_nibbles(p32).astype(int)
    assert float(s32[1, 1]) == 2.0 ** -27
    assert q32[1, g:g + 15].tolist() == list(range(1, 16))
    assert q32[1, :5].tolist() == [1, 15, 13, 2, 3]  # w/s = -7, 7, 5.25, -5.95, -5.25
    assert float(s32[3, 0]) == float(np.float32(np.float32(16e-30) / np.float32(7.0)))


def check_sym_brute_force():
    rng = np.random.default_rng(15)
    for (n, k, g) in ((4, 64, 32), (3, 128, 64), (2, 256, 128)):
        w = rng.normal(0, 0.05, (n, k)).astype(np.float32)
        w[0, 5] = -0.6
        w[-1, :g] = np.abs(w[-1, :g])
        for sz in ("f32", "f16"):
            for kind in ("f32", "bf16"):
                src = w if kind == "f32" else O.to_bf16(w)
                w32 = w if kind == "f32" else O.widen_bf16(src)
                p, s, z = O.quantize_pack_int4_sym(src, kind, g, sz)
                bp, bs, bz = BF.quantize_pack_sym(w32, g, sz)
                assert np.array_equal(p, bp), (n, k, g, sz, kind)
                assert np.array_equal(s.view(np.uint8), bs.view(np.uint8))
                assert np.array_equal(z.view(np.uint8), bz.view(np.uint8))
                d = O.dequant_f32(p, s, z, g)
                assert np.array_equal(d.view(np.uint32), BF.dequant(p, s, z, g).view(np.uint32))


def check_sym_exact_scaled_matmul():
    """W[r, group] = 2^e * Q with Q in -7..7 and |Q| = 7 in every group:
    quantization returns (2^e, Q + 8) exactly, and the matmuls equal the
    exact rational results."""
    rng = np.random.default_rng(16)
    n, k, g, m = 5, 128, 32, 3
    ng = k // g
    Q = rng.integers(-7, 8, (n, k))
    for r in range(n):
        for gi in range(ng):
            Q[r, gi * g + rng.integers(0, g)] = 7 * (1 if rng.integers(0, 2) else -1)
    E = rng.integers(-9, -3, (n, ng))
    w = np.repeat(2.0 ** E, g, axis=1) * Q
    w32 = w.astype(np.float32)
    xi = rng.integers(-127, 128, (m, k))
    for sz in ("f32", "f16"):
        p, s, z = O.quantize_pack_int4_sym(w32, "f32", g, sz)
        assert np.array_equal(np.asarray(s, np.float64), 2.0 ** E)
        assert np.array_equal(O.unpack_nibbles(p).astype(np.int64), Q + 8)
        assert np.array_equal(O.dequant_f32(p, s, z, g), w32)
        y = O.matmul_w4a16_f64(xi.astype(np.float32), p, s, z, g)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(int(xi[i, c])) * Fraction(float(w[j, c])) for c in range(k))
                assert y[i, j] == float(exact)
        xq, sa = O.act_quant_int8(xi.astype(np.float32))
        y8 = O.matmul_w4a8_f64(xq, sa, p, s, z, g)
        assert np.allclose(y8, (xq.astype(np.float64) * sa[:, None].astype(np.float64)) @ w.T,
                           rtol=1e-15, atol=0)


def check_sym_invariants():
    """Codes 1..15 (the -8 code needs a subnormal scale); the element of
    largest magnitude of each group takes code 1 or 15; every error within
    half a step; each code a nearest level of the stored grid; MSE near
    s^2/12 (one exact element per group lowers it by about 1/g)."""
    from workloads import weight
    rng = np.random.default_rng(17)
    cases = [(weight("W1").as_f32(), 32, "f32"), (weight("W1").as_f32(), 32, "f16"),
             (O.widen_bf16(O.to_bf16(rng.normal(0, 0.02, (64, 1024)).astype(np.float32))), 128, "f16")]
    for w, g, sz in cases:
        n, k = w.shape
        p, s, z = O.quantize_pack_int4_sym(w, "f32", g, sz)
        q = O.unpack_nibbles(p).astype(np.int64).reshape(n, k // g, g)
        assert q.min() >= 1 and q.max() <= 15
        wg = w.astype(np.float64).reshape(n, k // g, g)
        top = np.take_along_axis(q, np.abs(wg).argmax(axis=2)[..., None], 2)[..., 0]
        assert np.isin(top, (1, 15)).all()
        sv = np.asarray(s, np.float64)[..., None]
        err = np.abs(wg - (q - 8) * sv)
        slack = 2.0 ** -6 if sz == "f16" else 2.0 ** -16
        assert (err <= sv / 2 * (1 + slack)).all()
        for d in (-1, 1):
            qn = q + d
            ok = (qn >= 0) & (qn <= 15)
            errn = np.abs(wg - (qn - 8) * sv)
            assert (err[ok] <= errn[ok] + np.broadcast_to(sv, err.shape)[ok] * 2.0 ** -20).all()
        mse_ratio = float((err ** 2).mean() / (sv ** 2 / 12).mean())
        assert (1 - 2.0 / g) < mse_ratio < 1.05, (g, sz, mse_ratio)


# ---------------------------------------------------------------------------
# Range-clipping calibrators ("Building a From-Scratch Group-Wise INT4
# Quantization Layer for LLaMA Weights", Step 4)
# ---------------------------------------------------------------------------
def check_percentile_100_is_minmax():
    """The 100th percentile is the maximum: the outputs equal the plain
    symmetric quantizer's bit for bit."""
    rng = np.random.default_rng(21)
    w = rng.normal(0, 0.05, (16, 512)).astype(np.float32)
    w[3, 7] = -0.9
    for sz in ("f16", "f32"):
        for g in (32, 128):
            a = O.quantize_pack_int4_sym_percentile(w, "f32", g, sz, 100.0)
            b = O.quantize_pack_int4_sym(w, "f32", g, sz)
            for x, y in zip(a, b):
                assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


def check_percentile_vs_numpy():
    """Against NumPy's linear-interpolation quantile in float64, within fp32
    rounding."""
    rng = np.random.default_rng(22)
    w = rng.normal(0, 1, (8, 1024)).astype(np.float32)
    for g in (32, 128, 1024):
        for p in (50.0, 90.0, 99.0, 99.9):
            got = O.calib_percentile_range(w, g, p).astype(np.float64)
            want = np.quantile(np.abs(w.astype(np.float64)).reshape(8, -1, g), p / 100.0, axis=2,
                               method="linear")
            assert np.allclose(got, want, rtol=4e-6, atol=0), (g, p, float(np.abs(got - want).max()))


def check_percentile_vs_torch_quantile():
    """Bit for bit against the page's call, torch.quantile(|w|, p / 100), on
    1536 random groups (batched) and 48 single groups (the page's 1-D call),
    over sizes, scales, ties and percentiles that put the rank's fraction
    below and above 1/2."""
    import torch
    rng = np.random.default_rng(25)
    for g in (32, 96, 128, 640):
        w = (rng.normal(0, 1, (12, 4 * g)) * 10.0 ** rng.uniform(-5, 1, (12, 1))).astype(np.float32)
        w[0, : g // 2] = w[0, 0]                    # repeated values
        w[1, :g] = 0.0                              # an all-zero group
        for p in (0.5, 12.345, 33.3, 50.0, 75.0, 90.0, 99.0, 99.9, 99.99, 100.0):
            got = O.calib_percentile_range(w, g, p)
            ref = torch.quantile(torch.from_numpy(np.abs(w).reshape(12, 4, g)), p / 100, dim=2).numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (g, p)
    for t in range(48):
        g = (32, 128)[t % 2]
        v = (rng.normal(0, 0.02, g) * (1 + 9 * (t % 3))).astype(np.float32)
        p = float(rng.uniform(1, 100))
        got = O.calib_percentile_range(v.reshape(1, g), g, p)[0, 0]
        assert got.view(np.uint32) == PC.percentile(v, p).view(np.uint32), (t, g, p)


def check_percentile_exact_midpoint():
    """g = 32, p = 50: the rank is 15.5, so the range is the exact midpoint
    of the 16th and 17th smallest |w| (values chosen exact in binary)."""
    g = 32
    mags = np.arange(1, 33, dtype=np.float32) * np.float32(2.0 ** -8)  # 16th: 16/256, 17th: 17/256
    w = (mags * np.where(np.arange(32) % 3 == 0, -1, 1)).astype(np.float32)[np.random.default_rng(1).permutation(32)]
    r = O.calib_percentile_range(w.reshape(1, g), g, 50.0)
    assert float(r[0, 0]) == 16.5 / 256, float(r[0, 0])
    assert O.percentile_position(g, 50.0) == (15, 16, np.float32(0.5))
    # 100th and tiny percentiles: the extreme order statistics
    assert float(O.calib_percentile_range(w.reshape(1, g), g, 100.0)[0, 0]) == 32 / 256
    i0, i1, f = O.percentile_position(g, 1e-9)
    assert (i0, i1) == (0, 1) and 0 < f < 1e-9
    # p = 99.9 at g = 128: rank fl32(fl32(0.999) * 127) = 126.873..., so the
    # value is read from the upper end: a[127] - (1 - f)(a[127] - a[126])
    i0, i1, f = O.percentile_position(128, 99.9)
    assert (i0, i1) == (126, 127) and f == np.float32(np.float32(0.999) * np.float32(127)) - np.float32(126)


def _exact_round_f32(x) -> np.float32:
    """A rational (fractions.Fraction) rounded to the nearest float32, ties to
    even, in integer arithmetic (normal range)."""
    from fractions import Fraction
    x = Fraction(x)
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    unit = Fraction(2) ** (e - 23)               # 2^e <= x < 2^(e+1): 24-bit significand
    m = x / unit
    q = m.numerator // m.denominator
    rem = m - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q * unit))


def check_fma32_correctly_rounded():
    """fma32 against the exact rational a * b + c rounded once, on random
    operands of mixed scales and on sums that sit on, just off and across
    float32 rounding midpoints (where two roundings would differ)."""
    from fractions import Fraction
    rng = np.random.default_rng(26)
    a = (rng.normal(0, 1, 400) * 2.0 ** rng.integers(-30, 30, 400)).astype(np.float32)
    b = rng.integers(0, 70000, 400).astype(np.float32)
    c = (rng.normal(0, 1, 400) * 2.0 ** rng.integers(-40, 30, 400)).astype(np.float32)
    # midpoint constructions: a * b = 1 + 2^-24 (a midpoint of float32 at 1),
    # plus a tiny c of either sign, or none
    a = np.concatenate([a, np.float32([1.0 + 2.0 ** -23] * 3 + [3.0, 2.0 ** -24])])
    b = np.concatenate([b, np.float32([1.0 - 2.0 ** -24] * 3 + [1.0 / 3.0, 1.0])])
    c = np.concatenate([c, np.float32([2.0 ** -70, -(2.0 ** -70), 0.0, -1.0, 1.0])])
    got = O.fma32(a, b, c)
    for ai, bi, ci, gi in zip(a, b, c, got):
        want = _exact_round_f32(Fraction(float(ai)) * Fraction(float(bi)) + Fraction(float(ci)))
        assert gi.view(np.uint32) == want.view(np.uint32), (ai, bi, ci, gi, want)


def check_mse_candidates_vs_torch_linspace():
    """Bit for bit against torch.linspace(min|w|, max|w|, n) in float32 on
    1200 random groups and a range of n, including tiny, zero and equal
    ends; the ends are exact."""
    import torch
    rng = np.random.default_rng(27)
    for t in range(1200):
        v = np.abs(rng.normal(0, 1, 128) * 10.0 ** rng.uniform(-8, 2)).astype(np.float32)
        if t % 13 == 0:
            v[:] = v[0]
        if t % 7 == 0:
            v[5] = 0.0
        lo, hi = v.min(), v.max()
        n = (2, 3, 5, 17, 64, 100, 999, 1000, 1001, 4096)[t % 10]
        got = O.mse_candidates(np.float32(lo), np.float32(hi), n)
        ref = torch.linspace(torch.tensor(lo), torch.tensor(hi), n).numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (t, n)
        assert got[0] == lo and got[-1] == hi


def check_mse_codes_vs_torch():
    """The search's codes against torch's float32 division, round and clamp,
    on random pairs and on pairs where w / c is exactly a half-integer or one
    ulp from one, so that a product with a rounded reciprocal 1/c would take
    the other side (for example 0.04443359375 / (7 * 2^-10) = 6.5 rounds to
    6, while 0.04443359375 * fl32(1 / (7 * 2^-10)) rounds up to 6.5000005)."""
    import torch
    rng = np.random.default_rng(28)
    w = rng.normal(0, 0.05, 4000).astype(np.float32)
    c = np.abs(rng.normal(0, 0.01, 4000)).astype(np.float32) + np.float32(1e-6)
    tw, tc = [], []
    for j in range(3, 200, 2):
        cj = np.float32(j * 2.0 ** -10)
        for k in range(7):
            base = np.float32((k + 0.5) * float(cj))
            for d in (-1, 0, 1):
                tw.append((base.view(np.int32) + d).view(np.float32) * (1 if (j + k) % 2 else -1))
                tc.append(cj)
    w = np.concatenate([w, np.array(tw, np.float32)])
    c = np.concatenate([c, np.array(tc, np.float32)])
    got = O.mse_codes(w, c)
    ref = torch.clamp(torch.round(torch.from_numpy(w) / torch.from_numpy(c)), -7, 7).numpy()
    assert np.array_equal(got, ref)
    recip = np.clip(np.rint(w * (np.float32(1.0) / c)), -7, 7)
    assert (recip != ref).sum() > 50   # the constructed pairs do separate the two forms


def check_mse_step_vs_page_search():
    """The chosen step, bit for bit, against the page's mse_search evaluated
    with torch one group at a time: 1000 random groups with 100 candidates
    and 100 groups with 1000 (Gaussian weights at several scales, with and
    without an outlier, and a few all-equal or zero-containing groups)."""
    rng = np.random.default_rng(29)
    for n, count in ((100, 1000), (1000, 100)):
        for t in range(count):
            g = (32, 128, 64)[t % 3]
            v = (rng.normal(0, 1, g) * 10.0 ** rng.uniform(-4, 0)).astype(np.float32)
            if t % 4 == 0:
                v[rng.integers(0, g)] = np.float32(8.0 * np.abs(v).max())
            if t % 97 == 0:
                v[:] = v[0]
            if t % 89 == 0:
                v[: g // 4] = 0.0
            got = O.calib_mse_step(v.reshape(1, g), g, n)[0, 0]
            ref = PC.mse_search(v, n)
            assert got.view(np.uint32) == ref.view(np.uint32), (n, t, g, got, ref)


def check_calibrators_brute_force():
    rng = np.random.default_rng(23)
    w = rng.normal(0, 0.05, (3, 64)).astype(np.float32)
    w[0, 5] = 0.7
    w[2, 32:] = 0.0
    for sz in ("f16", "f32"):
        for p in (99.9, 75.0):
            a = O.quantize_pack_int4_sym_percentile(w, "f32", 32, sz, p)
            b = BF.quantize_pack_calibrated(w, 32, sz, "percentile", p)
            for x, y in zip(a, b):
                assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), (sz, p)
        a = O.quantize_pack_int4_sym_mse(w, "f32", 32, sz, 40)
        b = BF.quantize_pack_calibrated(w, 32, sz, "mse", 40)
        for x, y in zip(a, b):
            assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), sz


def check_mse_exact_grid():
    """Values on the grid j * u (j = -7 .. 7, zero included) with n = 8
    candidates: c_i = i * u exactly, c_0 = 0 is skipped and c_1 = u
    reproduces every value (error 0), so the step is u and the codes j + 8."""
    u = 2.0 ** -7
    j = np.array(list(range(-7, 8)) + [3, -3, 0, 7, -7, 1, 2, -1, -2, 5, -5, 4, -4, 6, -6, 0, 2], np.int64)
    w = (j * u).astype(np.float32).reshape(1, 32)
    assert float(O.calib_mse_step(w, 32, 8)[0, 0]) == u
    for sz in ("f16", "f32"):
        p, s, z = O.quantize_pack_int4_sym_mse(w, "f32", 32, sz, 8)
        assert float(s[0, 0]) == u and float(z[0, 0]) == 8
        assert np.array_equal(O.unpack_nibbles(p)[0].astype(np.int64), j + 8)


def check_mse_first_minimum_and_clamp():
    """Ties: 16 zeros and 16 fives, n = 11 (c_i = i / 2): the steps 1, 2.5
    and 5 all reproduce the group exactly, and the first (1) wins.
    Clamp: 16 values -8, one 7 and 15 zeros, n = 9 (c_i = i): with codes
    clamped to +-7 the step 1 leaves error 16 (each -8 becomes -7) and the
    step 2 leaves 1 (7 becomes 8), so 2 wins; a search clamped at -8 would
    pick 1."""
    w = np.array([0.0] * 16 + [5.0] * 16, np.float32)[np.random.default_rng(2).permutation(32)].reshape(1, 32)
    assert float(O.calib_mse_step(w, 32, 11)[0, 0]) == 1.0
    w2 = np.array([-8.0] * 16 + [7.0] + [0.0] * 15, np.float32).reshape(1, 32)
    assert float(O.calib_mse_step(w2, 32, 9)[0, 0]) == 2.0


def check_mse_skipped_candidates():
    """Candidates below 1e-10 are skipped; a group with none left takes
    1e-8, which underflows fp16 and is then stored as 1."""
    g = 32
    w = np.zeros((3, g), np.float32)
    w[1, :4] = np.float32(5e-11)                  # max|w| < 1e-10: every candidate skipped
    w[2, :] = np.float32(3e-10) * (np.arange(g) % 4)  # min 0, max 9e-10: c_0 = 0 skipped
    st = O.calib_mse_step(w, g, 10)
    assert st[0, 0] == O.MSE_NONE and st[1, 0] == O.MSE_NONE
    assert st[2, 0] >= O.MSE_SKIP_BELOW
    p16, s16, _ = O.quantize_pack_int4_sym_mse(w, "f32", g, "f16", 10)
    assert float(s16[0, 0]) == 1.0 and (O.unpack_nibbles(p16)[:2] == 8).all()
    p32, s32, _ = O.quantize_pack_int4_sym_mse(w, "f32", g, "f32", 10)
    assert s32[0, 0] == O.MSE_NONE and (O.unpack_nibbles(p32)[0] == 8).all()


def check_mse_is_least_error():
    """The chosen step's error (recomputed in float64) is the least over the
    candidates, up to fp32 rounding of the sums, and never above the plain
    absmax/7 step's error by more than that."""
    rng = np.random.default_rng(24)
    w = rng.normal(0, 0.02, (4, 256)).astype(np.float32)
    w[1, 3] = 0.3
    g, n = 64, 200
    st = O.calib_mse_step(w, g, n).astype(np.float64)
    wg = w.astype(np.float64).reshape(4, -1, g)
    a = np.abs(wg)
    c = O.mse_candidates(a.min(axis=2).astype(np.float32), a.max(axis=2).astype(np.float32), n).astype(np.float64)

    def err(step):
        q = np.clip(np.rint(wg / step[..., None]), -7, 7)
        return ((q * step[..., None] - wg) ** 2).sum(axis=2)

    e_best = err(st)
    for i in range(n):
        ci = c[..., i]
        ok = ci >= 1e-10
        e_i = err(np.where(ok, ci, 1.0))
        assert (e_best[ok] <= e_i[ok] * (1 + 1e-5) + 1e-30).all(), i
    assert (e_best <= err(a.max(axis=2) / 7.0) * (1 + 1e-5)).all()


# ---------------------------------------------------------------------------
# bf16 rounding of the oracle against the library routine (torch)
# ---------------------------------------------------------------------------
def check_bf16_rounding_vs_torch():
    import torch
    rng = np.random.default_rng(13)
    a = rng.normal(0, 1, 4096).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with even and odd kept parts
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties, np.float32([0.0, -0.0, 1e-40, 3.0e38])])
    ours = O.to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(O.widen_bf16(ours), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def check_max_rel_err():
    r = np.array([[1.0, -4.0], [2.0, 0.5]])
    y = r + np.array([[0.0, 0.04], [-0.02, 0.0]])
    assert abs(O.max_rel_err(y, r) - 0.01) < 1e-15


ALL_CHECKS = [
    check_pack_page_vector, check_pack_exhaustive, check_worked_example,
    check_degenerate_groups, check_tiny_range_scales, check_clamped_zero_point,
    check_groups_are_row_runs, check_brute_force_quantize, check_brute_force_act_quant,
    check_brute_force_matmul, check_exact_integer_matmul, check_codes_nearest_stored_level,
    check_exact_scaled_matmul,
    check_act_quant_closed_forms, check_act_quant_invariants, check_invariants_small_config,
    check_bf16_rounding_vs_torch, check_max_rel_err,
    check_sym_worked_example, check_sym_special_groups, check_sym_brute_force,
    check_sym_exact_scaled_matmul, check_sym_invariants,
    check_percentile_100_is_minmax, check_percentile_vs_numpy, check_percentile_exact_midpoint,
    check_percentile_vs_torch_quantile, check_fma32_correctly_rounded,
    check_mse_candidates_vs_torch_linspace, check_mse_codes_vs_torch,
    check_calibrators_brute_force, check_mse_exact_grid, check_mse_first_minimum_and_clamp,
    check_mse_skipped_candidates, check_mse_is_least_error,
    check_mse_step_vs_page_search,  # slowest: keep last
]
