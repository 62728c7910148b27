"""GPU parity for the symmetric variant: quantize_pack_int4_sym against the
oracle (bit-exact packed bytes, scales and zeros), then its outputs through
dequant_int4 (bit-exact) and both matmuls (the method's tolerances; bit-exact
for integer constructions) on every dispatch path.
"""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests import oracle_pins as PINS
from tests.gpu_util import TORCH_SZ, Canary, bits, to_dev, to_host, y_as_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 3e-3}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def gpu_quantize_sym(w4, w_np, kind, g, sz):
    n, k = w_np.shape
    cp = Canary((n, k // 2), torch.uint8)
    cs = Canary((n, k // g), TORCH_SZ[sz])
    cz = Canary((n, k // g), TORCH_SZ[sz])
    w4.quantize_pack_int4_sym(to_dev(w_np, kind), g, TORCH_SZ[sz], out=(cp.tensor, cs.tensor, cz.tensor))
    for c in (cp, cs, cz):
        c.check()
    return to_host(cp.tensor), to_host(cs.tensor), to_host(cz.tensor)


def assert_quant_equal(got, want, rows=None):
    gp, gs, gz = got
    wp, ws, wz = want
    if rows is not None:
        gp, gs, gz = gp[rows], gs[rows], gz[rows]
    bad = np.argwhere(gp != wp)
    assert bad.size == 0, f"{len(bad)} packed bytes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(bits(gs), bits(ws)), "scales differ"
    assert np.array_equal(bits(gz), bits(wz)), "zeros differ"


# every group-size path of the quantizer (one to sixteen lanes per group, the
# one-wave-per-group kernel for 96 and 640), ragged row counts and tails
SMALL = [(37, 640, 32), (37, 640, 64), (5, 640, 128), (3, 1024, 256), (2, 1536, 512),
         (7, 384, 96), (3, 640, 640), (129, 256, 128), (1, 32, 32)]


@pytest.mark.parametrize("n,k,g", SMALL)
@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("sz", ["f16", "f32"])
def test_sym_quantize_small(w4, n, k, g, kind, sz):
    rng = np.random.default_rng(2000 + n + k + g)
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 500), replace=False)] = -0.5
    w[0, :g] = np.abs(w[0, :g])          # one-signed group
    if n > 2:
        w[2, :g] = 0.25                  # constant group
    src = WL.bf16_round_bits(w) if kind == "bf16" else w
    assert_quant_equal(gpu_quantize_sym(w4, src, kind, g, sz), O.quantize_pack_int4_sym(src, kind, g, sz))


def test_sym_quantize_worked_example(w4):
    for kind in ("f32", "bf16"):
        vals, codes = PINS.worked_example_sym_group(kind)
        w = np.stack([vals, vals[::-1], -vals, np.zeros(32, np.float32)])
        src = w if kind == "f32" else O.to_bf16(w)
        for sz in ("f16", "f32"):
            got = gpu_quantize_sym(w4, src, kind, 32, sz)
            assert_quant_equal(got, O.quantize_pack_int4_sym(src, kind, 32, sz))
            assert np.array_equal(O.unpack_nibbles(got[0])[0], codes)
            assert float(got[1][0, 0]) == 2.0 ** -6 and float(got[2][0, 0]) == 8.0


def test_sym_quantize_special_groups(w4):
    """Zero, signed-zero and constant groups; a scale that underflows fp16;
    an fp16-subnormal scale that reaches the -8 code; a tiny fp32 range."""
    g = 32
    t = np.float32(2.0 ** -24)
    w = np.zeros((5, 2 * g), np.float32)
    w[0, g:] = -3.0
    w[1, :5] = np.array([-10, 10, 7.5, -8.5, -7.5], np.float32) * t
    w[1, g:g + 15] = np.arange(-7, 8) * np.float32(2.0 ** -27)
    w[2, ::2] = -0.0
    w[3, :g] = np.arange(-16, 16) * np.float32(1e-30)
    w[4] = np.linspace(1.0, 2.5, 2 * g, dtype=np.float32)
    for sz in ("f16", "f32"):
        got = gpu_quantize_sym(w4, w, "f32", g, sz)
        assert_quant_equal(got, O.quantize_pack_int4_sym(w, "f32", g, sz))
    got16 = gpu_quantize_sym(w4, w, "f32", g, "f16")
    assert O.unpack_nibbles(got16[0])[1, :5].tolist() == [0, 15, 15, 0, 0]


@pytest.mark.parametrize("name,g,sz", [("W1", 32, "f32"), ("W1", 32, "f16"), ("Wa", 128, "f16"),
                                       ("Wb", 128, "f16"), ("We", 128, "f16")])
def test_sym_quantize_workloads(w4, name, g, sz):
    """Full-size workload weights; every row of the smaller ones, 256 sampled
    rows (plus first and last) of the largest."""
    t = WL.weight(name)
    got = gpu_quantize_sym(w4, t.data, t.kind, g, sz)
    n = t.shape[0]
    if n * t.shape[1] <= 64 * 1024 * 1024:
        assert_quant_equal(got, O.quantize_pack_int4_sym(t.data, t.kind, g, sz))
    else:
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(4).choice(n, 256, replace=False)]))
        assert_quant_equal(got, O.quantize_pack_int4_sym(t.data[rows], t.kind, g, sz), rows=rows)


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("sz", ["f16", "f32"])
def test_sym_dequant(w4, out, sz):
    n, k, g = 37, 640, 128
    w = np.random.default_rng(31).normal(0, 0.05, (n, k)).astype(np.float32)
    P, S, Z = O.quantize_pack_int4_sym(w, "f32", g, sz)
    c = Canary((n, k), {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out])
    w4.dequant_int4(to_dev(P, "u8"), to_dev(S, sz), to_dev(Z, sz), g, out_dtype=c.tensor.dtype, out=c.tensor)
    c.check()
    assert np.array_equal(bits(to_host(c.tensor)), bits(O.dequant(P, S, Z, g, out)))


def sym_weights_on_gpu(w4, n, k, g, sz, seed, sigma=0.02):
    """Symmetric quantization on the GPU, checked bit-exact against the
    oracle, and both copies returned."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0, sigma, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 1000), replace=False)] = 0.5
    wb = WL.bf16_round_bits(w)
    dev = w4.quantize_pack_int4_sym(to_dev(wb, "bf16"), g, TORCH_SZ[sz])
    host = O.quantize_pack_int4_sym(wb, "bf16", g, sz)
    assert_quant_equal(tuple(to_host(t) for t in dev), host)
    return dev, host


# (m, n, k, g, sz, y): one token (dot2 GEMV), two to four (LDS decode), up to
# 128 (MFMA GEMV), larger M (MFMA GEMM), groups that are not multiples of 128
# (generic kernel), fp32 scales
W4A16_SYM = [(1, 300, 4096, 128, "f16", "bf16"), (1, 77, 640, 128, "f32", "f32"),
             (2, 130, 4096, 128, "f16", "bf16"), (3, 70, 4096, 128, "f16", "bf16"),
             (4, 64, 1536, 128, "f16", "f32"), (16, 300, 2560, 128, "f16", "bf16"),
             (64, 129, 11008, 128, "f16", "bf16"), (100, 70, 1024, 256, "f32", "bf16"),
             (200, 300, 1024, 128, "f16", "bf16"), (513, 256, 512, 128, "f16", "f32"),
             (3, 40, 384, 96, "f16", "bf16"), (9, 64, 640, 32, "f32", "bf16")]


@pytest.mark.parametrize("m,n,k,g,sz,ykind", W4A16_SYM)
def test_sym_w4a16(w4, m, n, k, g, sz, ykind):
    dev, (P, S, Z) = sym_weights_on_gpu(w4, n, k, g, sz, seed=m + 3 * n + k)
    x = WL.bf16_round_bits(np.random.default_rng(m + 41).normal(0, 1, (m, k)).astype(np.float32))
    c = Canary((m, n), TDT[ykind])
    w4.w4a16_matmul(to_dev(x, "bf16"), *dev, g, out=c.tensor)
    c.check()
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    assert O.max_rel_err(y_as_f64(c.tensor), ref) <= TOL[ykind]


# one token (dot4), up to 16 (int8 MFMA GEMV), larger M (int8 MFMA GEMM),
# group 32 (generic)
W4A8_SYM = [(1, 300, 8192, 128, "f16"), (3, 100, 4096, 128, "f16"), (8, 129, 1280, 256, "f32"),
            (40, 300, 1024, 128, "f16"), (300, 200, 768, 128, "f16"), (5, 64, 384, 32, "f16")]


@pytest.mark.parametrize("m,n,k,g,sz", W4A8_SYM)
@pytest.mark.parametrize("ykind", ["bf16", "f32"])
def test_sym_w4a8(w4, m, n, k, g, sz, ykind):
    dev, (P, S, Z) = sym_weights_on_gpu(w4, n, k, g, sz, seed=7 * m + n + k, sigma=0.015)
    rng = np.random.default_rng(m + 43)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 20), replace=False)] *= 20
    xb = WL.bf16_round_bits(x)
    xq, xs = w4.quantize_act_int8(to_dev(xb, "bf16"))
    oq, os_ = O.act_quant_int8(O.widen_bf16(xb))
    assert np.array_equal(to_host(xq), oq) and np.array_equal(bits(to_host(xs)), bits(os_))
    c = Canary((m, n), TDT[ykind])
    w4.w4a8_matmul(xq, xs, *dev, g, out=c.tensor)
    c.check()
    ref = O.matmul_w4a8_f64(oq, os_, P, S, Z, g)
    assert O.max_rel_err(y_as_f64(c.tensor), ref) <= TOL[ykind]


def _signed_integer_weights(rng, n, k, g):
    """Integers in [-7, 7] with |w| = 7 in every group (scale 1, codes w + 8)."""
    wi = rng.integers(-7, 8, (n, k))
    for r in range(n):
        for gi in range(k // g):
            wi[r, gi * g + rng.integers(0, g)] = 7 if rng.integers(0, 2) else -7
    return wi


@pytest.mark.parametrize("m,n,k", [(1, 64, 4096), (3, 48, 4096), (16, 64, 1024), (300, 130, 512)])
def test_sym_exact_integers(w4, m, n, k):
    """Signed integer weights and integer x: both products are exact integers
    below 2^24, so the bf16 outputs equal the correctly rounded exact values."""
    g = 128
    rng = np.random.default_rng(9 * m + n)
    wi = _signed_integer_weights(rng, n, k, g)
    p, s, z = w4.quantize_pack_int4_sym(to_dev(wi.astype(np.float32), "f32"), g, torch.float16)
    assert (to_host(s) == 1.0).all() and (to_host(z) == 8.0).all()
    assert np.array_equal(O.unpack_nibbles(to_host(p)).astype(np.int64), wi + 8)
    xi = rng.integers(-8, 9, (m, k))
    y = w4.w4a16_matmul(to_dev(WL.bf16_round_bits(xi.astype(np.float32)), "bf16"), p, s, z, g)
    assert np.array_equal(to_host(y), O.to_bf16((xi @ wi.T).astype(np.float32)))
    x8 = rng.integers(-127, 128, (m, k))
    x8[:, 0] = 127
    xq, xs = w4.quantize_act_int8(to_dev(WL.bf16_round_bits(x8.astype(np.float32)), "bf16"))
    y8 = w4.w4a8_matmul(xq, xs, p, s, z, g)
    assert np.array_equal(to_host(y8), O.to_bf16((x8 @ wi.T).astype(np.float32)))


# ---------------------------------------------------------------------------
# Range-clipping calibrators: bit-exact against the oracle
# ---------------------------------------------------------------------------
def gpu_quantize_cal(w4, w_np, kind, g, sz, method, param):
    n, k = w_np.shape
    cp = Canary((n, k // 2), torch.uint8)
    cs = Canary((n, k // g), TORCH_SZ[sz])
    cz = Canary((n, k // g), TORCH_SZ[sz])
    fn = w4.quantize_pack_int4_sym_percentile if method == "percentile" else w4.quantize_pack_int4_sym_mse
    fn(to_dev(w_np, kind), g, param, TORCH_SZ[sz], out=(cp.tensor, cs.tensor, cz.tensor))
    for c in (cp, cs, cz):
        c.check()
    return to_host(cp.tensor), to_host(cs.tensor), to_host(cz.tensor)


def oracle_cal(w_np, kind, g, sz, method, param):
    if method == "percentile":
        return O.quantize_pack_int4_sym_percentile(w_np, kind, g, sz, param)
    return O.quantize_pack_int4_sym_mse(w_np, kind, g, sz, param)


@pytest.mark.parametrize("n,k,g", [(37, 640, 32), (5, 640, 128), (3, 1024, 256), (2, 1536, 512),
                                   (7, 384, 96), (2, 2048, 1024), (129, 256, 128)])
@pytest.mark.parametrize("p", [99.9, 50.0, 100.0, 0.001])
@pytest.mark.parametrize("kind,sz", [("bf16", "f16"), ("f32", "f32"), ("f32", "f16")])
def test_percentile_small(w4, n, k, g, p, kind, sz):
    rng = np.random.default_rng(3000 + n + k + g)
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 300), replace=False)] = -0.4
    if n > 2:
        w[2, :g] = 0.0                      # all-zero group
        w[1, :g] = np.float32(0.125)        # constant group: ties everywhere
    src = WL.bf16_round_bits(w) if kind == "bf16" else w
    got = gpu_quantize_cal(w4, src, kind, g, sz, "percentile", p)
    assert_quant_equal(got, oracle_cal(src, kind, g, sz, "percentile", p))


@pytest.mark.parametrize("n,k,g,cand", [(9, 640, 128, 1000), (37, 256, 32, 200), (3, 1024, 256, 300),
                                        (2, 2048, 1024, 50), (5, 384, 96, 64), (4, 256, 128, 2)])
@pytest.mark.parametrize("kind,sz", [("bf16", "f16"), ("f32", "f32")])
def test_mse_small(w4, n, k, g, cand, kind, sz):
    rng = np.random.default_rng(4000 + n + k + g)
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 300), replace=False)] = 0.4
    if n > 2:
        w[2, :g] = 0.0
    src = WL.bf16_round_bits(w) if kind == "bf16" else w
    got = gpu_quantize_cal(w4, src, kind, g, sz, "mse", cand)
    assert_quant_equal(got, oracle_cal(src, kind, g, sz, "mse", cand))


def test_mse_pinned_groups(w4):
    """The groups that pin the search: an exact grid (n = 8), a three-way
    tie (n = 11), the -7 clamp (n = 9), skipped candidates (n = 10)."""
    g = 32
    u = 2.0 ** -7
    j = np.array(list(range(-7, 8)) + [3, -3, 0, 7, -7, 1, 2, -1, -2, 5, -5, 4, -4, 6, -6, 0, 2])
    rows = {8: (j * u).astype(np.float32),
            11: np.array([0.0] * 16 + [5.0] * 16, np.float32)[np.random.default_rng(2).permutation(32)],
            9: np.array([-8.0] * 16 + [7.0] + [0.0] * 15, np.float32),
            10: np.where(np.arange(32) < 4, np.float32(5e-11), np.float32(0.0)).astype(np.float32)}
    want_step = {8: u, 11: 1.0, 9: 2.0, 10: 1.0}
    for cand, row in rows.items():
        w = np.stack([row, -row[::-1]])
        for sz in ("f16", "f32"):
            got = gpu_quantize_cal(w4, w, "f32", g, sz, "mse", cand)
            assert_quant_equal(got, oracle_cal(w, "f32", g, sz, "mse", cand))
            if sz == "f16":
                assert float(got[1][0, 0]) == want_step[cand], (cand, float(got[1][0, 0]))


def _mse_tie_rows(rng, rows, k):
    """Rows whose groups make the search's quotients w / c land exactly on,
    or one ulp beside, half-integers: each group holds 0 and 63 * 2^-10, so
    with 64 candidates c_i = i * 2^-10 exactly, and the other values are
    (k + 1/2) * j * 2^-10 for odd j (steps with inexact reciprocals), nudged
    by -1, 0 or +1 ulp, with random signs."""
    u = 2.0 ** -10
    vals = []
    for j in range(3, 64, 2):
        for kk in range(7):
            if (kk + 0.5) * j <= 63:
                base = np.float32((kk + 0.5) * j * u)
                for d in (-1, 0, 1):
                    vals.append((base.view(np.int32) + d).view(np.float32))
    vals = np.array(vals, np.float32)
    w = rng.choice(vals, (rows, k)) * rng.choice(np.float32([-1, 1]), (rows, k))
    w[:, 0::32] = 0.0
    w[:, 1::32] = np.float32(63 * u)
    return w.astype(np.float32)


@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("sz", ["f16", "f32"])
def test_mse_quotient_ties(w4, g, sz):
    """Quotients on and beside half-integers (here about 90 of every 64,000
    quotients take the other side when computed with the rounded reciprocal
    1/c), so the kernel's near-tie path, the correctly rounded division, runs
    often; the outputs must still equal the oracle's bit for bit.  (Which
    side a near-tie takes moves an error by about one ulp of the step, so it
    rarely changes the chosen step; the division itself is pinned against
    torch on the CPU.)"""
    w = _mse_tie_rows(np.random.default_rng(4100 + g), 48, 256)
    got = gpu_quantize_cal(w4, w, "f32", g, sz, "mse", 64)
    assert_quant_equal(got, oracle_cal(w, "f32", g, sz, "mse", 64))


@pytest.mark.parametrize("p", [12.345, 33.3, 66.6, 99.99])
def test_percentile_both_interpolation_ends(w4, p):
    """Percentiles whose rank fraction lies below and above 1/2 (read from
    the lower or the upper order statistic)."""
    rng = np.random.default_rng(4200)
    w = (rng.normal(0, 0.02, (64, 512)) * 10.0 ** rng.uniform(-3, 1, (64, 1))).astype(np.float32)
    for g in (32, 128):
        got = gpu_quantize_cal(w4, w, "f32", g, "f32", "percentile", p)
        assert_quant_equal(got, oracle_cal(w, "f32", g, "f32", "percentile", p))


def test_calibrators_workload(w4):
    """The 4096 x 4096 weight (bf16, g = 128, fp16 scales): percentile on
    every row, MSE search (1000 candidates) on 64 sampled rows."""
    t = WL.weight("Wa")
    got = gpu_quantize_cal(w4, t.data, t.kind, 128, "f16", "percentile", 99.9)
    assert_quant_equal(got, oracle_cal(t.data, t.kind, 128, "f16", "percentile", 99.9))
    got = gpu_quantize_cal(w4, t.data, t.kind, 128, "f16", "mse", 1000)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(6).choice(4096, 62, replace=False)]))
    assert_quant_equal(got, oracle_cal(t.data[rows], t.kind, 128, "f16", "mse", 1000), rows=rows)


@pytest.mark.parametrize("m", [1, 16, 200])
def test_calibrated_weights_matmul(w4, m):
    """MSE-calibrated weights through the product (decode and GEMM paths)."""
    n, k, g = 300, 1024, 128
    w = np.random.default_rng(51).normal(0, 0.02, (n, k)).astype(np.float32)
    wb = WL.bf16_round_bits(w)
    dev = w4.quantize_pack_int4_sym_mse(to_dev(wb, "bf16"), g, 500, torch.float16)
    P, S, Z = O.quantize_pack_int4_sym_mse(wb, "bf16", g, "f16", 500)
    assert_quant_equal(tuple(to_host(t) for t in dev), (P, S, Z))
    x = WL.bf16_round_bits(np.random.default_rng(m).normal(0, 1, (m, k)).astype(np.float32))
    y = w4.w4a16_matmul(to_dev(x, "bf16"), *dev, g)
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL["bf16"]
