"""GPU parity: w4a16_matmul and w4a8_matmul vs the oracle's float64 products.

Bars (stated with the method's target): max|y - y64| / max|y64| <= 1e-2 for
bf16 outputs and <= 3e-3 for fp32 outputs; bit-exact where the exact result
is representable (integer constructions).  Small M takes the decode kernels,
large M the MFMA kernels; the shapes below reach every path, with ragged
tails in M, N and K.
"""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
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


def make_weights(n, k, g, sz, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, sigma, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 1000), replace=False)] = 0.5
    return O.quantize_pack_int4(w, "f32", g, sz)


def dev_weights(P, S, Z, sz):
    return to_dev(P, "u8"), to_dev(S, sz), to_dev(Z, sz)


def run_w4a16(w4, x_np, xkind, dw, g, ykind, canary=True):
    m = x_np.shape[0]
    n = dw[0].shape[0]
    xt = to_dev(x_np, xkind)
    if canary:
        c = Canary((m, n), TDT[ykind])
        w4.w4a16_matmul(xt, *dw, g, out=c.tensor)
        c.check()
        return c.tensor
    y = w4.w4a16_matmul(xt, *dw, g, out_dtype=TDT[ykind])
    torch.cuda.synchronize()
    return y


SHAPES = [  # (m, n, k, g)
    (1, 300, 640, 128), (2, 77, 384, 128), (4, 300, 1024, 128), (8, 129, 640, 128),
    (1, 64, 640, 32), (3, 40, 384, 96),
    (9, 300, 640, 128), (16, 256, 512, 128), (17, 300, 384, 128), (33, 129, 640, 128),
    (64, 520, 1024, 128), (130, 300, 640, 128), (256, 512, 768, 128), (100, 96, 640, 64),
]


@pytest.mark.parametrize("m,n,k,g", SHAPES)
@pytest.mark.parametrize("sz", ["f16", "f32"])
def test_w4a16_bf16(w4, m, n, k, g, sz):
    P, S, Z = make_weights(n, k, g, sz, seed=m * 1000 + n + k)
    x = WL.bf16_round_bits(np.random.default_rng(m + 5).normal(0, 1, (m, k)).astype(np.float32))
    y = run_w4a16(w4, x, "bf16", dev_weights(P, S, Z, sz), g, "bf16")
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    err = O.max_rel_err(y_as_f64(y), ref)
    assert err <= TOL["bf16"], err


# Decode shapes for the MFMA GEMV (M <= 128, groups a multiple of 128): one to
# sixteen 512-column slices, one to four blocks of 16 tokens with ragged last
# blocks, ragged row counts (workgroups of 32 or 16 rows), groups spanning
# several blocks, both scale and output dtypes.
DECODE = [(1, 33, 512, 128, "f16", "bf16"), (1, 4096, 4096, 128, "f16", "f32"),
          (2, 100, 1536, 128, "f32", "bf16"), (3, 77, 2048, 256, "f16", "bf16"),
          (5, 64, 8192, 128, "f16", "bf16"), (8, 130, 4096, 512, "f32", "f32"),
          (13, 31, 1024, 128, "f16", "f32"), (16, 300, 2560, 128, "f16", "bf16"),
          (1, 17, 8192, 1024, "f16", "bf16"), (16, 1, 512, 512, "f32", "bf16"),
          (17, 100, 1024, 128, "f16", "bf16"), (32, 300, 4096, 128, "f16", "bf16"),
          (33, 65, 512, 256, "f32", "f32"), (48, 40, 1536, 128, "f16", "bf16"),
          (64, 129, 2048, 128, "f16", "f32"),
          # K not a whole number of 512-column slices per wave (the slice loop,
          # with a partial last slice): Llama-7B down-projection K and others
          (5, 70, 640, 128, "f16", "bf16"), (12, 33, 11008, 128, "f16", "f32"),
          (24, 130, 1152, 128, "f32", "bf16"), (40, 64, 11008, 128, "f16", "bf16"),
          (64, 96, 2688, 128, "f16", "bf16"), (20, 50, 1280, 256, "f16", "bf16"),
          (6, 40, 9216, 128, "f16", "bf16"),
          # 65..128 tokens: launches of up to 64 tokens
          (65, 48, 1024, 128, "f16", "bf16"), (100, 70, 11008, 128, "f16", "f32"),
          (128, 33, 2048, 256, "f32", "bf16"),
          # two row blocks per workgroup (N >= 8192) with a ragged last one
          (9, 8200, 1024, 128, "f16", "bf16"), (24, 8208, 1536, 256, "f32", "f32"),
          # two to four tokens at K = 4096: the 4x4x4 matrix-core GEMV, groups
          # of 32 .. 4096 columns, ragged last row group, fp32 scales
          (3, 70, 4096, 128, "f16", "bf16"), (2, 33, 4096, 64, "f32", "f32"),
          (4, 130, 4096, 4096, "f16", "bf16"), (3, 16, 4096, 256, "f16", "f32"),
          (4, 1, 4096, 32, "f32", "bf16"), (2, 515, 4096, 1024, "f16", "bf16"),
          # one token, K not a multiple of 2048 (the dot2 kernel's partial
          # last chunk round), up to its K = 12288 limit
          (1, 50, 11008, 128, "f16", "bf16"), (1, 33, 2560, 256, "f32", "f32"),
          (1, 20, 12288, 128, "f16", "bf16"), (1, 7, 640, 128, "f16", "bf16"),
          # one token, K a whole number of 2048-column rounds (no clamps),
          # groups of 128 .. 2048 columns, 384 among them (a group index
          # that is not a shift)
          (1, 33, 2048, 128, "f16", "bf16"), (1, 50, 6144, 256, "f32", "f32"),
          (1, 17, 12288, 128, "f16", "bf16"), (1, 40, 8192, 2048, "f16", "bf16"),
          (1, 20, 6144, 384, "f16", "bf16"), (1, 130, 10240, 128, "f32", "bf16")]


@pytest.mark.parametrize("m,n,k,g,sz,ykind", DECODE)
def test_w4a16_decode_shapes(w4, m, n, k, g, sz, ykind):
    P, S, Z = make_weights(n, k, g, sz, seed=7 * m + n + k)
    x = WL.bf16_round_bits(np.random.default_rng(m + 17).normal(0, 1, (m, k)).astype(np.float32))
    y = run_w4a16(w4, x, "bf16", dev_weights(P, S, Z, sz), g, ykind)
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL[ykind]


@pytest.mark.parametrize("m,n,k,g", [(1, 256, 256, 32), (3, 100, 384, 128), (19, 64, 640, 64)])
@pytest.mark.parametrize("ykind", ["f32", "bf16"])
def test_w4a16_f32_activations(w4, m, n, k, g, ykind):
    P, S, Z = make_weights(n, k, g, "f32", seed=n + k)
    x = np.random.default_rng(m).normal(0, 1, (m, k)).astype(np.float32)
    y = run_w4a16(w4, x, "f32", dev_weights(P, S, Z, "f32"), g, ykind)
    ref = O.matmul_w4a16_f64(x, P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL[ykind]


@pytest.mark.parametrize("m,n,k", [(1, 64, 256), (1, 64, 4096), (8, 48, 512), (16, 64, 256), (40, 300, 1024),
                                   (256, 256, 2048)])
def test_w4a16_exact_integers(w4, m, n, k):
    """W integers 0..15 (each group holding 0 and 15 -> scale 1, zp 0), x
    integers in [-8, 8]: every partial sum is an exact integer below 2^24, so
    the bf16 output must equal the correctly rounded exact product bit for bit."""
    g = 128 if k % 128 == 0 else 32
    rng = np.random.default_rng(m + n + k)
    wi = rng.integers(0, 16, (n, k))
    for r in range(n):
        for gi in range(k // g):
            a, b = rng.choice(g, 2, replace=False)
            wi[r, gi * g + a], wi[r, gi * g + b] = 0, 15
    xi = rng.integers(-8, 9, (m, k))
    wt = to_dev(wi.astype(np.float32), "f32")
    p, s, z = w4.quantize_pack_int4(wt, g, torch.float16)
    y = w4.w4a16_matmul(to_dev(WL.bf16_round_bits(xi.astype(np.float32)), "bf16"), p, s, z, g)
    want = O.to_bf16((xi @ wi.T).astype(np.float32))
    got = to_host(y)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_w4a16_deterministic(w4):
    P, S, Z = make_weights(512, 1024, 128, "f16", seed=4)
    dw = dev_weights(P, S, Z, "f16")
    for m in (1, 8, 64):
        x = WL.bf16_round_bits(np.random.default_rng(m).normal(0, 1, (m, 1024)).astype(np.float32))
        a = to_host(run_w4a16(w4, x, "bf16", dw, 128, "bf16", canary=False))
        b = to_host(run_w4a16(w4, x, "bf16", dw, 128, "bf16", canary=False))
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------
_QCACHE = {}


def quantized(name, g, sz):
    key = (name, g, sz)
    if key not in _QCACHE:
        t = WL.weight(name)
        _QCACHE.clear()
        _QCACHE[key] = (t, O.quantize_pack_int4(t.data, t.kind, g, sz))
    return _QCACHE[key]


def test_workload_single_layer_fp32(w4):
    """256x256 fp32 layer, g=32, fp32 scales, fp32 x and y (tolerance 3e-3)."""
    t, (P, S, Z) = quantized("W1", 32, "f32")
    x = WL.activation(1, 1, 256)
    y = run_w4a16(w4, x.data, "f32", dev_weights(P, S, Z, "f32"), 32, "f32")
    ref = O.matmul_w4a16_f64(x.as_f32(), P, S, Z, 32)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL["f32"]


@pytest.mark.parametrize("name", ["Wa", "Wb"])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16, 32])
def test_workload_llama_decode(w4, name, m):
    """Llama-7B shapes at M = 1 (decode) and 2..32 (small batch)."""
    t, (P, S, Z) = quantized(name, 128, "f16")
    x = WL.activation(2 if m == 1 else 3, m, 4096)
    y = run_w4a16(w4, x.data, "bf16", dev_weights(P, S, Z, "f16"), 128, "bf16")
    ref = O.matmul_w4a16_f64(x.as_f32(), P, S, Z, 128)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL["bf16"]


@pytest.mark.parametrize("m", [1, 3, 17, 64, 100])
def test_workload_llama_down_decode(w4, m):
    """The Llama-7B down projection [4096, 11008] at decode and small-batch
    sizes (K is not a whole number of 512-column slices per wave)."""
    t, (P, S, Z) = quantized("Wd", 128, "f16")
    x = WL.activation(3, m, 11008)
    y = run_w4a16(w4, x.data, "bf16", dev_weights(P, S, Z, "f16"), 128, "bf16")
    ref = O.matmul_w4a16_f64(x.as_f32(), P, S, Z, 128)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL["bf16"]


@pytest.mark.parametrize("name,k", [("Wb", 4096), ("Wd", 11008)])
def test_workload_prefill(w4, name, k):
    """M = 2048 prefill; the oracle checks 96 sampled tokens (plus the first
    and last) against every output column."""
    t, (P, S, Z) = quantized(name, 128, "f16")
    x = WL.activation(4, 2048, k)
    y = run_w4a16(w4, x.data, "bf16", dev_weights(P, S, Z, "f16"), 128, "bf16")
    rows = np.unique(np.concatenate([[0, 2047], np.random.default_rng(9).choice(2048, 96, replace=False)]))
    ref = O.matmul_w4a16_f64(x.as_f32()[rows], P, S, Z, 128)
    got = y_as_f64(y)[rows]
    assert O.max_rel_err(got, ref) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# Split K (w4a16_matmul_ws): shapes whose output tiles fill few compute units
# ---------------------------------------------------------------------------
SPLITK_SHAPES = [  # (m, n, k, g): every one splits K (checked below)
    (200, 300, 2048, 128), (129, 96, 4096, 32), (300, 130, 2048, 256), (257, 520, 4096, 64),
    (133, 77, 1152, 96),
]


@pytest.mark.parametrize("m,n,k,g", SPLITK_SHAPES)
@pytest.mark.parametrize("sz,ykind", [("f16", "bf16"), ("f32", "f32")])
def test_w4a16_split_k(w4, m, n, k, g, sz, ykind):
    """The split-K GEMM (workspace given) against the oracle, against the
    same product without a workspace, and bit for bit across two calls."""
    assert w4.w4a16_matmul_workspace_size(m, k, n, g) > 0
    P, S, Z = make_weights(n, k, g, sz, seed=m + n + g)
    dw = dev_weights(P, S, Z, sz)
    x = WL.bf16_round_bits(np.random.default_rng(m * 3 + k).normal(0, 1, (m, k)).astype(np.float32))
    xt = to_dev(x, "bf16")
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    c = Canary((m, n), TDT[ykind])
    w4.w4a16_matmul(xt, *dw, g, out=c.tensor, workspace="auto")
    c.check()
    assert O.max_rel_err(y_as_f64(c.tensor), ref) <= TOL[ykind]
    again = w4.w4a16_matmul(xt, *dw, g, out_dtype=TDT[ykind], workspace="auto")
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(again)), bits(to_host(c.tensor)))
    plain = w4.w4a16_matmul(xt, *dw, g, out_dtype=TDT[ykind], workspace=None)
    assert O.max_rel_err(y_as_f64(plain), ref) <= TOL[ykind]
    # a workspace one byte short: the library runs the unsplit kernel
    short = torch.empty(w4.w4a16_matmul_workspace_size(m, k, n, g) - 1, dtype=torch.uint8, device="cuda")
    y2 = w4.w4a16_matmul(xt, *dw, g, out_dtype=TDT[ykind], workspace=short)
    assert np.array_equal(bits(to_host(y2)), bits(to_host(plain)))


def _wide(m, n):
    """The GEMM's choice of 192-column tiles (rounds of 256 workgroups)."""
    tm = -(-m // 256)
    r128 = -(-tm * -(-n // 128) // 256)
    r192 = -(-tm * -(-n // 192) // 256)
    return r192 * 1.36 < r128


WIDE_SHAPES = [(600, 22000, 256, 128), (520, 25000, 384, 64), (257, 45000, 256, 32)]


@pytest.mark.parametrize("m,n,k,g", WIDE_SHAPES)
@pytest.mark.parametrize("sz,ykind", [("f16", "bf16"), ("f32", "f32")])
def test_w4a16_wide_tiles(w4, m, n, k, g, sz, ykind):
    """Shapes that take the 192-column GEMM tiles (ragged N, every group
    size path), against the oracle on 48 sampled tokens."""
    assert _wide(m, n)
    P, S, Z = make_weights(n, k, g, sz, seed=n + g)
    x = WL.bf16_round_bits(np.random.default_rng(m + k).normal(0, 1, (m, k)).astype(np.float32))
    y = run_w4a16(w4, x, "bf16", dev_weights(P, S, Z, sz), g, ykind)
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(5).choice(m, 46, replace=False)]))
    ref = O.matmul_w4a16_f64(O.widen_bf16(x)[rows], P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL[ykind]


@pytest.mark.parametrize("m", [129, 256, 512])
def test_workload_down_proj_mid_m(w4, m):
    """The Llama-7B down projection [4096, 11008] at 129 to 512 tokens, where
    the unsplit GEMM has only 32 or 64 tiles: split K with the workspace the
    library asks for; the oracle checks 40 sampled tokens (plus the first
    and last) against every output column."""
    t, (P, S, Z) = quantized("Wd", 128, "f16")
    assert w4.w4a16_matmul_workspace_size(m, 11008, 4096, 128) > 0
    x = WL.activation(3, m, 11008)
    y = run_w4a16(w4, x.data, "bf16", dev_weights(P, S, Z, "f16"), 128, "bf16")
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(m).choice(m, 40, replace=False)]))
    ref = O.matmul_w4a16_f64(x.as_f32()[rows], P, S, Z, 128)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# W4A8
# ---------------------------------------------------------------------------
def run_w4a8(w4, x_np, xkind, dw, g, ykind="bf16"):
    xq, xs = w4.quantize_act_int8(to_dev(x_np, xkind))
    m, n = x_np.shape[0], dw[0].shape[0]
    c = Canary((m, n), TDT[ykind])
    w4.w4a8_matmul(xq, xs, *dw, g, out=c.tensor)
    c.check()
    return c.tensor, to_host(xq), to_host(xs)


W8_SHAPES = [(1, 300, 640, 128), (5, 129, 1024, 128), (8, 64, 384, 32), (16, 300, 640, 128),
             (40, 129, 1024, 128), (130, 256, 512, 128), (64, 96, 640, 64)]


@pytest.mark.parametrize("m,n,k,g", W8_SHAPES)
@pytest.mark.parametrize("ykind", ["bf16", "f32"])
def test_w4a8(w4, m, n, k, g, ykind):
    P, S, Z = make_weights(n, k, g, "f16", seed=m + 3 * n + k, sigma=0.015)
    rng = np.random.default_rng(m + 11)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 20), replace=False)] *= 20
    xb = WL.bf16_round_bits(x)
    y, xq, xs = run_w4a8(w4, xb, "bf16", dev_weights(P, S, Z, "f16"), g, ykind)
    oq, os_ = O.act_quant_int8(O.widen_bf16(xb))
    assert np.array_equal(xq, oq) and np.array_equal(bits(xs), bits(os_))
    ref = O.matmul_w4a8_f64(oq, os_, P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL[ykind]


# Shapes for the int8-MFMA GEMM (M > 16, group a multiple of 128): several
# 256 x 128 tiles with ragged M and N, one K step only, groups of 256 (two K
# steps per group), fp32 scales and zero-points; then the one-token GEMV.
W8_GEMM = [(17, 130, 128, 128, "f16"), (128, 260, 1024, 128, "f16"), (129, 100, 512, 128, "f32"),
           (257, 1000, 2048, 128, "f16"), (300, 200, 768, 256, "f16"),
           (512, 384, 1024, 128, "f32"), (64, 129, 640, 640, "f16"),
           # one to four tokens, group 128, K = 2048 .. 8192: the dot4 GEMV (ragged
           # row counts)
           (1, 1, 2048, 128, "f16"), (1, 300, 4096, 128, "f32"), (1, 17, 6144, 128, "f16"),
           (1, 1000, 8192, 128, "f16"), (3, 300, 4096, 128, "f32"), (4, 100, 2048, 128, "f16"),
           (4, 33, 8192, 128, "f16"),
           # up to 16 tokens, groups a multiple of 128, any K: the int8 MFMA GEMV
           # (slices shared by up to 8 waves, partial last slice)
           (1, 50, 28672, 128, "f16"), (7, 33, 1280, 256, "f16"), (12, 40, 11008, 128, "f32"),
           (2, 17, 8192, 128, "f16"), (16, 64, 128, 128, "f16"),
           # long K with N >= 8192: two row blocks per workgroup, ragged last one
           (16, 8200, 16384, 128, "f16"), (5, 8208, 16384, 256, "f32")]


@pytest.mark.parametrize("m,n,k,g,sz", W8_GEMM)
@pytest.mark.parametrize("ykind", ["bf16", "f32"])
def test_w4a8_gemm(w4, m, n, k, g, sz, ykind):
    P, S, Z = make_weights(n, k, g, sz, seed=5 * m + n + k, sigma=0.015)
    rng = np.random.default_rng(m + 13)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 20), replace=False)] *= 20
    xb = WL.bf16_round_bits(x)
    y, xq, xs = run_w4a8(w4, xb, "bf16", dev_weights(P, S, Z, sz), g, ykind)
    oq, os_ = O.act_quant_int8(O.widen_bf16(xb))
    assert np.array_equal(xq, oq) and np.array_equal(bits(xs), bits(os_))
    ref = O.matmul_w4a8_f64(oq, os_, P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL[ykind]


# Shapes whose int8-GEMM tiles leave most of the GPU idle split K over the
# workspace: ragged M and N, 128- and 256-token tiles, groups of 256 cut by a
# split boundary (K = 2304: 18 steps, splits of 9), fp32 scales.
W8_SPLITK = [(17, 300, 4096, 128, "f16"), (40, 1000, 8192, 128, "f32"), (129, 520, 4096, 128, "f16"),
             (300, 1000, 2304, 256, "f16"), (257, 130, 8192, 128, "f32")]


@pytest.mark.parametrize("m,n,k,g,sz", W8_SPLITK)
@pytest.mark.parametrize("ykind", ["bf16", "f32"])
def test_w4a8_splitk(w4, m, n, k, g, sz, ykind):
    assert w4.w4a8_matmul_workspace_size(m, k, n, g) > 0
    P, S, Z = make_weights(n, k, g, sz, seed=3 * m + n + k, sigma=0.015)
    rng = np.random.default_rng(m + 17)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 20), replace=False)] *= 20
    xb = WL.bf16_round_bits(x)
    y, xq, xs = run_w4a8(w4, xb, "bf16", dev_weights(P, S, Z, sz), g, ykind)
    oq, os_ = O.act_quant_int8(O.widen_bf16(xb))
    ref = O.matmul_w4a8_f64(oq, os_, P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y), ref) <= TOL[ykind]
    # the unsplit schedule meets the same bound
    dw = dev_weights(P, S, Z, sz)
    xq_d, xs_d = to_dev(oq, "i8"), to_dev(os_, "f32")
    plain = w4.w4a8_matmul(xq_d, xs_d, *dw, g, out_dtype=TDT[ykind], workspace=None)
    assert O.max_rel_err(y_as_f64(plain), ref) <= TOL[ykind]
    # deterministic: the split product again, bit for bit; a workspace one
    # byte short of the query runs the unsplit kernel, bit for bit
    nbytes = w4.w4a8_matmul_workspace_size(m, k, n, g)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    again = w4.w4a8_matmul(xq_d, xs_d, *dw, g, out_dtype=TDT[ykind], workspace=ws)
    assert np.array_equal(bits(to_host(again)), bits(to_host(y)))
    short = w4.w4a8_matmul(xq_d, xs_d, *dw, g, out_dtype=TDT[ykind], workspace=ws[: nbytes - 1])
    assert np.array_equal(bits(to_host(short)), bits(to_host(plain)))


def test_w4a8_splitk_tp8_shard(w4):
    """One GPU's 8-way column shard of the [28672, 8192] projection (its first
    3584 rows) at 512 tokens of heavy-tailed activations: 56 tiles, split K;
    64 sampled tokens against the oracle."""
    t = WL.weight("We")
    n, k, g = 3584, 8192, 128
    w = t.data[:n]
    P, S, Z = O.quantize_pack_int4(w, t.kind, g, "f16")
    assert w4.w4a8_matmul_workspace_size(512, k, n, g) > 0
    xb = WL.activation(5, 512, k)
    y, xq, xs = run_w4a8(w4, xb.data, xb.kind, dev_weights(P, S, Z, "f16"), g)
    rows = np.arange(0, 512, 8)
    ref = O.matmul_w4a8_f64(xq[rows], xs[rows], P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL["bf16"]


@pytest.mark.parametrize("m,n,k", [(1, 64, 8192), (3, 48, 4096), (8, 48, 1024), (16, 64, 1024),
                                   (64, 256, 8192), (300, 130, 256)])
def test_w4a8_exact_integers(w4, m, n, k):
    """x integers with |x| <= 127 and 127 present (scale 1, xq = x); W integer
    codes with scale 1, zp 0: y is an exact integer below 2^24 and the bf16
    output must be its correctly rounded value."""
    g = 128
    rng = np.random.default_rng(7 * m + n)
    wi = rng.integers(0, 16, (n, k))
    for r in range(n):
        for gi in range(k // g):
            a, b = rng.choice(g, 2, replace=False)
            wi[r, gi * g + a], wi[r, gi * g + b] = 0, 15
    xi = rng.integers(-127, 128, (m, k))
    xi[:, 0] = 127
    p, s, z = w4.quantize_pack_int4(to_dev(wi.astype(np.float32), "f32"), g, torch.float16)
    xq, xs = w4.quantize_act_int8(to_dev(WL.bf16_round_bits(xi.astype(np.float32)), "bf16"))
    assert (to_host(xs) == 1.0).all()
    y = w4.w4a8_matmul(xq, xs, p, s, z, g)
    want = O.to_bf16((xi @ wi.T).astype(np.float32))
    assert np.array_equal(to_host(y), want)


@pytest.mark.parametrize("m", [1, 512])
def test_workload_w4a8(w4, m):
    """70B-class MLP projection [28672, 8192], heavy-tailed activations; M = 1
    checked in full, M = 512 on 48 sampled tokens (plus first and last)."""
    t, (P, S, Z) = quantized("We", 128, "f16")
    x = WL.activation(5, m, 8192)
    y, xq, xs = run_w4a8(w4, x.data, "bf16", dev_weights(P, S, Z, "f16"), 128)
    oq, os_ = O.act_quant_int8(x.as_f32())
    assert np.array_equal(xq, oq) and np.array_equal(bits(xs), bits(os_))
    rows = np.arange(m) if m == 1 else np.unique(np.concatenate([[0, m - 1], np.random.default_rng(5).choice(m, 48, replace=False)]))
    ref = O.matmul_w4a8_f64(oq[rows], os_[rows], P, S, Z, 128)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL["bf16"]


def test_empty_inputs(w4):
    """Zero tokens or zero weight rows: valid calls that launch nothing and
    return correctly shaped empty outputs."""
    dev = torch.device("cuda")
    p0, s0, z0 = w4.quantize_pack_int4(torch.zeros((0, 256), dtype=torch.bfloat16, device=dev), 128,
                                       torch.float16)
    assert tuple(p0.shape) == (0, 128) and tuple(s0.shape) == (0, 2)
    P, S, Z = make_weights(64, 256, 128, "f16", seed=1)
    dw = dev_weights(P, S, Z, "f16")
    x0 = torch.zeros((0, 256), dtype=torch.bfloat16, device=dev)
    assert tuple(w4.w4a16_matmul(x0, *dw, 128).shape) == (0, 64)
    xq, xs = w4.quantize_act_int8(x0)
    assert tuple(xq.shape) == (0, 256) and tuple(xs.shape) == (0,)
    assert tuple(w4.w4a8_matmul(xq, xs, *dw, 128).shape) == (0, 64)
    x3 = torch.ones((3, 256), dtype=torch.bfloat16, device=dev)
    y = w4.w4a16_matmul(x3, p0, s0, z0, 128)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (3, 0)
