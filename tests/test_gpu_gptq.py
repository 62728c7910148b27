"""GPU parity of the GPTQ path (gptq_hessian, gptq_inverse_cholesky,
gptq_quantize_pack_int4) against oracle/gptq_oracle.py.

Hessian and factor are float64 on both sides and must agree to rounding.
The sweep's integer decisions are taken on values that the GPU updates in
float32, 128 columns at a time, so a decision that lies within 1e-3 of a
rounding boundary may go either way: the oracle replays the sweep in
float64, accepts the GPU's choice only there, and the count of such
choices must stay small.  Everything else must match exactly."""
import numpy as np
import pytest
import torch

import oracle.gptq_oracle as G
import oracle.w4_oracle as O
from tests.gpu_util import TORCH_SZ, bits, to_dev, to_host
from tests.gptq_pins import page_outlier_setup

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def f64_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).cuda()


def _data(n, k, t, seed, wstd=0.05):
    rng = np.random.default_rng(seed)
    return rng.normal(0, wstd, (n, k)).astype(np.float32), rng.normal(0, 1, (t, k)).astype(np.float32)


@pytest.mark.parametrize("t,k", [(5, 1), (37, 100), (256, 384), (64, 1024)])
def test_hessian(w4, t, k):
    _, x = _data(1, k, t, 100 + k)
    h = to_host(w4.gptq_hessian(to_dev(x, "f32")))
    ref = G.gptq_hessian(x)
    assert np.abs(h - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.array_equal(bits(h), bits(np.ascontiguousarray(h.T)))


@pytest.mark.parametrize("k,t", [(1, 3), (7, 20), (64, 100), (100, 40), (200, 64), (640, 2000)])
def test_inverse_cholesky(w4, k, t):
    _, x = _data(1, k, t, 200 + k)
    h = G.gptq_hessian(x)                   # t < k: rank-deficient data, damping decides
    u = to_host(w4.gptq_inverse_cholesky(f64_dev(h)))
    ref = G.gptq_inverse_cholesky(h)
    assert np.all(np.tril(u, -1) == 0)
    assert np.abs(u - ref).max() <= 1e-9 * np.abs(ref).max(), np.abs(u - ref).max() / np.abs(ref).max()
    assert np.abs(u @ h @ u.T - np.eye(k)).max() <= 1e-8


def test_inverse_cholesky_reads_upper_triangle_only(w4):
    _, x = _data(1, 96, 200, 7)
    h = G.gptq_hessian(x)
    hh = h.copy()
    hh[np.tril_indices(96, -1)] = np.nan
    u = to_host(w4.gptq_inverse_cholesky(f64_dev(hh)))
    assert np.array_equal(bits(u), bits(to_host(w4.gptq_inverse_cholesky(f64_dev(h)))))


@pytest.mark.parametrize("diag,want", [((1.0, 1.0, -1.0, 1.0), 3), ((2.0, 0.0, 1.0, 1.0), 2),
                                       ((0.0,) * 70, 70), ((1.0,) * 130, 0)])
def test_inverse_cholesky_info(w4, diag, want):
    """info names the first non-positive pivot in visiting order (last
    column first), 1-based; 0 for a positive definite matrix."""
    u, info = w4.gptq_inverse_cholesky(f64_dev(np.diag(diag)), check=False)
    assert int(info.item()) == want
    if want:
        with pytest.raises(ValueError, match="not positive definite"):
            w4.gptq_inverse_cholesky(f64_dev(np.diag(diag)))


def _replay_ok(w, u, g, sz, symmetric, out, codes_frac=5e-3, zeros_frac=1e-2):
    """Replay with the GPU's decisions as the guide (scales held to about one
    unit in their last place, codes and zero-points to near-ties only)."""
    packed, s, z = (to_host(a) for a in out)
    _, _, _, stats, _ = G.gptq_quantize(w, u, g, sz, symmetric, guide=(packed, s, z))
    n, k = w.shape
    assert stats["codes_accepted"] <= max(2, codes_frac * n * k), stats
    assert stats["zeros_accepted"] <= max(2, zeros_frac * n * (k // g)), stats
    if symmetric:
        assert np.all(z == 8)
    return stats


SWEEP_CASES = [  # n, k, g, symmetric, sz, calibration rows
    (37, 256, 32, False, "f16", 300),
    (130, 384, 128, True, "f32", 200),
    (64, 512, 256, False, "f16", 600),
    (200, 352, 32, True, "f16", 100),      # last block 96 columns
    (16, 640, 64, False, "f32", 1000),
    (1, 128, 128, False, "f16", 50),
    (129, 768, 384, True, "f16", 800),     # a group of three blocks
    (50, 1024, 1024, False, "f16", 300),   # one group per row, eight blocks
    (300, 96, 32, False, "f32", 40),       # one partial block of 96 columns
]


@pytest.mark.parametrize("n,k,g,symmetric,sz,t", SWEEP_CASES)
def test_sweep_with_oracle_factor(w4, n, k, g, symmetric, sz, t):
    w, x = _data(n, k, t, n + k + g)
    u = G.gptq_inverse_cholesky(G.gptq_hessian(x))
    wd = to_dev(w, "f32")
    out = w4.gptq_quantize_pack_int4(wd, f64_dev(u), g, symmetric, TORCH_SZ[sz])
    assert np.array_equal(to_host(wd), w)          # the wrapper sweeps a copy
    _replay_ok(w, u, g, sz, symmetric, out)


def test_sweep_diagonal_hessian_is_rtn(w4):
    """A diagonal Hessian couples nothing: the sweep must give the
    round-to-nearest quantizers' outputs bit for bit."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.05, (70, 512)).astype(np.float32)
    u = G.gptq_inverse_cholesky(np.diag(rng.uniform(0.5, 2.0, 512)))
    for symmetric, fn in ((False, O.quantize_pack_int4), (True, O.quantize_pack_int4_sym)):
        for g in (32, 128, 256):
            got = w4.gptq_quantize_pack_int4(to_dev(w, "f32"), f64_dev(u), g, symmetric, torch.float16)
            want = fn(w, "f32", g, "f16")
            for a, b in zip(got, want):
                assert np.array_equal(bits(to_host(a)), bits(b)), (symmetric, g)


def test_end_to_end_page_setup(w4):
    """The page's outlier setup through all three GPU calls; the replay uses
    the oracle's own Hessian and factor; the layer-output error beats
    round-to-nearest as the oracle's does."""
    w, x = page_outlier_setup()
    wd = to_dev(w, "f32")
    h = w4.gptq_hessian(to_dev(x, "f32"))
    u = w4.gptq_inverse_cholesky(h)
    for symmetric in (False, True):
        out = w4.gptq_quantize_pack_int4(wd, u, 128, symmetric, torch.float16)
        href = G.gptq_hessian(x)
        _replay_ok(w, G.gptq_inverse_cholesky(href), 128, "f16", symmetric, out)
        rtn = (O.quantize_pack_int4_sym if symmetric else O.quantize_pack_int4)(w, "f32", 128, "f16")
        lg = G.proxy_loss(w, O.dequant_f64(*(to_host(a) for a in out), 128), href)
        lr = G.proxy_loss(w, O.dequant_f64(*rtn, 128), href)
        assert lg < 0.5 * lr


def test_end_to_end_page_demo_and_layer(w4):
    """The page's demo shape (1024 x 1024 weight, 256 calibration rows,
    group 128) through QuantizedLinear(mode="gptq"); its forward against the
    oracle's product of the same codes."""
    w, x = _data(1024, 1024, 256, 0)
    layer = w4.QuantizedLinear.from_weight(to_dev(w, "f32"), group_size=128, mode="gptq",
                                           param=to_dev(x, "f32"))
    out = (layer.packed, layer.scales, layer.zeros)
    _replay_ok(w, G.gptq_inverse_cholesky(G.gptq_hessian(x)), 128, "f16", False, out)
    xt = np.random.default_rng(1).normal(0, 1, (8, 1024)).astype(np.float32)
    y = layer(to_dev(xt, "f32")).double().cpu().numpy()
    ref = O.matmul_w4a16_f64(xt, *(to_host(a) for a in out), 128)
    assert O.max_rel_err(y, ref) <= 3e-3


def test_llama_gate_shape_sampled_rows(w4):
    """[11008, 4096] weight, 4096 calibration rows, group 128 (the benchmark
    shape): full Hessian and factor against the oracle; the sweep replayed on
    sampled rows (rows are independent)."""
    n, k, t, g = 11008, 4096, 4096, 128
    w, x = _data(n, k, t, 42, wstd=0.02)
    h = w4.gptq_hessian(to_dev(x, "f32"))
    href = G.gptq_hessian(x)
    hh = to_host(h)
    assert np.abs(hh - href).max() <= 1e-12 * np.abs(href).max()
    u = w4.gptq_inverse_cholesky(h, overwrite_h=True)
    uref = G.gptq_inverse_cholesky(href)
    uu = to_host(u)
    assert np.abs(uu - uref).max() <= 1e-9 * np.abs(uref).max()
    out = w4.gptq_quantize_pack_int4(to_dev(w, "f32"), u, g, False, torch.float16)
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(n, 12, replace=False)
    rows = np.concatenate([rows, [0, n - 1]])
    p, s, z = (to_host(a)[rows] for a in out)
    _, _, _, stats, _ = G.gptq_quantize(w[rows], uref, g, "f16", False, guide=(p, s, z))
    assert stats["codes_accepted"] <= max(2, 5e-3 * len(rows) * k), stats


def test_layer_gptq_sym_bf16(w4):
    """QuantizedLinear(mode="gptq_sym") from a bf16 weight: the layer quantizes
    the weight's float32 values; codes checked by the oracle's replay, the
    forward against the oracle's product of the same codes."""
    import workloads as WL
    w, x = _data(256, 512, 400, 9)
    wb = WL.bf16_round_bits(w)
    layer = w4.QuantizedLinear.from_weight(to_dev(wb, "bf16"), group_size=64, mode="gptq_sym",
                                           param=to_dev(x, "f32"))
    out = (layer.packed, layer.scales, layer.zeros)
    _replay_ok(O.widen_bf16(wb), G.gptq_inverse_cholesky(G.gptq_hessian(x)), 64, "f16", True, out)
    xt = WL.bf16_round_bits(np.random.default_rng(2).normal(0, 1, (3, 512)).astype(np.float32))
    y = layer(to_dev(xt, "bf16")).float().cpu().numpy().astype(np.float64)
    ref = O.matmul_w4a16_f64(O.widen_bf16(xt), *(to_host(a) for a in out), 64)
    assert O.max_rel_err(y, ref) <= 1e-2
