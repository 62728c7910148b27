"""GPU parity: quantize_pack_int4, dequant_int4, quantize_act_int8 vs the oracle.

Bar: bit-exact (packed bytes, scale and zero-point bit patterns, dequantized
values, int8 codes and activation scales).
"""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests import oracle_pins as PINS
from tests.gpu_util import TORCH_SZ, Canary, bits, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def gpu_quantize(w4, w_np, kind, g, sz, canary=False):
    wt = to_dev(w_np, kind)
    n, k = w_np.shape
    if canary:
        cp = Canary((n, k // 2), torch.uint8)
        cs = Canary((n, k // g), TORCH_SZ[sz])
        cz = Canary((n, k // g), TORCH_SZ[sz])
        w4.quantize_pack_int4(wt, g, TORCH_SZ[sz], out=(cp.tensor, cs.tensor, cz.tensor))
        for c in (cp, cs, cz):
            c.check()
        p, s, z = cp.tensor, cs.tensor, cz.tensor
    else:
        p, s, z = w4.quantize_pack_int4(wt, g, TORCH_SZ[sz])
    torch.cuda.synchronize()
    return to_host(p), to_host(s), to_host(z)


def assert_quant_equal(got, want, rows=None):
    gp, gs, gz = got
    wp, ws, wz = want
    if rows is not None:
        gp, gs, gz = gp[rows], gs[rows], gz[rows]
    assert gp.shape == wp.shape and gs.shape == ws.shape
    bad = np.argwhere(gp != wp)
    assert bad.size == 0, f"{len(bad)} packed bytes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(bits(gs), bits(ws)), "scales differ"
    assert np.array_equal(bits(gz), bits(wz)), "zeros differ"


SMALL = [  # (n, k, g): several tiles and ragged tails for every path
    (37, 640, 32), (37, 640, 64), (5, 640, 128), (3, 1024, 256), (2, 1536, 512),
    (7, 384, 96), (3, 640, 640), (1, 4096, 4096), (129, 256, 128), (1, 32, 32),
]


@pytest.mark.parametrize("n,k,g", SMALL)
@pytest.mark.parametrize("kind", ["bf16", "f32"])
@pytest.mark.parametrize("sz", ["f16", "f32"])
def test_quantize_small(w4, n, k, g, kind, sz):
    rng = np.random.default_rng(1000 + n + k + g)
    w = rng.normal(0, 0.02, (n, k)).astype(np.float32)
    w.reshape(-1)[rng.choice(n * k, max(1, n * k // 500), replace=False)] = 0.5
    w[0, :g] = np.abs(w[0, :g])          # clamped zero-point
    if n > 2:
        w[2, :g] = 0.25                  # constant group
    src = WL.bf16_round_bits(w) if kind == "bf16" else w
    got = gpu_quantize(w4, src, kind, g, sz, canary=True)
    assert_quant_equal(got, O.quantize_pack_int4(src, kind, g, sz))


def test_quantize_worked_example(w4):
    vals, codes = PINS.worked_example_group()
    w = np.stack([vals, vals[::-1], -vals, np.zeros(32, np.float32)])
    for sz in ("f16", "f32"):
        for kind in ("f32", "bf16"):
            src = w if kind == "f32" else O.to_bf16(w)
            got = gpu_quantize(w4, src, kind, 32, sz)
            assert_quant_equal(got, O.quantize_pack_int4(src, kind, 32, sz))
            assert np.array_equal(O.unpack_nibbles(got[0])[0], codes)
            assert float(got[1][0, 0]) == 2.0 ** -6 and float(got[2][0, 0]) == 5.0


def test_quantize_special_groups(w4):
    g = 32
    w = np.zeros((6, 2 * g), np.float32)
    w[0, :g] = 3.0
    w[0, g:] = -3.0
    w[1, :g] = (np.arange(g) % 16) * np.float32(2.0 ** -20)   # fp16-subnormal scale
    w[1, g:] = (np.arange(g) % 16) * np.float32(2.0 ** -27)   # scale underflows fp16
    w[2] = np.linspace(1.0, 2.5, 2 * g, dtype=np.float32)      # zp clamps to 0
    w[3] = -w[2]                                               # zp clamps to 15
    w[4, ::2] = -0.0                                           # signed zeros
    w[5] = np.float32(1e-30) * np.arange(2 * g)                # tiny fp32 range
    for sz in ("f16", "f32"):
        got = gpu_quantize(w4, w, "f32", g, sz)
        assert_quant_equal(got, O.quantize_pack_int4(w, "f32", g, sz))
        assert not np.signbit(got[2].astype(np.float32)).any()


@pytest.mark.parametrize("name,g,sz", [("W1", 32, "f32"), ("W1", 32, "f16"), ("Wa", 128, "f16"),
                                       ("Wb", 128, "f16"), ("Wd", 128, "f16"), ("We", 128, "f16")])
def test_quantize_workloads(w4, name, g, sz):
    """Full-size workload weights; the oracle checks every row of the smaller
    ones and 256 sampled rows (plus first/last) of the largest."""
    t = WL.weight(name)
    got = gpu_quantize(w4, t.data, t.kind, g, sz)
    n = t.shape[0]
    if n * t.shape[1] <= 64 * 1024 * 1024:
        assert_quant_equal(got, O.quantize_pack_int4(t.data, t.kind, g, sz))
    else:
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(3).choice(n, 256, replace=False)]))
        assert_quant_equal(got, O.quantize_pack_int4(t.data[rows], t.kind, g, sz), rows=rows)


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("sz", ["f16", "f32"])
@pytest.mark.parametrize("n,k,g", [(37, 640, 32), (9, 384, 128), (3, 672, 96)])
def test_dequant(w4, out, sz, n, k, g):
    rng = np.random.default_rng(77 + n)
    w = rng.normal(0, 0.05, (n, k)).astype(np.float32)
    P, S, Z = O.quantize_pack_int4(w, "f32", g, sz)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]
    c = Canary((n, k), tdt)
    w4.dequant_int4(to_dev(P, "u8"), to_dev(S, sz), to_dev(Z, sz), g, out_dtype=tdt, out=c.tensor)
    c.check()
    got = to_host(c.tensor)
    want = O.dequant(P, S, Z, g, out)
    assert np.array_equal(bits(got), bits(want))


def test_dequant_workload(w4):
    t = WL.weight("Wa")
    P, S, Z = O.quantize_pack_int4(t.data, t.kind, 128, "f16")
    got = to_host(w4.dequant_int4(to_dev(P, "u8"), to_dev(S, "f16"), to_dev(Z, "f16"), 128,
                                  out_dtype=torch.bfloat16))
    assert np.array_equal(got, O.dequant(P, S, Z, 128, "bf16"))


# shapes cover the three kernel paths: one wide block per token (m < 64,
# k <= 8192), 256 lanes with the row in registers (k <= 8192), and the
# two-pass kernel for longer rows
@pytest.mark.parametrize("m,k", [(1, 8192), (5, 640), (64, 4096), (3, 8), (2, 2056), (70, 8192),
                                 (3, 16400), (65, 8200)])
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_act_quant(w4, m, k, kind):
    rng = np.random.default_rng(m * 31 + k)
    x = rng.normal(0, 1, (m, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 20), replace=False)] *= 20
    if m > 2:
        x[1] = 0.0
        x[2] *= np.float32(1e-12)
    src = WL.bf16_round_bits(x) if kind == "bf16" else x
    x32 = O.as_f32(src, kind)
    cq = Canary((m, k), torch.int8)
    cs = Canary((m,), torch.float32)
    w4.quantize_act_int8(to_dev(src, kind), out=(cq.tensor, cs.tensor))
    cq.check()
    cs.check()
    xq, sa = O.act_quant_int8(x32)
    assert np.array_equal(to_host(cq.tensor), xq)
    assert np.array_equal(bits(to_host(cs.tensor)), bits(sa))


def test_act_quant_ties_and_closed_forms(w4):
    k = 64
    x = np.zeros((3, k), np.float32)
    x[0] = np.arange(-32, 32)
    x[0, 5] = 127.0
    x[1] = (np.arange(k) % 9 - 4 + 0.5) * 0.25
    x[1, 0] = 31.75
    xq, sa = w4.quantize_act_int8(to_dev(x, "f32"))
    oq, osa = O.act_quant_int8(x)
    assert np.array_equal(to_host(xq), oq) and np.array_equal(bits(to_host(sa)), bits(osa))


@pytest.mark.parametrize("m", [1, 512])
def test_act_quant_workload(w4, m):
    x = WL.activation(5, m, 8192)
    xq, sa = w4.quantize_act_int8(to_dev(x.data, x.kind))
    oq, osa = O.act_quant_int8(x.as_f32())
    assert np.array_equal(to_host(xq), oq) and np.array_equal(bits(to_host(sa)), bits(osa))
