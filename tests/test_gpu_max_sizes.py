"""The longest rows the library takes: K = 2^23 columns (65536 groups of 128
per row), three weight rows, on every path such rows reach: the quantizer, the
W4A16 MFMA GEMV (slice loop) and the split-K GEMM (256 splits of 512 K steps,
reduced in order), the per-token INT8 quantizer, and the W4A8 int8 MFMA GEMV
and split-K GEMM.  Codes, scales, zero-points and INT8 activations are
compared bit for bit with the oracle; products on sampled tokens against the
oracle's float64 result ("Building a From-Scratch Group-Wise INT4
Quantization Layer for LLaMA Weights", Step 2; "Hands-on Build Guide:
Group-wise INT4 Weight-only Quantization with Per-channel Scales", Step 5).
"""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests.gpu_util import TORCH_SZ, bits, to_dev, to_host, y_as_f64

pytestmark = pytest.mark.gpu

K = 1 << 23
G = 128
N = 3
TOL = 1e-2  # bf16 outputs


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def bf16_rows(rng, m, sigma):
    """[m, K] bf16 bit patterns of N(0, sigma) draws, converted row by row."""
    out = np.empty((m, K), np.uint16)
    for r in range(m):
        out[r] = WL.bf16_round_bits(rng.standard_normal(K, dtype=np.float32) * np.float32(sigma))
    return out


@pytest.fixture(scope="module")
def weights(w4):
    wb = bf16_rows(np.random.default_rng(2023), N, 0.02)
    P, S, Z = O.quantize_pack_int4(wb, "bf16", G, "f16")
    p, s, z = w4.quantize_pack_int4(to_dev(wb, "bf16"), G, TORCH_SZ["f16"])
    return (P, S, Z), (p, s, z)


def test_quantize_max_k(weights):
    (P, S, Z), (p, s, z) = weights
    assert np.array_equal(to_host(p), P)
    assert np.array_equal(bits(to_host(s)), bits(S))
    assert np.array_equal(bits(to_host(z)), bits(Z))


@pytest.mark.parametrize("m", [1, 3, 65])
def test_w4a16_max_k(w4, weights, m):
    (P, S, Z), dw = weights
    if m == 65:
        assert w4.w4a16_matmul_workspace_size(m, K, N, G) > 0   # the split-K GEMM
    xb = bf16_rows(np.random.default_rng(100 + m), m, 1.0)
    y = w4.w4a16_matmul(to_dev(xb, "bf16"), *dw, G)
    rows = sorted({0, m // 2, m - 1})
    ref = O.matmul_w4a16_f64(O.widen_bf16(xb[rows]), P, S, Z, G)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL


@pytest.mark.parametrize("m", [1, 17])
def test_w4a8_max_k(w4, weights, m):
    (P, S, Z), dw = weights
    if m == 17:
        assert w4.w4a8_matmul_workspace_size(m, K, N, G) > 0    # the split-K GEMM
    xb = bf16_rows(np.random.default_rng(500 + m), m, 1.0)
    xq, xs = w4.quantize_act_int8(to_dev(xb, "bf16"))
    rows = sorted({0, m // 2, m - 1})
    oq, os_ = O.act_quant_int8(O.widen_bf16(xb[rows]))
    assert np.array_equal(to_host(xq)[rows], oq) and np.array_equal(bits(to_host(xs)[rows]), bits(os_))
    y = w4.w4a8_matmul(xq, xs, *dw, G)
    ref = O.matmul_w4a8_f64(oq, os_, P, S, Z, G)
    assert O.max_rel_err(y_as_f64(y)[rows], ref) <= TOL
