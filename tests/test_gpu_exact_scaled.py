"""Bit-exact group indexing on every kernel of both products.

Each group of W is 2^e * (Q - Z) with its own power-of-two scale 2^e
(e in [-9, -6]) and zero-point Z in 0..15, and holds the codes 0 and 15
("From Scratch: Building a GPTQ INT4 Quantizer in Pure Python", Step 4:
dequantized weight (q - zp) * scale).  Quantizing such a W gives back
exactly (Q, 2^e, Z), and with integer activations every product and every
partial sum is a multiple of 2^-9 below 2^24 * 2^-9, so each kernel's float32
arithmetic is exact whatever its summation order: a bf16 output must equal
the correctly rounded exact product, an fp32 output the exact product.  A
kernel that read a neighbouring group's scale or zero-point, or a wrong
group's codes, changes the result.
"""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests.gpu_util import TORCH_SZ, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def scaled_weights(rng, n, k, g):
    """(W float32, Q, E, Z): W[r, group j] = 2^E[r, j] * (Q - Z[r, j])."""
    ng = k // g
    q = rng.integers(0, 16, (n, k))
    for r in range(n):
        for j in range(ng):
            a, b = rng.choice(g, 2, replace=False)
            q[r, j * g + a], q[r, j * g + b] = 0, 15
    e = rng.integers(-9, -5, (n, ng))
    z = rng.integers(0, 16, (n, ng))
    w = np.ldexp((q.reshape(n, ng, g) - z[..., None]).astype(np.float64), e[..., None]).reshape(n, k)
    return w.astype(np.float32), q, e, z


def exact_product(xi, q, e, z, g):
    """sum_k x[m, k] * 2^e (q - z) as float64 (exact: integers times 2^-9)."""
    n, k = q.shape
    d = (q.reshape(n, k // g, g) - z[..., None]) << (e[..., None] + 9)  # in units of 2^-9
    return (xi.astype(np.int64) @ d.reshape(n, k).T).astype(np.float64) * 2.0 ** -9


def quantize_on_gpu(w4, w, g, sz, q, e, z):
    p, s, zz = w4.quantize_pack_int4(to_dev(w, "f32"), g, TORCH_SZ[sz])
    assert np.array_equal(O.unpack_nibbles(to_host(p)), q.astype(np.uint8))
    assert np.array_equal(to_host(s).astype(np.float64), np.ldexp(1.0, e))
    assert np.array_equal(to_host(zz).astype(np.float64), z.astype(np.float64))
    return p, s, zz


W4A16_CASES = [  # (m, n, k, g, sz, xkind) and the kernel the dispatcher picks
    (1, 300, 4096, 128, "f16", "bf16"),    # dot2
    (1, 129, 11008, 128, "f32", "bf16"),   # dot2, two rows per wave above K = 8192
    (1, 64, 8192, 256, "f16", "bf16"),     # dot2, groups of 256
    (2, 300, 4096, 128, "f16", "bf16"),    # 4x4x4 matrix-core GEMV
    (3, 77, 4096, 128, "f16", "bf16"),     # 4x4x4 matrix-core GEMV, ragged last row group
    (4, 45, 4096, 32, "f32", "bf16"),      # 4x4x4 matrix-core GEMV, groups of 32
    (2, 40, 4096, 512, "f16", "bf16"),     # 4x4x4 matrix-core GEMV, groups of 512
    (3, 70, 2048, 128, "f16", "bf16"),     # decode, looped form
    (4, 200, 2048, 128, "f32", "bf16"),    # decode, looped form
    (4, 100, 1024, 256, "f16", "bf16"),    # decode, looped form, groups of 256
    (5, 300, 1024, 128, "f16", "bf16"),    # MFMA GEMV
    (16, 256, 4096, 128, "f16", "bf16"),   # MFMA GEMV
    (33, 129, 11008, 128, "f16", "bf16"),  # MFMA GEMV, slice loop
    (64, 520, 2048, 128, "f32", "bf16"),   # MFMA GEMV, two launches
    (100, 96, 640, 128, "f16", "bf16"),    # MFMA GEMV, partial slice
    (200, 300, 1024, 128, "f16", "bf16"),  # GEMM
    (129, 130, 640, 64, "f16", "bf16"),    # GEMM, groups of 64
    (300, 256, 768, 32, "f32", "bf16"),    # GEMM, groups of 32
    (1, 64, 640, 32, "f16", "bf16"),       # general kernel (groups below 128)
    (3, 40, 384, 96, "f16", "bf16"),       # general kernel (groups of 96)
    (5, 70, 512, 128, "f16", "f32"),       # general kernel (fp32 activations)
    (40, 50, 256, 32, "f32", "f32"),       # general kernel (fp32 activations)
]


@pytest.mark.parametrize("m,n,k,g,sz,xkind", W4A16_CASES)
@pytest.mark.parametrize("ykind", ["bf16", "f32"])
def test_w4a16_scaled_exact(w4, m, n, k, g, sz, xkind, ykind):
    rng = np.random.default_rng(m * 7919 + n * 31 + k + g)
    w, q, e, z = scaled_weights(rng, n, k, g)
    p, s, zz = quantize_on_gpu(w4, w, g, sz, q, e, z)
    xi = rng.integers(-8, 9, (m, k))
    x = WL.bf16_round_bits(xi.astype(np.float32)) if xkind == "bf16" else xi.astype(np.float32)
    ydt = torch.bfloat16 if ykind == "bf16" else torch.float32
    y = to_host(w4.w4a16_matmul(to_dev(x, xkind), p, s, zz, g, out_dtype=ydt))
    exact = exact_product(xi, q, e, z, g).astype(np.float32)
    want = O.to_bf16(exact) if ykind == "bf16" else exact
    bad = np.argwhere(y != want)
    assert bad.size == 0, (bad[:5], y[tuple(bad[0])], want[tuple(bad[0])])


W4A8_CASES = [  # (m, n, k, g, sz)
    (1, 300, 8192, 128, "f16"),    # dot4
    (4, 129, 4096, 128, "f32"),    # dot4, four tokens
    (2, 64, 2048, 128, "f16"),     # dot4
    (1, 100, 640, 128, "f16"),     # int8 MFMA GEMV (K not a multiple of 2048)
    (8, 300, 1024, 128, "f16"),    # int8 MFMA GEMV
    (16, 129, 4096, 256, "f32"),   # int8 MFMA GEMV, groups of 256
    (64, 256, 4096, 128, "f16"),   # int8 GEMM, 128-token tiles
    (129, 130, 2048, 128, "f32"),  # int8 GEMM, 256-token tiles, ragged
    (300, 130, 1024, 256, "f16"),  # int8 GEMM, groups of 256
    (129, 520, 4096, 128, "f16"),  # int8 GEMM, split K over the workspace (4 splits)
    (300, 130, 2304, 256, "f32"),  # int8 GEMM, split K at step 9: inside a group of 256
    (40, 1000, 8192, 128, "f16"),  # int8 GEMM, 128-token tiles, split K (8 splits)
    (3, 48, 512, 64, "f16"),       # general kernel (groups of 64)
    (40, 64, 256, 32, "f32"),      # general kernel (groups of 32)
]


@pytest.mark.parametrize("m,n,k,g,sz", W4A8_CASES)
@pytest.mark.parametrize("ws", ["auto", None])
def test_w4a8_scaled_exact(w4, m, n, k, g, sz, ws):
    """Activations: integers with |x| <= 8 and one 127 per token, so the
    per-token scale is 1 and xq = x.  ws: with the workspace the library asks
    for (split K where the shape splits) and without one."""
    rng = np.random.default_rng(m * 104729 + n * 17 + k + g)
    w, q, e, z = scaled_weights(rng, n, k, g)
    p, s, zz = quantize_on_gpu(w4, w, g, sz, q, e, z)
    xi = rng.integers(-8, 9, (m, k))
    xi[np.arange(m), rng.integers(0, k, m)] = 127
    xq, xs = w4.quantize_act_int8(to_dev(WL.bf16_round_bits(xi.astype(np.float32)), "bf16"))
    assert (to_host(xs) == 1.0).all() and np.array_equal(to_host(xq), xi.astype(np.int8))
    y = to_host(w4.w4a8_matmul(xq, xs, p, s, zz, g, workspace=ws))
    want = O.to_bf16(exact_product(xi, q, e, z, g).astype(np.float32))
    bad = np.argwhere(y != want)
    assert bad.size == 0, (bad[:5], y[tuple(bad[0])], want[tuple(bad[0])])
