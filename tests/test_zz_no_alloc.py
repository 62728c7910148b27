"""w4a16_matmul_noalloc (the entry point for callers that cannot allocate)
through the C ABI: the same product as w4a16_matmul_ws with a workspace of
the queried size, bit for bit, on two calls in a row (the second smaller,
so it reads a scratch that still holds the first call's partials), and on a
shape that needs no scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests.gpu_util import bits, to_dev, to_host, y_as_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def _weights(n, k, g, seed):
    w = np.random.default_rng(seed).normal(0, 0.02, (n, k)).astype(np.float32)
    return O.quantize_pack_int4(w, "f32", g, "f16")


def _args(x, p, s, z, g, y):
    m, k = x.shape
    n = p.shape[0]
    return (ctypes.c_void_p(x.data_ptr()), 2, m, k, ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(s.data_ptr()),
            ctypes.c_void_p(z.data_ptr()), 1, n, g, ctypes.c_void_p(y.data_ptr()), 2)


def test_noalloc_matches_workspace_entry(w4):
    lib = w4.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # (m, n, k, g): the first two split K (the first with the largest scratch,
    # 32 MiB; the second smaller), the third is a decode shape (no scratch)
    for m, n, k, g in ((512, 1024, 8192, 128), (200, 300, 2048, 64), (1, 256, 4096, 128)):
        need = lib.w4a16_matmul_workspace_size(m, k, n, g, 2)
        assert (need > 0) == (m > 1), (m, need)
        P, S, Z = _weights(n, k, g, seed=m + n)
        p, s, z = to_dev(P, "u8"), to_dev(S, "f16"), to_dev(Z, "f16")
        x = to_dev(WL.bf16_round_bits(np.random.default_rng(k).normal(0, 1, (m, k)).astype(np.float32)), "bf16")
        y_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        y_ws = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        assert lib.w4a16_matmul_noalloc(*_args(x, p, s, z, g, y_na), stream) == 0, lib.w4_last_error()
        assert lib.w4a16_matmul_ws(*_args(x, p, s, z, g, y_ws), ctypes.c_void_p(ws.data_ptr()), need,
                                   stream) == 0, lib.w4_last_error()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(y_na)), bits(to_host(y_ws))), (m, n, k, g)
        rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(1).choice(m, min(m, 24), replace=False)]))
        ref = O.matmul_w4a16_f64(O.widen_bf16(to_host(x))[rows], P, S, Z, g)
        assert O.max_rel_err(y_as_f64(y_na)[rows], ref) <= 1e-2


def test_noalloc_rejects_before_any_hip_call(w4):
    lib = w4.load()
    A = ctypes.c_void_p(0x10000)
    # y NULL: invalid, reported before the scratch is looked up
    assert lib.w4a16_matmul_noalloc(A, 2, 256, 11008, A, A, A, 1, 4096, 128, None, 2, None) == -1
    assert b"y is NULL" in lib.w4_last_error()
