"""Launch robustness: the entry points captured in a HIP graph and replayed,
and launched on a side stream, give the same bits as eager launches on the
current stream (every kernel here is deterministic: fixed reduction orders,
no atomics)."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_util import bits, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def _inputs():
    rng = np.random.default_rng(90)
    w = to_dev(WL.bf16_round_bits(rng.normal(0, 0.02, (1100, 4096)).astype(np.float32)), "bf16")
    xs = {m: to_dev(WL.bf16_round_bits(rng.normal(0, 1, (m, 4096)).astype(np.float32)), "bf16")
          for m in (1, 3, 16, 300)}
    # GPTQ: weight [300, 512] and 700 calibration rows
    xs["gptq"] = (to_dev(rng.normal(0, 0.05, (300, 512)).astype(np.float32), "f32"),
                  to_dev(rng.normal(0, 1, (700, 512)).astype(np.float32), "f32"))
    return w, xs


def _run(w4, w, xs, outs):
    """Every entry point once, writing into the preallocated outputs."""
    p, s, z = outs["q"]
    w4.quantize_pack_int4(w, 128, torch.float16, out=(p, s, z))
    w4.quantize_pack_int4_sym(w, 128, torch.float16, out=outs["qs"])
    for m, x in xs.items():
        if m == "gptq":
            wg, xg = x
            w4.gptq_hessian(xg, out=outs["gh"])
            outs["ghw"].copy_(outs["gh"])
            w4.gptq_inverse_cholesky(outs["ghw"], out=outs["gu"], overwrite_h=True, check=False)
            outs["gwork"].copy_(wg)
            w4.gptq_quantize_pack_int4(outs["gwork"], outs["gu"], 128, False, torch.float16, overwrite_w=True,
                                       out=outs["gq"])
            continue
        w4.w4a16_matmul(x, p, s, z, 128, out=outs[("y", m)])
        xq, xsc = outs[("a", m)]
        w4.quantize_act_int8(x, out=(xq, xsc))
        w4.w4a8_matmul(xq, xsc, p, s, z, 128, out=outs[("y8", m)])
    w4.dequant_int4(p, s, z, 128, out=outs["d"])


def _alloc(w, xs):
    n, k = w.shape
    dev = w.device
    outs = {"q": (torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                  torch.empty((n, k // 128), dtype=torch.float16, device=dev),
                  torch.empty((n, k // 128), dtype=torch.float16, device=dev)),
            "d": torch.empty((n, k), dtype=torch.bfloat16, device=dev)}
    outs["qs"] = tuple(torch.empty_like(t) for t in outs["q"])
    outs["gh"] = torch.empty((512, 512), dtype=torch.float64, device=dev)
    outs["ghw"] = torch.empty_like(outs["gh"])
    outs["gu"] = torch.empty_like(outs["gh"])
    outs["gwork"] = torch.empty((300, 512), dtype=torch.float32, device=dev)
    outs["gq"] = (torch.empty((300, 256), dtype=torch.uint8, device=dev),
                  torch.empty((300, 4), dtype=torch.float16, device=dev),
                  torch.empty((300, 4), dtype=torch.float16, device=dev))
    for m in xs:
        if m == "gptq":
            continue
        outs[("y", m)] = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        outs[("y8", m)] = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        outs[("a", m)] = (torch.empty((m, k), dtype=torch.int8, device=dev),
                          torch.empty((m,), dtype=torch.float32, device=dev))
    return outs


def _snapshot(outs):
    snap = {}
    for key, v in outs.items():
        ts = v if isinstance(v, tuple) else (v,)
        snap[key] = [bits(to_host(t)).copy() for t in ts]
    return snap


def _clobber(outs):
    for v in outs.values():
        for t in (v if isinstance(v, tuple) else (v,)):
            t.view(torch.uint8).fill_(0xA5)


def test_graph_replays_match_eager(w4):
    w, xs = _inputs()
    outs = _alloc(w, xs)
    _run(w4, w, xs, outs)
    torch.cuda.synchronize()
    eager = _snapshot(outs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _run(w4, w, xs, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        _clobber(outs)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs)
        for key in eager:
            for a, b in zip(got[key], eager[key]):
                assert np.array_equal(a, b), (rep, key)


def test_side_stream_matches_default(w4):
    w, xs = _inputs()
    outs = _alloc(w, xs)
    _run(w4, w, xs, outs)
    torch.cuda.synchronize()
    eager = _snapshot(outs)
    _clobber(outs)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _run(w4, w, xs, outs)
    side.synchronize()
    got = _snapshot(outs)
    for key in eager:
        for a, b in zip(got[key], eager[key]):
            assert np.array_equal(a, b), key
