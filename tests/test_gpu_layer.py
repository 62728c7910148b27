"""The PyTorch layer (QuantizedLinear, replace_linears) against the oracle:
its quantizers bit-exact, its forward within the method's tolerances."""
import numpy as np
import pytest
import torch

import oracle.w4_oracle as O
import workloads as WL
from tests.gpu_util import bits, to_dev, to_host, y_as_f64

pytestmark = pytest.mark.gpu

ORACLE_Q = {
    "asym": lambda w, g: O.quantize_pack_int4(w, "bf16", g, "f16"),
    "sym": lambda w, g: O.quantize_pack_int4_sym(w, "bf16", g, "f16"),
    "percentile": lambda w, g: O.quantize_pack_int4_sym_percentile(w, "bf16", g, "f16", 99.9),
    "mse": lambda w, g: O.quantize_pack_int4_sym_mse(w, "bf16", g, "f16", 1000),
}


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dequant_gemm_quantize_amd as m
    m.load()
    return m


def _weight(n, k, seed):
    w = np.random.default_rng(seed).normal(0, 0.02, (n, k)).astype(np.float32)
    return WL.bf16_round_bits(w)


@pytest.mark.parametrize("mode", sorted(ORACLE_Q))
@pytest.mark.parametrize("lead", [(1,), (2, 3), (40,)])
def test_layer_forward(w4, mode, lead):
    n, k, g = 200, 512, 128
    wb = _weight(n, k, 61)
    layer = w4.QuantizedLinear.from_weight(to_dev(wb, "bf16"), group_size=g, mode=mode)
    P, S, Z = ORACLE_Q[mode](wb, g)
    assert np.array_equal(to_host(layer.packed), P)
    assert np.array_equal(bits(to_host(layer.scales)), bits(S))
    assert np.array_equal(bits(to_host(layer.zeros)), bits(Z))
    m = int(np.prod(lead))
    x = WL.bf16_round_bits(np.random.default_rng(m).normal(0, 1, (m, k)).astype(np.float32))
    y = layer(to_dev(x, "bf16").reshape(*lead, k))
    assert tuple(y.shape) == (*lead, n) and y.dtype == torch.bfloat16
    ref = O.matmul_w4a16_f64(O.widen_bf16(x), P, S, Z, g)
    assert O.max_rel_err(y_as_f64(y.reshape(m, n)), ref) <= 1e-2


def test_layer_fp32_and_int8(w4):
    n, k, g = 96, 256, 32
    w = np.random.default_rng(62).normal(0, 0.02, (n, k)).astype(np.float32)
    layer = w4.QuantizedLinear.from_weight(to_dev(w, "f32"), group_size=g, scale_dtype=torch.float32)
    P, S, Z = O.quantize_pack_int4(w, "f32", g, "f32")
    x = np.random.default_rng(63).normal(0, 1, (5, k)).astype(np.float32)
    y = layer(to_dev(x, "f32"))
    assert y.dtype == torch.float32
    assert O.max_rel_err(y_as_f64(y), O.matmul_w4a16_f64(x, P, S, Z, g)) <= 3e-3
    # INT8 activations, bf16 output
    l8 = w4.QuantizedLinear.from_weight(to_dev(w, "f32"), group_size=g, scale_dtype=torch.float32, act_int8=True)
    xb = WL.bf16_round_bits(x)
    y8 = l8(to_dev(xb, "bf16"))
    xq, sa = O.act_quant_int8(O.widen_bf16(xb))
    assert O.max_rel_err(y_as_f64(y8), O.matmul_w4a8_f64(xq, sa, P, S, Z, g)) <= 1e-2
    # the dense weight, bit-exact
    assert np.array_equal(bits(to_host(layer.dequantize(torch.float32))), bits(O.dequant(P, S, Z, g, "f32")))


def test_replace_linears(w4):
    """A small bias-free MLP: every eligible Linear is replaced; the model's
    output equals the chain of oracle products (bf16 between layers)."""
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(256, 384, bias=False), torch.nn.Linear(384, 128, bias=False),
                                torch.nn.Linear(128, 64, bias=True), torch.nn.Linear(128, 96, bias=False))
    model = model.to("cuda", torch.bfloat16)
    dense = [l.weight.detach().clone() for l in model]
    w4.replace_linears(model, group_size=128, mode="sym")
    kinds = [type(l).__name__ for l in model]
    assert kinds == ["QuantizedLinear", "QuantizedLinear", "Linear", "QuantizedLinear"]
    x = WL.bf16_round_bits(np.random.default_rng(64).normal(0, 1, (3, 256)).astype(np.float32))
    h = to_dev(x, "bf16")
    for i in (0, 1):
        wb = to_host(dense[i])
        P, S, Z = O.quantize_pack_int4_sym(wb, "bf16", 128, "f16")
        assert np.array_equal(to_host(model[i].packed), P)
        ref = O.matmul_w4a16_f64(O.widen_bf16(to_host(h)), P, S, Z, 128)
        h = model[i](h)
        assert O.max_rel_err(y_as_f64(h), ref) <= 1e-2


@pytest.mark.parametrize("mode", ["gptq", "gptq_sym"])
def test_layer_gptq_leaves_weight_unchanged(w4, mode):
    """The GPTQ sweep uses its weight argument as working storage; a float32
    contiguous weight (the usual nn.Linear case, possibly a tied parameter)
    must come out of from_weight / replace_linears bit for bit unchanged."""
    n, k, g = 64, 256, 64
    rng = np.random.default_rng(65)
    w = rng.normal(0, 0.05, (n, k)).astype(np.float32)
    x = to_dev(rng.normal(0, 1, (300, k)).astype(np.float32), "f32")
    wt = to_dev(w, "f32")
    w4.QuantizedLinear.from_weight(wt, group_size=g, mode=mode, param=x)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(wt).view(np.uint32), w.view(np.uint32))
    lin = torch.nn.Linear(k, n, bias=False).cuda()
    with torch.no_grad():
        lin.weight.copy_(wt)
    model = torch.nn.Sequential(lin)
    w4.replace_linears(model, group_size=g, mode=mode, param=x)
    torch.cuda.synchronize()
    assert type(model[0]).__name__ == "QuantizedLinear"
    assert np.array_equal(to_host(lin.weight.detach()).view(np.uint32), w.view(np.uint32))
