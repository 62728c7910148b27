"""The GPTQ oracle against its pins (tests/gptq_pins.py), the pins against
planted mistakes, and the oracle's replay checker against its own output and
a planted wrong decision.  CPU only."""
import numpy as np
import pytest

import oracle.gptq_oracle as G
import oracle.w4_oracle as O
from tests import gptq_pins as P

_orig = {n: getattr(G, n) for n in ("gptq_hessian", "gptq_inverse_cholesky", "gptq_quantize", "group_params")}


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


def _u_patched(fn):
    def quantize(w, u, *a, **k):
        return _orig["gptq_quantize"](w, fn(np.asarray(u, np.float64)), *a, **k)
    return quantize


def _params_from_original():
    state = {}

    def quantize(w, u, g, sz, symmetric, **k):
        state["w"] = np.asarray(w, np.float32)
        state["col"] = 0
        state["g"] = g
        return _orig["gptq_quantize"](w, u, g, sz, symmetric, **k)

    def group_params(vals32, symmetric, sz):
        c = state["col"]
        state["col"] = c + state["g"]
        return _orig["group_params"](state["w"][:, c:c + state["g"]], symmetric, sz)
    return {"gptq_quantize": quantize, "group_params": group_params}


def _no_damp(x):
    x64 = np.asarray(x, np.float32).astype(np.float64)
    return x64.T @ x64 / x64.shape[0]


def _no_mean(x):
    x64 = np.asarray(x, np.float32).astype(np.float64)
    h = x64.T @ x64
    return h + 1e-4 * np.mean(np.diag(h)) * np.eye(h.shape[0])


def _offdiag_sign(u):
    return np.diag(np.diag(u)) - np.triu(u, 1)


MUTATIONS = {
    "error_not_divided_by_pivot": {"gptq_quantize": _u_patched(lambda u: u - np.diag(np.diag(u)) + np.eye(len(u)))},
    "update_sign_flipped": {"gptq_quantize": _u_patched(_offdiag_sign)},
    "transposed_factor": {"gptq_quantize": _u_patched(lambda u: u.T.copy())},
    "params_from_original_weights": _params_from_original(),
    "hessian_without_damping": {"gptq_hessian": _no_damp},
    "hessian_not_averaged": {"gptq_hessian": _no_mean},
    "lower_factor_returned": {"gptq_inverse_cholesky":
                              lambda h: np.linalg.cholesky(np.linalg.inv(np.asarray(h, np.float64)))},
    "page_listing_factor": {"gptq_inverse_cholesky":
                            lambda h: np.linalg.inv(np.linalg.cholesky(np.linalg.inv(np.asarray(h, np.float64))))},
    "factor_of_h_not_inverse": {"gptq_inverse_cholesky":
                                lambda h: np.linalg.cholesky(np.asarray(h, np.float64)).T},
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name].items():
        monkeypatch.setattr(G, attr, fn)
    failed = []
    for check in P.ALL_CHECKS:
        try:
            check()
        except (AssertionError, np.linalg.LinAlgError):
            failed.append(check.__name__)
    assert failed, f"mutation {name} survived every pin"


def test_replay_accepts_own_output_and_rejects_a_wrong_code():
    rng = np.random.default_rng(21)
    w = rng.normal(0, 0.05, (12, 96)).astype(np.float32)
    h = G.gptq_hessian(rng.normal(0, 1, (40, 96)).astype(np.float32))
    u = G.gptq_inverse_cholesky(h)
    for symmetric in (False, True):
        packed, s, z = G.gptq_quantize_pack_int4(w, "f32", u, 32, "f16", symmetric)
        _, _, _, stats, _ = G.gptq_quantize(w, u, 32, "f16", symmetric, guide=(packed, s, z))
        assert stats == {"codes_accepted": 0, "zeros_accepted": 0, "scales_differing": 0}
        codes = O.unpack_nibbles(packed)
        _, _, _, _, tr = G.gptq_quantize(w, u, 32, "f16", symmetric, trace=True)
        # the code whose decision variable is farthest from a rounding boundary
        t = tr[:, 40] / s[:, 1].astype(np.float64) + (z[:, 1].astype(np.float64) if not symmetric else 8)
        r = int(np.argmax(np.abs(t - np.floor(t) - 0.5)))
        bad = codes.copy()
        bad[r, 40] = bad[r, 40] + 1 if bad[r, 40] < 15 else bad[r, 40] - 1
        with pytest.raises(AssertionError):
            G.gptq_quantize(w, u, 32, "f16", symmetric, guide=(O.pack_nibbles(bad), s, z))
        s_bad = s.copy()
        s_bad[3, 2] = np.float16(float(s[3, 2]) * 1.01)
        with pytest.raises(AssertionError):
            G.gptq_quantize(w, u, 32, "f16", symmetric, guide=(packed, s_bad, z))
