"""Pins of the oracle's software-exp2 cores (Appendix B.1) against the values
the pages print (tests/golden/exp2_table8.json): the fitted parameters of
PWL2 and D2 under both objectives, every Table 8 error, the FP16 PWL2
core's error after rounding, FA4's D3 p(1); and the endpoint invariants
p(0) = 1, p(1) = 2 of D1, PWL2 and D2 in target precision.  Then the
attention rows with a core: invariant to an integer shift of the scores and
within the core's error bound of exact softmax attention."""
import json
import math
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "exp2_table8.json")))


def sig4(x):
    return float(f"{x:.3e}")


@pytest.mark.parametrize("name,core,minimax", [("PWL2_minimax", 2, True), ("PWL2_lsq", 2, False),
                                               ("D2_minimax", 3, True), ("D2_lsq", 3, False)])
def test_fitted_parameters_and_errors(orc, name, core, minimax):
    a = orc.exp2_fit(core, minimax)
    assert abs(a - G["params"][name]) < 6e-11, (name, a)
    mx, rms = orc.exp2_errors(core, a)
    assert sig4(mx) == G["table8"][name]["max_rel"], (name, mx)
    assert sig4(rms) == G["table8"][name]["rms_rel"], (name, rms)


def test_d1_and_d3_errors(orc):
    for name, core in (("D1", 1), ("D3", 4)):
        mx, rms = orc.exp2_errors(core)
        assert sig4(mx) == G["table8"][name]["max_rel"]
        assert sig4(rms) == G["table8"][name]["rms_rel"]
    assert round(orc.lib().orc_exp2_core(4, 0.0, 1.0), 5) == G["table8"]["D3"]["p1"]
    # D1 in closed form: the maximum of (1 + f) / 2^f sits at f = 1/ln 2 - 1
    f = 1 / math.log(2) - 1
    assert abs((1 + f) / 2 ** f - 1 - orc.exp2_errors(1)[0]) < 1e-11


def test_pwl2_fp16_core_error(orc):
    f = np.arange(1_000_001) / 1e6
    p = orc.exp2_core_target(2, f.astype(np.float32)).astype(np.float64)
    assert sig4(np.max(np.abs(p / 2.0 ** f - 1))) == G["pwl2_fp16"]["max_rel"]
    # the FP16 coefficients are the minimax fit's a and 2 (1 - a), each rounded
    # to FP16 (so p(1) = 2 holds only after the FP16 rounding of the FMAs)
    a = orc.exp2_fit(2, True)
    assert float(np.float16(a)) == G["pwl2_fp16"]["a"]
    assert float(np.float16(2 * (1 - a))) == G["pwl2_fp16"]["two_one_minus_a"]


def test_endpoint_invariants_after_rounding(orc):
    for core in (1, 2, 3):
        p = orc.exp2_core_target(core, np.array([0.0, 1.0], np.float32))
        assert p[0] == 1.0 and p[1] == 2.0, core
    p = orc.exp2_core_target(4, np.array([0.0, 1.0], np.float32))
    assert p[0] == 1.0 and p[1] != 2.0
    # monotone over [0, 1] in target precision
    f = np.linspace(0, 1, 20001, dtype=np.float32)
    for core in (1, 2, 3, 4):
        assert np.all(np.diff(orc.exp2_core_target(core, f)) >= 0), core


def _inputs(seed, S=96, D=32, sd=1.0):
    import synth_inputs as si
    rng = np.random.default_rng(seed)
    return tuple(si.to_bf16_bits(rng.standard_normal((1, 2, S, D)) * sd) for _ in range(3))


@pytest.fixture(scope="module")
def tp(orc):
    g = [p for p in json.load(open(os.path.join(HERE, "golden", "programs.json")))["programs"]
         if p["name"] == "tanh_fwd_d4"][0]
    return orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])


@pytest.mark.parametrize("core", [1, 2, 3, 4])
def test_attention_with_core_within_bound_of_exact_exp(orc, tp, core):
    """Weights w (1 + e), |e| <= E (the core's error in target precision, plus
    the FP32 rounding of z), normalise to P (1 + e) / (1 + mean): so
    |O_core - O| <= 2 E / (1 - E) sum_j P_j |V_j|."""
    q, k, v = _inputs(3 + core, sd=2.0)
    rows = np.arange(2 * 96)
    f = np.arange(1_000_001) / 1e6
    E = np.max(np.abs(orc.exp2_core_target(core, f.astype(np.float32)) / 2.0 ** f - 1)) + 1e-5
    o0, l0, _ = orc.attn_fwd_rows(orc.ATTN_SOFTCAP_POLY, q, k, v, rows, cap=50.0, tanh_prog=tp)
    o1, l1, _ = orc.attn_fwd_rows(orc.ATTN_SOFTCAP_POLY, q, k, v, rows, cap=50.0, tanh_prog=tp,
                                  exp2_core=core)
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[0]
    o1_, l1_ = o1.reshape(2, 96, -1), l1.reshape(2, 96)
    bound = 2 * E / (1 - E) * np.abs(vf).max() + 1e-12
    assert np.max(np.abs(o1 - o0)) <= bound
    assert np.max(np.abs(l1 - l0)) <= 2 * E
    assert np.max(np.abs(o1 - o0)) > 0           # the core is really used


def test_attention_core_shift_invariance(orc, tp):
    """p(0) = 1, p(1) = 2 make 2^(z + k) = 2^k 2^z exact for integers k, so the
    normalised weights only see the fractional parts of the scores: doubling
    cap keeps them in a different place, while scaling Q by a power of two
    changes everything -- check instead that the weights of a row do not
    depend on which key holds the maximum (a permutation of the keys gives the
    permuted output)."""
    q, k, v = _inputs(11, S=64)
    perm = np.random.default_rng(12).permutation(64)
    rows = np.arange(64)
    a, _, _ = orc.attn_fwd_rows(orc.ATTN_SOFTCAP_POLY, q, k, v, rows, causal=False,
                                tanh_prog=tp, exp2_core=2)
    b, _, _ = orc.attn_fwd_rows(orc.ATTN_SOFTCAP_POLY, q, k[:, :, perm], v[:, :, perm], rows,
                                causal=False, tanh_prog=tp, exp2_core=2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
