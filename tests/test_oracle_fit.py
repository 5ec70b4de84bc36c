"""Pins for the oracle's fit and (Li, Lc) selection.

Independent evidence used here:
  * values the paper prints (tests/golden/table2_bounds.txt, Table 2);
  * the figure-2 configuration (Li, Lc) = (5.0, 5.28125) of the D4 sigmoid;
  * scipy.special for every target function;
  * first-order optimality of least squares (the residual at the 2,000
    Chebyshev nodes is orthogonal to every free basis term of Eq. 8) and the
    two endpoint constraints of Eq. 7, checked in numpy on the FP64 fit.
"""
import json
import os

import numpy as np
import pytest
from scipy import special as sp

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bounds():
    out = {}
    for line in open(os.path.join(GOLD, "table2_bounds.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f, d, deg, val, sol = line.split()
        out[(f, d, int(deg))] = (float(val) * 1e-3, float(sol) * 1e-3)
    return out


def _scipy_ref(func, deriv, x):
    s = sp.expit(x)
    if not deriv:
        return {1: s, 2: np.tanh(x), 3: x * s, 4: x * sp.ndtr(x)}[func]
    sn = sp.expit(-x)
    with np.errstate(over="ignore"):
        return {1: s * sn, 2: 1 / np.cosh(x) ** 2,
                3: s * (1 + x * sn), 4: sp.ndtr(x) + x * np.exp(-x * x / 2) / np.sqrt(2 * np.pi)}[func]


@pytest.mark.parametrize("func,deriv", [(1, 0), (2, 0), (3, 0), (4, 0), (1, 1), (2, 1), (3, 1), (4, 1)])
def test_reference_functions_match_scipy(orc, func, deriv):
    """Relative accuracy over the whole range the 16-bit formats reach before
    the function under- or overflows (BF16 reaches sigma(-x) ~ 1e-38)."""
    xs = np.concatenate([np.linspace(-12, 12, 4001), np.linspace(-100, 100, 2001),
                         [0.0, 1e-8, -1e-8, 30.0, -30.0, -87.5]])
    got = np.array([orc.lib().orc_ref(func, deriv, float(x)) for x in xs])
    ref = _scipy_ref(func, deriv, xs)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_sigmoid_bwd_d4_reproduces_table2_exactly(orc):
    """Table 2, sigmoid backward D4: 4.46e-3.  The full search (no bound) lands
    on (Li, Lc) = (4.75, 4.75); its metric rounds to the printed value."""
    p, obj, met = orc.search(orc.SIGMOID, 1, 4)
    assert (p.Li, p.Lc) == (4.75, 4.75)
    assert p.coeff_bits() == [0x3E80, 0xBB79, 0xBD8F, 0x3CB3, 0xBB00]
    assert round(met * 1e3, 2) == round(_bounds()[("sigmoid", "bwd", 4)][0] * 1e3, 2)


def test_sigmoid_fwd_d3_at_configured_clamp(orc):
    """Table 2, sigmoid forward D3: 5.44e-3.  With Lc = 5.28125 the best
    reachable metric is 5.474e-3 (0.6 % above the printed value; equal to the
    Sollya control 5.47 to three figures)."""
    p, obj, met = orc.search(orc.SIGMOID, 0, 3, Lc_fixed=5.28125, bound=5.445e-3)
    assert p.Li == 6.5
    assert p.coeff_bits() == [0, 0x3E90, 0xBD5B, 0x3B5D]
    printed, sollya = _bounds()[("sigmoid", "fwd", 3)]
    assert abs(met - printed) / printed < 0.01
    assert round(met * 1e3, 2) == round(sollya * 1e3, 2)


def test_silu_d3_reuses_sigmoid_polynomial(orc):
    """Table 2, SiLU D3 (x/2 + even): 21.74e-3.  x/2 + |x| p(|x|) with the
    sigmoid D3 polynomial gives 21.81e-3 (0.3 % above)."""
    sig = orc.make_prog(orc.SIGMOID, 0, 3, 6.5, 5.28125)
    silu = orc.make_prog(orc.SILU, 0, 3, 6.5, 5.28125)
    assert silu.coeff_bits() == sig.coeff_bits()
    met = orc.table2_metric(silu)
    printed = _bounds()[("silu", "fwd", 3)][0]
    assert 0 <= (met - printed) / printed < 0.005


def test_fig2_d4_sigmoid_configuration(orc):
    """Figure 2 selects (Li, Lc) = (5.0, 5.28125) for the D4 centered sigmoid."""
    p = orc.make_prog(orc.SIGMOID, 0, 4, 5.0, 5.28125)
    assert p.coeff_bits() == [0, 0x3E8B, 0xBD25, 0xBABD, 0x3A07]
    assert abs(orc.table2_metric(p) - 3.50e-3) < 0.01e-3


def test_tanh_d4_meets_printed_bound(orc):
    p, obj, met = orc.search(orc.TANH, 0, 4, bound=9.615e-3)
    assert met <= _bounds()[("tanh", "fwd", 4)][0]
    # the unrestricted optimum violates it (recorded reading)
    p2, obj2, met2 = orc.search(orc.TANH, 0, 4)
    assert met2 > _bounds()[("tanh", "fwd", 4)][0]
    assert obj <= 2 * obj2


@pytest.mark.parametrize("func,deriv,degree,Li", [(1, 0, 3, 6.5), (2, 0, 4, 2.5), (4, 0, 5, 3.75),
                                                   (1, 1, 4, 4.75), (2, 1, 4, 2.75), (1, 0, 6, 7.0)])
def test_fit_is_endpoint_constrained_least_squares(orc, func, deriv, degree, Li):
    c = orc.fit(func, deriv, degree, Li)
    k = np.arange(1, 2001)
    t = 0.5 * Li * (1 + np.cos((2 * k - 1) * np.pi / 4000))
    if deriv:
        f = _scipy_ref(func, 1, t) - (0.5 if func in (3, 4) else 0.0)
        f0 = _scipy_ref(func, 1, np.array([0.0]))[0] - (0.5 if func in (3, 4) else 0.0)
        fL = _scipy_ref(func, 1, np.array([Li]))[0] - (0.5 if func in (3, 4) else 0.0)
    else:
        half = {1: lambda z: sp.expit(z) - 0.5, 2: np.tanh, 3: lambda z: sp.expit(z) - 0.5,
                4: lambda z: sp.ndtr(z) - 0.5}[func]
        f, f0, fL = half(t), half(np.array([0.0]))[0], half(np.array([Li]))[0]
    P = np.polyval(c[::-1], t)
    assert abs(c[0] - f0) < 1e-15
    assert abs(np.polyval(c[::-1], Li) - fL) < 1e-13
    r = P - f
    u = t / Li
    for j in range(2, degree + 1):
        phi = u ** j - u
        assert abs(r @ phi) <= 1e-9 * np.linalg.norm(r) * np.linalg.norm(phi) + 1e-14


def test_table2_metric_independent(orc):
    """Recompute the Table 2 metric of two programs in numpy with scipy's
    functions over the same point set."""
    for (func, deriv, degree, Li, Lc) in [(1, 1, 4, 4.75, 4.75), (4, 0, 5, 3.75, 2.75)]:
        p = orc.make_prog(func, deriv, degree, Li, Lc)
        cs = np.array([orc.lib().orc_bf16_to_f64(b) for b in p.coeff_bits()])
        xs = np.linspace(-Lc, Lc, 20001)
        f16 = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
        bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
        extra = np.concatenate([f16, bf])
        extra = extra[np.isfinite(extra) & (np.abs(extra) <= Lc)]
        xs = np.concatenate([xs, extra])
        t = np.minimum(np.abs(xs), Lc)
        v = np.polyval(cs[::-1], t)
        if deriv:
            y = v
        else:
            y = 0.5 * xs + np.abs(xs) * v
        err = np.max(np.abs(y - _scipy_ref(func, deriv, xs)))
        assert abs(err - orc.table2_metric(p)) < 1e-12


def test_golden_programs_are_oracle_output(orc):
    """tests/golden/programs.json is regenerated by make_programs.py; it must
    equal what the oracle selects now."""
    gold = json.load(open(os.path.join(GOLD, "programs.json")))["programs"]
    byname = {g["name"]: g for g in gold}
    sel = {
        "sigmoid_fwd_d3": orc.search(orc.SIGMOID, 0, 3, Lc_fixed=5.28125, bound=5.445e-3),
        "tanh_fwd_d4": orc.search(orc.TANH, 0, 4, bound=9.615e-3),
        "gelu_fwd_d5": orc.search(orc.GELU, 0, 5, bound=1.065e-3),
        "sigmoid_bwd_d4": orc.search(orc.SIGMOID, 1, 4, bound=4.465e-3),
        "tanh_bwd_d4": orc.search(orc.TANH, 1, 4),
        "silu_bwd_d3": orc.search(orc.SILU, 1, 3),
        "gelu_bwd_d5": orc.search(orc.GELU, 1, 5),
    }
    for name, (p, obj, met) in sel.items():
        g = byname[name]
        assert (g["Li"], g["Lc"], g["coeff_bits"]) == (p.Li, p.Lc, p.coeff_bits()), name
        assert g["table2_metric"] == met
    s = byname["silu_fwd_d3"]
    assert s["coeff_bits"] == byname["sigmoid_fwd_d3"]["coeff_bits"]


def test_search_replay_orders_agree_on_selection(orc):
    """The deployed two-rounding BF16 order and the paper's single-rounding
    packed-FMA order select the same programs."""
    for args, kw in [((1, 1, 4), {}), ((1, 0, 3), {"Lc_fixed": 5.28125}), ((2, 1, 4), {})]:
        a = orc.search(*args, order=orc.ORDER_BF16_FMA, **kw)[0]
        b = orc.search(*args, order=orc.ORDER_F32FMA_BF16, **kw)[0]
        assert (a.Li, a.Lc, a.coeff_bits()) == (b.Li, b.Lc, b.coeff_bits())


def test_figs_4_5_degree_is_not_monotone(orc):
    """Appendix A (Figs. 4-5): in each of the six D3-D6 sweeps (sigmoid, tanh,
    SiLU; forward and derivative) at least one higher-degree program has a
    larger maximum error than a lower-degree one after BF16 replay.  Error:
    max |replay - f| over every BF16 value in [0, 12] (the replay is odd or
    even in x, so the positive half suffices)."""
    import numpy as np
    bf = (np.arange(0, 0x4141, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    xs = np.arange(0, 0x4141, dtype=np.uint16)[(bf >= 0) & (bf <= 12)]
    xv = (xs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for func in (orc.SIGMOID, orc.TANH, orc.SILU):
        for deriv in (0, 1):
            errs = []
            for degree in (3, 4, 5, 6):
                kw = {"Lc_fixed": 5.28125} if (func != orc.TANH and deriv == 0) else {}
                p, _, _ = orc.search(func, deriv, degree, **kw)
                y = orc.act_fwd(p, xs, orc.ORDER_F32FMA_BF16)
                yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                ref = np.array([orc.lib().orc_ref(func, deriv, float(v)) for v in xv])
                errs.append(float(np.max(np.abs(yv - ref))))
            inversions = [(a, b) for a in range(4) for b in range(a + 1, 4) if errs[b] > errs[a]]
            assert inversions, (func, deriv, errs)
