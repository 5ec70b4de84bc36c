"""Why the deployed GELU D5 program misses Table 2's 1.06e-3: a tested fact,
not prose.

Fast Polynomial Transcendentals for LLMs, Table 2 prints 1.06e-3 for the
constrained GELU D5 fit (maximum absolute error over [-Lc, Lc], BF16
coefficients, real arithmetic; section 4.1).  Section 3.2 fits with the
endpoint-constrained basis of Eq. 8 (P(0) = f(0), P(Li) = f(Li)).  The test
enumerates readings of "GELU D5 = x/2 + even residual" (section 3.3, Eq. 6):

  R1  x/2 + t p(t^), p of degree 5 with p(0) = 0 fit to Phi(t) - 1/2
      (the oracle's reading, SiLU's construction with Phi; evaluated with the
      oracle's own fitter and Table-2 metric, which also takes every FP16 and
      BF16 input in [-Lc, Lc]);
  R2  x/2 + r(t^), r of degree 5 in t fit to the residual t (Phi(t) - 1/2);
  R3  x (1/2 + q(x)), q odd of degree 5 (t^1, t^3, t^5) fit to Phi - 1/2;
  R4  x/2 + r, r a polynomial in x^2 (t^2, t^4, t^6) fit to the residual;
  R5  x/2 + t p(t^), p of degree 5 chosen so that t p fits the residual
      (the residual the metric measures);

each with the Eq. 8 endpoint constraint, over the pages' search grid
(Li in 0.25 .. 12 by 0.25, Lc <= Li + 1) restricted to Lc >= 2: a smaller
clamp makes the tail error beyond Lc grow to ~0.07 at |x| = 3, so no sane
program lies there.  Every reading's best metric stays above the printed
value's rounding interval (1.065e-3); the metric on the 20,001-point grid is
a lower bound of the full metric, so R2-R5 are checked on it alone.  Without
the endpoint constraint the bound is reachable (R1 at about 0.87e-3), so the
printed value was presumably fit differently; the deployed program keeps the
method's constrained fit (parity unpinned for that selection).
"""
import numpy as np
import pytest
from scipy.special import erf

import synth_inputs as si

BOUND = 1.065e-3


def phi_half(t):
    return 0.5 * erf(t / np.sqrt(2.0))


def resid(t):
    return t * phi_half(t)


def bf16(a):
    b = si.to_bf16_bits(np.asarray(a, dtype=np.float64))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cheb(Li, n=2000):
    k = np.arange(1, n + 1)
    return Li / 2 * (1 + np.cos((2 * k - 1) * np.pi / (2 * n)))


def fit(powers, target, times_t, Li, endpoint=True):
    """Least squares of sum c_j t^p_j (times t when times_t) against target on
    2,000 first-kind Chebyshev nodes of [0, Li]; with the endpoint constraint
    the value at Li is matched exactly (the value at 0 is 0 for every basis
    here, as is the target's).  Coefficients rounded to BF16."""
    t = cheb(Li)
    A = np.stack([t ** p for p in powers], 1) * (t[:, None] if times_t else 1.0)
    y = target(t)
    if endpoint:
        aL = np.array([Li ** p for p in powers]) * (Li if times_t else 1.0)
        yL = target(np.array([Li]))[0]
        A2 = A[:, :-1] - np.outer(A[:, -1], aL[:-1] / aL[-1])
        c, *_ = np.linalg.lstsq(A2, y - A[:, -1] * yL / aL[-1], rcond=None)
        c = np.append(c, (yL - aL[:-1] @ c) / aL[-1])
    else:
        c, *_ = np.linalg.lstsq(A, y, rcond=None)
    return bf16(c)


def metric(powers, c, times_t, Lc):
    x = np.linspace(-Lc, Lc, 20001)
    t = np.abs(x)
    r = sum(ci * t ** p for ci, p in zip(c, powers)) * (t if times_t else 1.0)
    return float(np.max(np.abs(x / 2 + r - (x / 2 + resid(t)))))


# name: (powers, fit target, fit basis times t, residual = t * polynomial)
READINGS = {
    "R2": ([1, 2, 3, 4, 5], resid, False, False),
    "R3": ([1, 3, 5], phi_half, False, True),
    "R4": ([2, 4, 6], resid, False, False),
    "R5": ([1, 2, 3, 4, 5], resid, True, True),
}


def grid():
    for Li in np.arange(0.25, 12.0 + 1e-9, 0.25):
        Lcs = np.arange(2.0, min(Li + 1.0, 12.0) + 1e-9, 0.25)
        if Lcs.size:
            yield Li, Lcs


def best(powers, target, times_t, eval_times_t, endpoint=True):
    b = (np.inf, None)
    for Li, Lcs in grid():
        c = fit(powers, target, times_t, Li, endpoint)
        for Lc in Lcs:
            m = metric(powers, c, eval_times_t, Lc)
            if m < b[0]:
                b = (m, (Li, Lc))
    return b


def test_r1_oracle_reading_never_meets_the_printed_bound(orc):
    """The oracle's own fitter and Table-2 metric (all FP16 / BF16 inputs in
    [-Lc, Lc] included) over the grid: best > 1.065e-3."""
    b = (np.inf, None)
    for Li, Lcs in grid():
        for Lc in Lcs:
            m = orc.table2_metric(orc.make_prog(orc.GELU, 0, 5, Li, Lc))
            if m < b[0]:
                b = (m, (Li, Lc))
    print(f"R1 best Table-2 metric {b[0]:.4e} at (Li, Lc) = {b[1]}")
    assert b[0] > BOUND
    # the same construction in numpy gives the same best (cross-check of the
    # numpy fitter the other readings use)
    nb = best([1, 2, 3, 4, 5], phi_half, False, True)
    assert nb[1] == b[1] and abs(nb[0] - b[0]) < 2e-5, (nb, b)


@pytest.mark.parametrize("name", sorted(READINGS))
def test_other_readings_never_meet_the_printed_bound(name):
    powers, target, times_t, eval_times_t = READINGS[name]
    b = best(powers, target, times_t, eval_times_t)
    print(f"{name} best metric {b[0]:.4e} at (Li, Lc) = {b[1]}")
    assert b[0] > BOUND


def test_without_the_endpoint_constraint_the_bound_is_reachable():
    """What the constraint costs: the unconstrained least-squares R1 reaches
    the printed value on the same grid."""
    b = best([1, 2, 3, 4, 5], phi_half, False, True, endpoint=False)
    print(f"unconstrained R1 best metric {b[0]:.4e} at (Li, Lc) = {b[1]}")
    assert b[0] <= BOUND


def test_deployed_gelu_program_is_the_constrained_search_winner(orc):
    """The deployed program is the unrestricted search winner (no candidate
    meets the bound, so the restriction is void) and its metric is recorded
    beside the printed bound."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "programs.json")))
    g = [p for p in gold["programs"] if p["name"] == "gelu_fwd_d5"][0]
    p, _, met = orc.search(orc.GELU, 0, 5, bound=BOUND)
    q, _, met0 = orc.search(orc.GELU, 0, 5)
    assert (p.Li, p.Lc) == (q.Li, q.Lc) == (g["Li"], g["Lc"])
    assert met == met0 == pytest.approx(g["table2_metric"], rel=1e-12)
    assert g["table2_metric"] > g["table2_bound"] == BOUND
