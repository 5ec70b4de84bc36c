"""Pins of the oracle's rotary-embedding programs ("Fast Polynomial
Transcendentals for LLMs", Appendix B.2; the readings are listed in
oracle/orc_rope.c) against things other than the oracle itself:

* the fit: the endpoint values imposed (Eq. 8) hold, and an independent
  least-squares solve (numpy's, on the same constrained bases) gives the same
  free coefficients;
* the turn increment and the Q15 reduction: Python big-integer arithmetic
  and numpy's float16 rounding;
* the packed-FP16 evaluation and the rotation: an exact rational replay with
  a round-to-nearest-even FP16 written here from the format's definition;
* the structure: sine odd and cosine even bit for bit, sin(0) = 0, and the
  rotation by (sin, cos) = (0, 1) is the identity.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest


@pytest.fixture(scope="module")
def rp(orc):
    return orc.rope_prog()


def bf16_frac(b):
    return Fr(float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]))


def f16_frac(b):
    return Fr(float(np.array([int(b)], dtype=np.uint16).view(np.float16)[0]))


def rn16(x: Fr) -> Fr:
    """Round an exact rational to the nearest FP16 value (ties to even);
    +-inf as float('inf') beyond the largest finite value."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    e = max(e, -14)                      # subnormals share the quantum 2^-24
    q = Fr(2) ** (e - 10)
    n = a / q
    k = math.floor(n)
    r = n - k
    if r > Fr(1, 2) or (r == Fr(1, 2) and k % 2 == 1):
        k += 1
    v = k * q
    if v > 65504:
        return sign * Fr(10 ** 30)       # overflow marker (never reached here)
    return sign * v


def test_fit_endpoint_values(orc):
    s, c = orc.rope_fit()
    assert abs(s.sum()) < 1e-13                     # sin(pi) = 0: a1 + a3 + a5 = 0
    assert c[0] == 1.0                              # cos(0) = 1
    assert abs(c.sum() + 1.0) < 1e-13               # cos(pi) = -1


def test_fit_matches_an_independent_least_squares(orc):
    n = 4096
    k = np.arange(1, n + 1)
    u = 0.5 * (1.0 + np.cos((2.0 * k - 1.0) * np.pi / (2.0 * n)))
    A = np.stack([u ** 3 - u, u ** 5 - u], axis=1)
    xs = np.linalg.lstsq(A, np.sin(np.pi * u), rcond=None)[0]
    u2 = u * u
    A = np.stack([u2 ** 2 - u2, u2 ** 3 - u2], axis=1)
    xc = np.linalg.lstsq(A, np.cos(np.pi * u) - 1.0 + 2.0 * u2, rcond=None)[0]
    s, c = orc.rope_fit()
    np.testing.assert_allclose(s[1:], xs, rtol=1e-10)
    np.testing.assert_allclose(c[2:], xc, rtol=1e-10)


def test_fit_error_is_that_of_a_least_squares_fit(orc):
    """Real-arithmetic error of the FP64 fit well below the truncated Taylor
    series of the same degrees (0.52 for the sine, 0.21 for the cosine at
    u = 1), and the FP64 fit a better fit than its BF16 rounding."""
    s, c = orc.rope_fit()
    u = np.linspace(-1.0, 1.0, 100001)
    w = u * u
    es = np.max(np.abs(u * (s[0] + w * (s[1] + w * s[2])) - np.sin(np.pi * u)))
    ec = np.max(np.abs(c[0] + w * (c[1] + w * (c[2] + w * c[3])) - np.cos(np.pi * u)))
    assert es < 0.52 / 20 and ec < 0.21 / 20
    rp = orc.rope_prog()
    sb = [float(bf16_frac(b)) for b in rp.sin_c]
    cb = [float(bf16_frac(b)) for b in rp.cos_c]
    es_b = np.max(np.abs(u * (sb[0] + w * (sb[1] + w * sb[2])) - np.sin(np.pi * u)))
    ec_b = np.max(np.abs(cb[0] + w * (cb[1] + w * (cb[2] + w * cb[3])) - np.cos(np.pi * u)))
    assert es <= es_b and ec <= ec_b


def test_turn_increments(orc):
    inc = orc.rope_inc(128, 10000.0)
    assert inc[0] == 683565276                      # round(2^32 / (2 pi))
    assert np.all(np.diff(inc.astype(np.int64)) < 0)
    for i in (1, 17, 63):
        w = 10000.0 ** (-2.0 * i / 128)
        assert abs(int(inc[i]) - w * 2 ** 32 / (2 * math.pi)) <= 0.5


def test_q15_coordinate_and_phase_wraparound(orc):
    rng = np.random.default_rng(7)
    inc = orc.rope_inc(128, 10000.0)
    for p in [0, 1, 6, 7, 1000, 65535, 65536, 123456789, 2 ** 31 - 1]:
        for i in rng.integers(0, 64, 4):
            phase = (p * int(inc[i])) % 2 ** 32         # big-integer arithmetic
            v = ((phase >> 16) ^ 0x8000) - 0x8000
            want = np.float16(v / 32768.0).view(np.uint16)
            assert orc.rope_coord(phase)[0] == want
            # the coordinate is the phase's half-turn position (mod 2)
            turns = phase / 2 ** 32
            d = (2 * turns - v / 32768.0) % 2.0
            assert min(d, 2.0 - d) < 2 ** -15 + 1e-12


def test_sincos_replay_matches_exact_rational_replay(orc, rp):
    a1, a3, a5 = (f16_frac(orc.lib().orc_f64_to_f16(float(bf16_frac(b)))) for b in rp.sin_c)
    b0, b2, b4, b6 = (f16_frac(orc.lib().orc_f64_to_f16(float(bf16_frac(b)))) for b in rp.cos_c)
    # the BF16 coefficients are FP16 values
    assert [a1, a3, a5] == [bf16_frac(b) for b in rp.sin_c]
    vs = list(range(-32768, 32768, 37)) + [-32768, -1, 0, 1, 2, 16384, -16384, 32767]
    phases = np.array([(v & 0xFFFF) << 16 for v in vs], dtype=np.uint64)
    sb, cb = orc.rope_sincos(rp, phases)
    for v, sbit, cbit in zip(vs, sb, cb):
        u = rn16(Fr(v, 32768))
        w = rn16(u * u)
        q = rn16(rn16(a5 * w + a3) * w + a1)
        s = rn16(q * u)
        c = rn16(rn16(rn16(b6 * w + b4) * w + b2) * w + b0)
        assert f16_frac(sbit) == s, v
        assert f16_frac(cbit) == c, v


def test_sine_odd_cosine_even_bit_exact(orc, rp):
    v = np.arange(1, 32768)
    sp, cp = orc.rope_sincos(rp, (v.astype(np.uint64) & 0xFFFF) << 16)
    sn, cn = orc.rope_sincos(rp, ((-v).astype(np.int64).astype(np.uint64) & 0xFFFF) << 16)
    assert np.all(sn == (sp ^ 0x8000))
    assert np.all(cn == cp)
    s0, c0 = orc.rope_sincos(rp, [0])
    assert s0[0] == 0x0000 and c0[0] == 0x3C00        # sin = +0, cos = b0 = 1


def test_rotation_replay_and_identity(orc):
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (400, 4)).astype(np.float16).view(np.uint16)
    for x0, x1, s, c in x:
        y0, y1 = orc.rope_rotate(x0, x1, s, c)
        X0, X1, S, Cc = (f16_frac(t) for t in (x0, x1, s, c))
        assert f16_frac(y0) == rn16(X0 * Cc - rn16(X1 * S))
        assert f16_frac(y1) == rn16(X1 * Cc + rn16(X0 * S))
    for x0, x1 in x[:, :2]:
        assert orc.rope_rotate(x0, x1, 0x0000, 0x3C00) == (x0, x1)


def test_rows_against_fp64_rotation(orc, rp):
    """Whole rows at large positions: the replay's outputs are the FP64
    rotation by the true angle within the programs' error (|sin|, |cos|
    off by at most 0.017 over every coordinate) plus the roundings."""
    rng = np.random.default_rng(11)
    D = 64
    inc = orc.rope_inc(D, 10000.0)
    pos = np.array([0, 1, 2, 1000, 70000, 2 ** 20 + 3], dtype=np.int64)
    x = rng.normal(0, 1, (pos.size, D)).astype(np.float16)
    y = orc.rope_rows(rp, inc, x.view(np.uint16), pos).view(np.float16).astype(np.float64)
    xd = x.astype(np.float64)
    for r, p in enumerate(pos):
        for i in range(D // 2):
            ph = (int(p) * int(inc[i])) % 2 ** 32
            v = ((ph >> 16) ^ 0x8000) - 0x8000
            th = math.pi * float(np.float16(v / 32768.0))
            y0 = xd[r, 2 * i] * math.cos(th) - xd[r, 2 * i + 1] * math.sin(th)
            y1 = xd[r, 2 * i] * math.sin(th) + xd[r, 2 * i + 1] * math.cos(th)
            tol = 0.017 * (abs(xd[r, 2 * i]) + abs(xd[r, 2 * i + 1])) + 3e-3 * (abs(y0) + abs(y1) + 0.01)
            assert abs(y[r, 2 * i] - y0) <= tol and abs(y[r, 2 * i + 1] - y1) <= tol
