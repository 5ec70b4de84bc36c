"""Pins for the oracle's program replay, fused SwiGLU and attention.

Evidence independent of the oracle's own code:
  * the symmetry identities of the paper (Eqs. 3, 4, 9 and the odd/even forms
    of section 3.3), which hold bit for bit for the replayed residual;
  * a rounding-error bound around the real-arithmetic program (numpy Horner
    on the BF16 coefficients): every replayed FP16/BF16 output lies within it;
  * numpy / torch IEEE arithmetic for the backward product and the SwiGLU
    combination; scipy's functions for the approximation error;
  * a textbook FP64 softcapped attention in numpy for the attention rows.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy import special as sp

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALL = np.arange(65536, dtype=np.uint16)


def _progs(orc):
    out = {}
    for g in json.load(open(os.path.join(GOLD, "programs.json")))["programs"]:
        out[g["name"]] = orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])
    return out


@pytest.fixture(scope="module")
def progs(orc):
    return _progs(orc)


def f16v(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16v(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


FMT = {
    "f16": dict(order=1, val=f16v, nan=0x7C00, quiet=0x0200, u=2.0 ** -11, tiny=2.0 ** -25),
    "bf16": dict(order=3, val=bf16v, nan=0x7F80, quiet=0x0040, u=2.0 ** -8, tiny=2.0 ** -134),
}


def _finite(bits, fmt):
    return (bits & 0x7FFF) < FMT[fmt]["nan"]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identities_bitwise(orc, progs, fmt):
    F = FMT[fmt]
    pos = ALL[(ALL < 0x8000) & _finite(ALL, fmt)]
    neg = pos | 0x8000
    tanh_p = orc.act_fwd(progs["tanh_fwd_d4"], pos, F["order"])
    tanh_n = orc.act_fwd(progs["tanh_fwd_d4"], neg, F["order"])
    assert np.array_equal(tanh_n, tanh_p ^ 0x8000)           # odd: tanh~(-x) = -tanh~(x)
    for name in ("sigmoid_bwd_d4", "tanh_bwd_d4"):              # even derivatives
        assert np.array_equal(orc.act_fwd(progs[name], pos, F["order"]),
                              orc.act_fwd(progs[name], neg, F["order"]))
    # centered sigmoid: y(x) + y(-x) - 1 is only the rounding of the two 1/2 + r
    yp = F["val"](orc.act_fwd(progs["sigmoid_fwd_d3"], pos, F["order"]))
    yn = F["val"](orc.act_fwd(progs["sigmoid_fwd_d3"], neg, F["order"]))
    half_ulp = lambda y: np.where(y >= 0.5, 0.5, 0.25) * F["u"] * 2  # noqa: E731
    assert np.all(np.abs(yp + yn - 1.0) <= half_ulp(yp) / 2 + half_ulp(yn) / 2)
    # centered-odd derivatives (Eq. 9): s'(x) + s'(-x) - 1 is only the rounding
    # of the two 1/2 + r (values in (-0.1, 1.1))
    ulp_of = lambda y: 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -14))) - (10 if fmt == "f16" else 7))  # noqa: E731
    for name in ("silu_bwd_d3", "gelu_bwd_d5"):
        dp = F["val"](orc.act_fwd(progs[name], pos, F["order"]))
        dn = F["val"](orc.act_fwd(progs[name], neg, F["order"]))
        assert np.all(np.abs(dp + dn - 1.0) <= ulp_of(dp) / 2 + ulp_of(dn) / 2), name


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("name", ["sigmoid_fwd_d3", "tanh_fwd_d4", "silu_fwd_d3", "gelu_fwd_d5",
                                  "sigmoid_bwd_d4", "tanh_bwd_d4", "silu_bwd_d3", "gelu_bwd_d5"])
def test_replay_within_rounding_bound_of_real_program(orc, progs, fmt, name):
    """Every finite input: |replay - P(x)| <= gamma_{D+1} sum|c_j| t^j (Horner
    with one rounding per FMA) propagated through the reconstruction, plus the
    final rounding and underflow slack.  P(x) is evaluated here in numpy."""
    F = FMT[fmt]
    p = progs[name]
    xs = ALL[_finite(ALL, fmt)]
    x = F["val"](xs)
    y = F["val"](orc.act_fwd(p, xs, F["order"]))
    c = bf16v(np.array(p.coeff_bits(), dtype=np.uint16))
    t = np.abs(x)
    th = np.minimum(t, p.Lc)
    v = np.polyval(c[::-1], th)
    absv = np.polyval(np.abs(c)[::-1], th)
    D = p.degree
    u = F["u"] if fmt == "f16" else 2.0 ** -8 + 2.0 ** -24   # FP32 then BF16 per stage
    gamma = (D + 1) * u / (1 - (D + 1) * u)
    chain = gamma * absv + (D + 2) * F["tiny"]
    sg = np.where(np.signbit(x), -1.0, 1.0)
    if name.startswith("sigmoid_fwd") or name in ("silu_bwd_d3", "gelu_bwd_d5"):
        P, err = 0.5 + sg * v, chain
    elif name.startswith("tanh_fwd") or name.endswith("bwd_d4"):
        P, err = (sg * v if name.startswith("tanh_fwd") else v), chain
    else:   # SiLU / GELU: x/2 + t v, t unclamped
        P, err = 0.5 * x + t * v, t * chain + np.abs(0.5 * x) * u + 2 * F["tiny"]
    bound = err + np.abs(P) * u + F["tiny"]
    bad = ~(np.abs(y - P) <= bound) & np.isfinite(P)
    assert not bad.any(), (name, fmt, x[bad][:5], y[bad][:5], P[bad][:5])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_clamp_holds_the_chain_at_lc(orc, progs, fmt):
    """t^ = min(|x|, Lc) (Eq. 2): every input with |x| >= Lc gives exactly the
    output at sign(x) Lc for the clamped programs, and for SiLU / GELU the
    chain value v = (y - x/2) / t is that of Lc (checked through the
    derivative-free identity y(x) = x/2 + |x| v(Lc) in real arithmetic within
    one rounding of y)."""
    F = FMT[fmt]
    xs = ALL[_finite(ALL, fmt)]
    x = F["val"](xs)
    for name in ("sigmoid_fwd_d3", "tanh_fwd_d4", "sigmoid_bwd_d4", "tanh_bwd_d4",
                 "silu_bwd_d3", "gelu_bwd_d5"):
        p = progs[name]
        big = np.abs(x) >= p.Lc
        y = orc.act_fwd(p, xs[big], F["order"])
        enc = (lambda v: np.array([v], np.float16).view(np.uint16)[0]) if fmt == "f16" else \
            (lambda v: torch.tensor([v]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0])
        at = orc.act_fwd(p, np.array([enc(p.Lc), enc(-p.Lc)], np.uint16), F["order"])
        want = np.where(np.signbit(x[big]), at[1], at[0])
        assert np.array_equal(y, want), name
        # and just below the clamp the chain is not held
        below = (np.abs(x) < p.Lc) & (np.abs(x) > p.Lc * 0.75)
        assert not np.all(orc.act_fwd(p, xs[below & (x > 0)], F["order"]) == at[0]), name


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_special_values(orc, progs, fmt):
    F = FMT[fmt]
    inf, ninf = F["nan"], F["nan"] | 0x8000
    nans = np.array([F["nan"] | 1, F["nan"] | F["quiet"], 0xFFFF, F["nan"] | 0x8000 | 3],
                    dtype=np.uint16)
    enc = (lambda v: np.array([v], np.float16).view(np.uint16)[0]) if fmt == "f16" else \
        (lambda v: torch.tensor([v]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0])
    for name, p in progs.items():
        y = orc.act_fwd(p, nans, F["order"])
        assert np.array_equal(y, nans | F["quiet"]), name           # NaN -> quiet NaN
    for name in ("sigmoid_fwd_d3", "tanh_fwd_d4", "sigmoid_bwd_d4", "tanh_bwd_d4"):
        p = progs[name]
        lc, nlc = enc(p.Lc), enc(-p.Lc)
        y = orc.act_fwd(p, np.array([inf, ninf, lc, nlc], np.uint16), F["order"])
        assert y[0] == y[2] and y[1] == y[3], name                  # clamp at +-Lc
    for name in ("silu_fwd_d3", "gelu_fwd_d5"):
        y = orc.act_fwd(progs[name], np.array([inf, ninf, 0, 0x8000], np.uint16), F["order"])
        # -0: fma(+0, v, -0 * 1/2) = +0 + -0 = +0 under round-to-nearest
        assert list(y) == [inf, 0x8000, 0, 0], name
    y = orc.act_fwd(progs["tanh_fwd_d4"], np.array([0, 0x8000], np.uint16), F["order"])
    assert list(y) == [0, 0x8000]
    y = orc.act_fwd(progs["sigmoid_fwd_d3"], np.array([0, 0x8000], np.uint16), F["order"])
    assert F["val"](y).tolist() == [0.5, 0.5]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_backward_is_rounded_product(orc, progs, fmt):
    """dx = RN(g * q(x)): the product of two 16-bit values is exact in FP64,
    and numpy / torch round FP64 -> FP16 and FP32 -> BF16 to nearest even."""
    F = FMT[fmt]
    rng = np.random.default_rng(5)
    xs = ALL[_finite(ALL, fmt)]
    g = rng.integers(0, 65536, xs.size).astype(np.uint16)
    g = np.where(_finite(g, fmt), g, np.uint16(0x3C00 if fmt == "f16" else 0x3F80)).astype(np.uint16)
    for name in ("sigmoid_bwd_d4", "tanh_bwd_d4", "silu_bwd_d3", "gelu_bwd_d5"):
        p = progs[name]
        q = F["val"](orc.act_fwd(p, xs, F["order"]))
        dx = orc.act_bwd(p, xs, g, F["order"])
        prod = F["val"](g) * q
        if fmt == "f16":
            ref = prod.astype(np.float16).view(np.uint16)
        else:   # deployed BF16 order: RN_bf16(RN_f32(g q))
            ref = torch.from_numpy(prod).to(torch.float32).to(torch.bfloat16) \
                .view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(dx, ref), name
        if name in ("sigmoid_bwd_d4", "tanh_bwd_d4"):
            assert np.all(q > 0), name              # no inf * 0 can arise


def test_swiglu_matches_ieee_float32(orc, progs):
    rng = np.random.default_rng(6)
    rows, cols = 37, 200
    def bf(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    g = bf(rng.standard_normal((rows, cols)) * 2)
    u = bf(rng.standard_normal((rows, cols)) * 2)
    dh = bf(rng.standard_normal((rows, cols)))
    sig = progs["sigmoid_fwd_d3"]
    h = orc.swiglu_fwd(sig, g, u)
    dg, du = orc.swiglu_bwd(sig, g, u, dh)
    p = bf16v(orc.act_fwd(sig, g.ravel(), 3)).reshape(rows, cols).astype(np.float32)
    gf, uf, dhf = (bf16v(a).astype(np.float32) for a in (g, u, dh))
    gp = gf * p
    tob = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    assert np.array_equal(h, tob(gp * uf))
    ds = (gp.astype(np.float64) * (np.float32(1) - p) + p).astype(np.float32)  # one rounding
    assert np.array_equal(du, tob(dhf * gp))
    assert np.array_equal(dg, tob((dhf * uf) * ds))
    # approximation: h is SiLU(g) u to within the sigmoid program's error
    silu = gf * sp.expit(gf.astype(np.float64))
    eps = 5.5e-3 + 2.0 ** -8
    assert np.all(np.abs(bf16v(h) - silu * uf) <= np.abs(gf * uf) * eps + np.abs(bf16v(h)) * 2 ** -8 + 1e-30)


def test_swiglu_row_range(orc, progs):
    rng = np.random.default_rng(7)
    g = rng.integers(0, 0x4000, (10, 16)).astype(np.uint16)
    u = rng.integers(0, 0x4000, (10, 16)).astype(np.uint16)
    h = orc.swiglu_fwd(progs["sigmoid_fwd_d3"], g, u, 3, 7)
    full = orc.swiglu_fwd(progs["sigmoid_fwd_d3"], g, u)
    assert np.array_equal(h[3:7], full[3:7])
    assert not h[:3].any() and not h[7:].any()


def test_bf16_rounding_orders_agree_on_every_input(orc, progs):
    """The deployed BF16 order (FP32 FMA rounded to FP32, then to BF16) and the
    pages' single-rounding BF16 FMA (section 3.4, fma.rn.bf16x2) give the same
    output for every BF16 input of every program: a Horner step's exact
    result fits FP32 unless the product is far below the addend, where both
    orders round to the addend.  A split multiply / add does differ."""
    g = np.random.default_rng(5).integers(0, 65536, 65536).astype(np.uint16)
    for name, p in progs.items():
        if p.deriv:
            run = lambda order: orc.act_bwd(p, ALL, g, order)  # noqa: E731
        else:
            run = lambda order: orc.act_fwd(p, ALL, order)  # noqa: E731
        deployed = run(orc.ORDER_F32FMA_BF16)
        assert np.array_equal(deployed, run(orc.ORDER_BF16_FMA)), name
        assert (deployed != run(orc.ORDER_BF16_SPLIT)).any(), name
