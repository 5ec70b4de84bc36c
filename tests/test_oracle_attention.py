"""Pins of the oracle's attention (forward rows, backward rows, the sigmoid-
attention program) against things other than itself:

* forward O and log-sum-exp against textbook FP64 attention (softmax of the
  transformed scores, or the unnormalised sigmoid of Eq. 14);
* every gradient against automatic differentiation (torch, FP64) of textbook
  attention: with the exact transforms directly; for the programs, with the
  oracle's elementwise program values wrapped as a custom autograd function
  (checks the attention-level chain rule exactly), and, for the softcap, with
  the real-arithmetic D4 polynomial (checks that the backward program is the
  derivative of the forward one);
* the printed sigmoid-attention program against sigma(s - ln 4096);
* the differentiated tanh program against a central difference of the real
  polynomial.
"""
import copy
import json
import math
import os

import numpy as np
import pytest
import torch

import synth_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))
B3 = json.load(open(os.path.join(HERE, "golden", "sigmoid_attn_b3.json")))


def bf16_bits(a):
    return si.to_bf16_bits(np.asarray(a, dtype=np.float64))


def bf16v(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16v(bits):
    return bits.view(np.float16).astype(np.float64)


@pytest.fixture(scope="module")
def tanh_prog(orc):
    g = [p for p in json.load(open(os.path.join(HERE, "golden", "programs.json")))["programs"]
         if p["name"] == "tanh_fwd_d4"][0]
    return orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])


@pytest.fixture(scope="module")
def sig_prog(orc):
    return orc.sig_prog_from_golden(B3)


def inputs(B, H, Hkv, S, D, sd_q=1.0, seed=0):
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((B, H, S, D)) * sd_q)
    k = bf16_bits(rng.standard_normal((B, Hkv, S, D)))
    v = bf16_bits(rng.standard_normal((B, Hkv, S, D)))
    do = bf16_bits(rng.standard_normal((B, H, S, D)))
    return q, k, v, do


def textbook(q, k, v, causal, transform, softmax):
    """FP64 torch attention; q [B, H, S, D], k, v [B, Hkv, S, D]."""
    G = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(G, 1)
    vv = v.repeat_interleave(G, 1)
    z = transform(q @ kk.transpose(-1, -2))
    S = q.shape[2]
    vis = torch.ones(S, S, dtype=torch.bool).tril() if causal else torch.ones(S, S, dtype=torch.bool)
    if softmax:
        z = z.masked_fill(~vis, -math.inf)
        lse = torch.logsumexp(z, -1)
        P = torch.softmax(z, -1)
    else:
        lse = None
        P = z.masked_fill(~vis, 0.0)
    return P @ vv, lse


def table_fn(values, grads):
    """Custom autograd function: y = values(S), dy/dS = grads(S) (numpy callables)."""
    class F(torch.autograd.Function):
        @staticmethod
        def forward(ctx, s):
            ctx.save_for_backward(s)
            return torch.from_numpy(values(s.detach().numpy()))

        @staticmethod
        def backward(ctx, g):
            (s,) = ctx.saved_tensors
            return g * torch.from_numpy(grads(s.detach().numpy()))
    return F.apply


def run_both(orc, kind, q, k, v, do, causal, transform, softmax, **kw):
    """Oracle forward + backward over all rows, and the autograd reference."""
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    qt, kt, vt = (torch.from_numpy(bf16v(a)).requires_grad_(True) for a in (q, k, v))
    o_ref, lse_ref = textbook(qt, kt, vt, causal, transform, softmax)
    (o_ref * torch.from_numpy(bf16v(do))).sum().backward()
    rows = np.arange(B * H * S)
    kw.setdefault("replay", False)
    o, lse, noise = orc.attn_fwd_rows(kind, q, k, v, rows, causal=causal, **kw)
    o_exact = o_ref.detach().numpy()
    lse_exact = None if lse_ref is None else lse_ref.detach().numpy()
    dq, dk, dv, sq, sk, sv = orc.attn_bwd_rows(kind, q, k, v, o_exact, do, lse_exact, rows,
                                               np.arange(B * Hkv * S), causal=causal, **kw)
    ref = dict(o=o_exact.reshape(-1, D), lse=None if lse_exact is None else lse_exact.ravel(),
               dq=qt.grad.numpy().reshape(-1, D), dk=kt.grad.numpy().reshape(-1, D),
               dv=vt.grad.numpy().reshape(-1, D))
    got = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, spread=(noise, sq, sk, sv))
    return got, ref


def close(a, b, rtol):
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= rtol, f"max error {err:.3e} of max |ref| (allowed {rtol:.1e})"


CASES = [(1, 4, 2, 37, 16, True), (2, 2, 2, 21, 8, False), (1, 3, 1, 16, 16, True)]


@pytest.mark.parametrize("B,H,Hkv,S,D,causal", CASES)
def test_softcap_exact_fwd_bwd_vs_autograd(orc, tanh_prog, B, H, Hkv, S, D, causal):
    cap = 2.0
    q, k, v, do = inputs(B, H, Hkv, S, D, sd_q=2.0, seed=S)
    got, ref = run_both(orc, orc.ATTN_SOFTCAP_EXACT, q, k, v, do, causal,
                        lambda s: cap * torch.tanh(s / (cap * math.sqrt(D))), True, cap=cap)
    for name in ("o", "lse", "dq", "dk", "dv"):
        close(got[name], ref[name], 1e-12)
    # the real-arithmetic model has nothing to round, so no spread
    assert all(np.all(n == 0) for n in got["spread"])


@pytest.mark.parametrize("B,H,Hkv,S,D,causal", CASES)
def test_sigmoid_exact_fwd_bwd_vs_autograd(orc, B, H, Hkv, S, D, causal):
    q, k, v, do = inputs(B, H, Hkv, S, D, sd_q=2.0, seed=S + 1)
    got, ref = run_both(orc, orc.ATTN_SIGMOID_EXACT, q, k, v, do, causal,
                        lambda s: torch.sigmoid(s / math.sqrt(D) - math.log(S)), False)
    for name in ("o", "dq", "dk", "dv"):
        close(got[name], ref[name], 1e-12)
    assert np.all(np.isnan(got["lse"]))


def program_tables(orc, tanh_prog, fmt):
    """The tanh program and its derivative program over every 16-bit input of
    the format (values), and the map from an FP32 scaled score to the input's
    bits."""
    allx = np.arange(65536, dtype=np.uint16)
    vals = f16v if fmt == "f16" else bf16v
    t_tab = vals(orc.act_fwd(tanh_prog, allx, orc.TANH_ORDERS[fmt]))
    d_tab = vals(orc.dtanh_prog(tanh_prog, allx, fmt))

    def xbits(xs):
        xs = np.asarray(xs, dtype=np.float64).astype(np.float32)
        if fmt == "f16":
            return xs.astype(np.float16).view(np.uint16)
        return bf16_bits(xs.astype(np.float64))
    return t_tab, d_tab, xbits


def softcap_tables(orc, tanh_prog, cap, D, fmt="f16"):
    """The oracle's elementwise programs as functions of the raw score."""
    scale = np.float32(1.0 / (cap * np.sqrt(D)))
    t_tab, d_tab, xbits = program_tables(orc, tanh_prog, fmt)

    def xb(s):
        return xbits((s.astype(np.float32) * scale).astype(np.float32))
    return (lambda s: cap * t_tab[xb(s)],
            lambda s: cap * np.float64(scale) * d_tab[xb(s)])


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("B,H,Hkv,S,D,causal", CASES)
def test_softcap_poly_chain_rule_exact(orc, tanh_prog, B, H, Hkv, S, D, causal, fmt):
    """With the program values as the transform, the oracle's poly attention
    (real-arithmetic model) equals autograd of textbook attention to
    rounding, for either program format."""
    cap = 1.0
    q, k, v, do = inputs(B, H, Hkv, S, D, sd_q=0.7, seed=S + 2)
    val, der = softcap_tables(orc, tanh_prog, cap, D, fmt)
    got, ref = run_both(orc, orc.ATTN_SOFTCAP_POLY, q, k, v, do, causal, table_fn(val, der),
                        True, cap=cap, tanh_prog=tanh_prog, tanh_fmt=fmt)
    for name in ("o", "lse", "dq", "dk", "dv"):
        close(got[name], ref[name], 1e-12)


def test_softcap_poly_backward_is_derivative_of_forward(orc, tanh_prog):
    """Autograd of the real-arithmetic D4 polynomial (BF16 coefficients, no
    rounding anywhere) against the oracle's forward and differentiated
    backward in either format: they differ only by the program's rounding
    (~1e-3 in FP16, a few 1e-3 in BF16), while a wrong derivative coefficient
    moves the gradients by ~1e-1."""
    B, H, Hkv, S, D, cap = 1, 2, 1, 48, 16, 1.0
    q, k, v, do = inputs(B, H, Hkv, S, D, sd_q=0.45, seed=5)
    c = [bf16v(np.array([b], np.uint16))[0] for b in tanh_prog.coeff_bits()]
    x_all = bf16v(q).reshape(B, H, S, D) @ np.swapaxes(bf16v(k), -1, -2) / (cap * math.sqrt(D))
    assert np.abs(x_all).max() < 0.95 * tanh_prog.Lc     # the clamp never binds

    def real_tanh(s):
        u = s / (cap * math.sqrt(D))
        a = u.abs()
        p = sum(cj * a ** j for j, cj in enumerate(c))
        return cap * torch.sign(u) * p
    for fmt in ("bf16", "f16"):
        got, ref = run_both(orc, orc.ATTN_SOFTCAP_POLY, q, k, v, do, True, real_tanh, True,
                            cap=cap, tanh_prog=tanh_prog, tanh_fmt=fmt)
        for name in ("o", "dq", "dk", "dv"):
            close(got[name], ref[name], 1e-2)


def sigmoid_tables(orc, sp, D):
    scale = np.float32(1.0 / np.sqrt(D))
    allx = np.arange(65536, dtype=np.uint16)
    p, g = orc.sig_prog_eval(sp, allx)
    p_tab, g_tab = bf16v(p), bf16v(g)

    def xbits(s):
        return bf16_bits((s.astype(np.float32) * scale).astype(np.float32).astype(np.float64))
    return (lambda s: p_tab[xbits(s)], lambda s: np.float64(scale) * g_tab[xbits(s)])


@pytest.mark.parametrize("B,H,Hkv,S,D,causal", CASES)
def test_sigmoid_poly_chain_rule_exact(orc, sig_prog, B, H, Hkv, S, D, causal):
    sp = copy.deepcopy(sig_prog)
    sp.n = S          # the same coefficients, admitted at this length
    q, k, v, do = inputs(B, H, Hkv, S, D, sd_q=2.0, seed=S + 3)
    val, der = sigmoid_tables(orc, sp, D)
    got, ref = run_both(orc, orc.ATTN_SIGMOID_POLY, q, k, v, do, causal, table_fn(val, der),
                        False, sig=sp)
    for name in ("o", "dq", "dk", "dv"):
        close(got[name], ref[name], 1e-12)


def test_sigmoid_poly_length_guard(orc, sig_prog):
    q, k, v, do = inputs(1, 1, 1, 64, 8)
    with pytest.raises(ValueError):
        orc.attn_fwd_rows(orc.ATTN_SIGMOID_POLY, q, k, v, [0], sig=sig_prog)


@pytest.mark.parametrize("order", [2, 3])
def test_b3_program_against_closed_form(orc, sig_prog, order):
    """The printed program tracks sigma(s - ln 4096) (Eq. 14 at n = 4096) where
    attention scores live, and its factored derivative tracks sigma(1 - sigma);
    where the true value is below ~3e-5 the floor at zero is within that."""
    assert sig_prog.n == 4096
    allx = np.arange(65536, dtype=np.uint16)
    xv = bf16v(allx)
    keep = np.isfinite(xv) & (np.abs(xv) <= 8)
    xb, xv = allx[keep], xv[keep]
    p, g = orc.sig_prog_eval(sig_prog, xb, order)
    pv, gv = bf16v(p), bf16v(g)
    ref = 1.0 / (1.0 + np.exp(-(xv - math.log(4096))))
    dref = ref * (1.0 - ref)
    mid = (xv >= -2) & (xv <= 4)
    low = xv < -2
    assert np.max(np.abs(pv[mid] - ref[mid]) / ref[mid]) < 0.10
    assert np.max(np.abs(gv[mid] - dref[mid]) / dref[mid]) < 0.12
    assert np.max(np.abs(pv[low] - ref[low])) < 3e-5
    assert np.max(np.abs(gv[low] - dref[low])) < 4e-5
    assert np.all(pv >= 0)
    # at s = 0 the value is c_0 = 2^-12, within 0.03 % of 1 / (1 + 4096)
    p0, _ = orc.sig_prog_eval(sig_prog, [0], order)
    assert abs(bf16v(p0)[0] * 4097 - 1) < 3e-4
    # the two regions meet at the threshold 1.25 to within 2 %
    r = [bf16v(orc.sig_prog_eval(sig_prog, bf16_bits([t]), order)[0])[0]
         for t in (1.2421875, 1.25)]
    assert abs(r[1] - r[0]) / r[1] < 0.02


@pytest.mark.parametrize("order", [2, 3])
def test_b3_program_range(orc, sig_prog, order):
    """Over every finite BF16 input the program's value lies in [0, 0.06):
    the attention kernels clamp its last FMA to [0, 1] before rounding in
    place of the floor at zero after it, which is the same value only when
    the program never reaches 1."""
    allx = np.arange(65536, dtype=np.uint16)
    allx = allx[np.isfinite(bf16v(allx))]
    p, _ = orc.sig_prog_eval(sig_prog, allx, order)
    pv = bf16v(p)
    assert np.all(pv >= 0) and np.max(pv) < 0.06


@pytest.mark.parametrize("fmt,tol", [("f16", 3e-3), ("bf16", 1.2e-2)])
def test_dtanh_program_is_derivative_of_tanh_program(orc, tanh_prog, fmt, tol):
    """q(x) = p'(|x|) for |x| <= Lc: against a central difference of the real
    polynomial (orc_prog_real), to the format's Horner accuracy; beyond the
    clamp the forward program is constant and its derivative is exactly 0."""
    allx = np.arange(0, 0x7C00 if fmt == "f16" else 0x7F80, dtype=np.uint16)
    xv = f16v(allx) if fmt == "f16" else bf16v(allx)
    keep = xv <= tanh_prog.Lc
    xb, xv = allx[keep], xv[keep]
    qv = orc.dtanh_prog(tanh_prog, xb, fmt)
    q = f16v(qv) if fmt == "f16" else bf16v(qv)
    L = orc.lib()
    h = 1e-6
    Lc = tanh_prog.Lc

    def fdiff(x):   # one-sided at 0 and at the clamp (the real program is flat beyond)
        lo, hi = (x, x + h) if x <= h else ((x - h, x) if x >= Lc - h else (x - h, x + h))
        return (L.orc_prog_real(tanh_prog, hi) - L.orc_prog_real(tanh_prog, lo)) / (hi - lo)
    fd = np.array([fdiff(x) for x in xv])
    assert np.max(np.abs(q - fd)) < tol
    # beyond the clamp, either sign: 0
    big = allx[~keep]
    for sign in (0, 0x8000):
        assert not np.any(orc.dtanh_prog(tanh_prog, big | sign, fmt))
    # the derivative's coefficients are the forward's (j + 1) c_{j+1} in the
    # format: q(0) = c_1 exactly
    assert q[0] == bf16v(np.array([tanh_prog.c[1]], np.uint16))[0]
