"""Pins of the oracle's replay model of attention (orc_attn.replay = 1): the
method's FP32 score path and the BF16 rounding of P and dS before the MFMA
products (Fast Polynomial Transcendentals for LLMs, Eq. 1, section 3.4 and
section 5.2.2), against an independent vectorized FP64 torch attention that
performs the same rounding steps with torch's own FP32 / BF16 conversions:

* forward O and log-sum-exp, backward dQ, dK, dV, for the softcap with the
  BF16 and the FP16 tanh program, the softcap with exact tanh, both sigmoid
  transforms, the software exp2 cores, the fixed and the running reference,
  causal and not, grouped query heads;
* the replay model differs from the real-arithmetic model (pinned against
  autograd in test_oracle_attention.py) by BF16-level amounts only;
* a planted mistake (P not rounded to BF16) is visible at the comparison's
  resolution.

The elementwise programs enter as tables over every 16-bit input (they are
pinned by the program tests); everything else is written here again.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))
B3 = json.load(open(os.path.join(HERE, "golden", "sigmoid_attn_b3.json")))
LOG2E32 = float(np.float32(math.log2(math.e)))


def bf16v(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def r32(x):
    """Round to FP32 (x is float64)."""
    return x.to(torch.float32).to(torch.float64)


def rbf(x):
    """Round an FP32 value to BF16 (nearest even)."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def to_fmt_bits(xs, fmt):
    """Bits of the FP32 values xs rounded to the program's format."""
    a = xs.to(torch.float32)
    if fmt == "f16":
        return a.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    return a.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.fixture(scope="module")
def tanh_prog(orc):
    g = [p for p in json.load(open(os.path.join(HERE, "golden", "programs.json")))["programs"]
         if p["name"] == "tanh_fwd_d4"][0]
    return orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])


def inputs(B, H, Hkv, S, D, sd=1.0, seed=0):
    rng = np.random.default_rng(seed)
    q = si.to_bf16_bits(rng.standard_normal((B, H, S, D)) * sd)
    k = si.to_bf16_bits(rng.standard_normal((B, Hkv, S, D)) * sd)
    v = si.to_bf16_bits(rng.standard_normal((B, Hkv, S, D)))
    do = si.to_bf16_bits(rng.standard_normal((B, H, S, D)))
    return q, k, v, do


class Transform:
    """Elementwise pieces of one score transform, as tables or closed forms."""

    def __init__(self, orc, kind, cap, D, S, tanh_prog=None, fmt="bf16", core=0):
        self.kind, self.cap, self.D, self.S, self.fmt, self.core = kind, cap, D, S, fmt, core
        allx = np.arange(65536, dtype=np.uint16)
        if kind == "softcap_poly":
            vals = f16v if fmt == "f16" else bf16v
            self.t_tab = torch.from_numpy(vals(orc.act_fwd(tanh_prog, allx, orc.TANH_ORDERS[fmt])))
            self.d_tab = torch.from_numpy(vals(orc.dtanh_prog(tanh_prog, allx, fmt)))
        if kind == "sigmoid_poly":
            sp = orc.sig_prog_from_golden(B3)
            sp.n = S
            p, g = orc.sig_prog_eval(sp, allx)
            self.p_tab, self.g_tab = torch.from_numpy(bf16v(p)), torch.from_numpy(bf16v(g))
        if core:
            # the cores' FP32 / FP16 values at every FP32 f are needed only at
            # the f that occur; they are evaluated on demand
            self.orc = orc
        self.scale = float(np.float32(1.0 / (cap * math.sqrt(D)))) if "softcap" in kind else \
            float(np.float32(1.0 / math.sqrt(D)))
        self.c2 = float(np.float32(cap * math.log2(math.e)))
        self.mref = math.ceil(float(np.float32(np.float32(self.c2) - np.float32(40.0))))
        self.logn32 = float(np.float32(math.log(S)))
        self.rsd32 = float(np.float32(1.0 / math.sqrt(D)))

    def softcap_t(self, S32, ch):
        """(t, q') from FP32 raw scores."""
        xs = r32(S32 * self.scale)
        if self.kind == "softcap_poly":
            idx = torch.from_numpy(to_fmt_bits(xs, self.fmt).astype(np.int64))
            return self.t_tab[idx], self.d_tab[idx]
        t = ch.fn(r32(torch.tanh(xs)), 4)
        return t, r32(1.0 - t * t)          # fma(-t, t, 1): one rounding

    def sigmoid(self, S32, ch):
        """(P, g): P in FP32 (or the BF16 program value), g the derivative
        value the backward multiplies dP by."""
        if self.kind == "sigmoid_poly":
            xs = r32(S32 * self.scale)
            idx = torch.from_numpy(to_fmt_bits(xs, "bf16").astype(np.int64))
            return self.p_tab[idx], self.g_tab[idx]
        u = r32(S32 * self.scale - self.logn32)      # fma: one rounding
        p = ch.fn(r32(torch.sigmoid(u)), 4)
        return p, r32(p * r32(1.0 - p))

    def exp2(self, z, ref):
        """FP32 2^z relative to 2^ref by the exponential or the core."""
        if self.core == 0:
            return r32(torch.exp2(z - ref))
        zc = torch.clamp(z, min=-16384.0)
        n = torch.floor(zc)
        f = (zc - n).numpy().astype(np.float32)
        core = torch.from_numpy(self.orc.exp2_core_target(self.core, f.ravel()).astype(np.float64))
        return r32(core.reshape(z.shape) * torch.exp2(n - ref))


class Exact:
    """The replay model's primary choices: RN32 of exact dot products,
    correctly rounded exponentials and comparator functions."""

    def dot(self, exact, abs_sum, steps):
        return r32(exact)

    def fn(self, value, ulps):
        return value


class Alternative(Exact):
    """An admissible alternative for every decision: dot products moved to the
    edge of their admissible range (steps u sum |a b|, random sign) and
    rounded inward, exponentials and comparator functions moved by a random
    admissible number of ulps."""

    def __init__(self, seed):
        self.g = torch.Generator().manual_seed(seed)

    def dot(self, exact, abs_sum, steps):
        sign = torch.randint(0, 2, exact.shape, generator=self.g).to(torch.float64) * 2 - 1
        target = exact + sign * steps * 2.0 ** -24 * abs_sum
        f = target.to(torch.float32).to(torch.float64)
        # round toward the exact value so the choice stays within the range
        over = (f - exact).abs() > steps * 2.0 ** -24 * abs_sum
        f32 = target.to(torch.float32)
        toward = torch.nextafter(f32, exact.to(torch.float32))
        return torch.where(over, toward.to(torch.float64), f)

    def fn(self, value, ulps):
        k = torch.randint(-ulps, ulps + 1, value.shape, generator=self.g)
        x = value.to(torch.float32)
        for step in range(1, ulps + 1):
            x = torch.where(k >= step, torch.nextafter(x, torch.tensor(float("inf"))), x)
            x = torch.where(k <= -step, torch.nextafter(x, torch.tensor(float("-inf"))), x)
        return x.to(torch.float64)


def replay_torch(tr, q, k, v, do, causal, ch=None):
    """The replay model, vectorized: (O, lse, dQ, dK, dV) as float64 arrays.
    ch: the choice of each open rounding decision (Exact by default)."""
    ch = ch or Exact()
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    Q, K, V, dO = (torch.from_numpy(bf16v(a)) for a in (q, k, v, do))
    Kg, Vg = K.repeat_interleave(G, 1), V.repeat_interleave(G, 1)
    vis = torch.ones(S, S, dtype=torch.bool)
    if causal:
        vis = vis.tril()
    S32 = ch.dot(Q @ Kg.transpose(-1, -2), Q.abs() @ Kg.abs().transpose(-1, -2), 8)
    hw = tr.core == 0
    if "softcap" in tr.kind:
        t, dq_ = tr.softcap_t(S32, ch)
        if tr.core == 0 and tr.c2 <= 80:
            ref = torch.full(S32.shape[:-1] + (1,), float(tr.mref), dtype=torch.float64)
            P = ch.fn(r32(torch.exp2(r32(t * tr.c2 - tr.mref))), 1)
        else:
            z = r32(t * tr.c2)
            ref = torch.floor(torch.clamp(z, min=-16384.0)).masked_fill(~vis, -math.inf)
            ref = ref.amax(-1, keepdim=True)
            P = tr.exp2(z, ref)
            if hw:
                P = ch.fn(P, 1)
        P = P.masked_fill(~vis, 0.0)
        l = P.sum(-1, keepdim=True)
        O = (rbf(P) @ Vg) / l
        lse = ((ref + torch.log2(l)) * math.log(2.0)).squeeze(-1)
    else:
        P, g = tr.sigmoid(S32, ch)
        P = P.masked_fill(~vis, 0.0)
        O = rbf(P) @ Vg
        lse = None
    # backward from O rounded to BF16 and the FP32 lse
    Ob = rbf(O)
    dP = ch.dot(dO @ Vg.transpose(-1, -2), dO.abs() @ Vg.abs().transpose(-1, -2), 8)
    if "softcap" in tr.kind:
        lse32 = r32(lse).unsqueeze(-1)
        nl = -r32(lse32 * LOG2E32)
        z = r32(t * tr.c2 + nl)
        Pb_ = tr.exp2(z, 0.0) if tr.core else ch.fn(r32(torch.exp2(z)), 1)
        delta = ch.dot((dO * Ob).sum(-1, keepdim=True), (dO * Ob).abs().sum(-1, keepdim=True), 128)
        dS = r32(dq_ * r32(Pb_ * r32(dP - delta)))
    else:
        Pb_ = P
        dS = r32(dP * g)
    Pb = rbf(Pb_).masked_fill(~vis, 0.0)
    dSb = rbf(dS).masked_fill(~vis, 0.0)
    dQ = (dSb @ Kg) * tr.rsd32
    dK = (dSb.transpose(-1, -2) @ Q).reshape(B, Hkv, G, S, D).sum(2) * tr.rsd32
    dV = (Pb.transpose(-1, -2) @ dO).reshape(B, Hkv, G, S, D).sum(2)
    return (O.numpy(), None if lse is None else lse.numpy(), Ob.numpy(),
            None if lse is None else r32(lse).numpy(), dQ.numpy(), dK.numpy(), dV.numpy())


ORC_KIND = {"softcap_poly": 1, "softcap_exact": 2, "sigmoid_poly": 3, "sigmoid_exact": 4}


def replay_oracle(orc, tr, tanh_prog, q, k, v, do, o_b, lse32, causal, spreads=False):
    B, H, S, D = q.shape
    kind = ORC_KIND[tr.kind]
    sp = None
    if tr.kind == "sigmoid_poly":
        sp = orc.sig_prog_from_golden(B3)
        sp.n = S
    kw = dict(cap=tr.cap, causal=causal, tanh_prog=tanh_prog, sig=sp, tanh_fmt=tr.fmt,
              exp2_core=tr.core, replay=True)
    rows = np.arange(B * H * S)
    o, lse, so = orc.attn_fwd_rows(kind, q, k, v, rows, **kw)
    g = orc.attn_bwd_rows(kind, q, k, v, o_b, do, lse32, rows, np.arange(B * k.shape[1] * S), **kw)
    if spreads:
        return (o, lse, g[0], g[1], g[2]), (so, g[3], g[4], g[5])
    return o, lse, g[0], g[1], g[2]


def close(a, b, rtol, what):
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= rtol, f"{what}: max error {err:.3e} of max |ref| (allowed {rtol:.1e})"


CASES = [(1, 4, 2, 37, 16, True), (2, 2, 2, 21, 8, False), (1, 3, 1, 16, 16, True)]
TRANSFORMS = [("softcap_poly", "bf16", 0), ("softcap_poly", "f16", 0), ("softcap_exact", "bf16", 0),
              ("sigmoid_poly", "bf16", 0), ("sigmoid_exact", "bf16", 0),
              ("softcap_poly", "bf16", 1), ("softcap_poly", "bf16", 2), ("softcap_poly", "bf16", 3),
              ("softcap_poly", "bf16", 4)]


@pytest.mark.parametrize("kind,fmt,core", TRANSFORMS)
@pytest.mark.parametrize("B,H,Hkv,S,D,causal", CASES)
@pytest.mark.parametrize("cap", [50.0, 100.0, 2.0])
def test_replay_matches_vectorized_rounding(orc, tanh_prog, kind, fmt, core, B, H, Hkv, S, D,
                                            causal, cap):
    if "sigmoid" in kind and cap != 50.0:
        pytest.skip("no cap")
    # scores large enough that P spans many binades and dP - Delta is exercised
    sd = 2.0 if "softcap" in kind else 1.5
    q, k, v, do = inputs(B, H, Hkv, S, D, sd=sd, seed=S + int(cap) + core)
    tr = Transform(orc, kind, cap, D, S, tanh_prog, fmt, core)
    O, lse, Ob, lse32, dQ, dK, dV = replay_torch(tr, q, k, v, do, causal)
    o_b = Ob.reshape(B, H, S, D)
    lse_in = None if lse32 is None else lse32.reshape(B, H, S)
    o, ls, dq, dk, dv = replay_oracle(orc, tr, tanh_prog, q, k, v, do, o_b, lse_in, causal)
    close(o, O.reshape(-1, D), 1e-12, "O")
    if lse is not None:
        close(ls, lse.ravel(), 1e-12, "lse")
    close(dq, dQ.reshape(-1, D), 1e-12, "dQ")
    close(dk, dK.reshape(-1, D), 1e-12, "dK")
    close(dv, dV.reshape(-1, D), 1e-12, "dV")


@pytest.mark.parametrize("kind,fmt", [("softcap_poly", "bf16"), ("softcap_poly", "f16"),
                                      ("softcap_exact", "bf16"), ("sigmoid_exact", "bf16")])
def test_replay_is_real_arithmetic_up_to_bf16_rounding(orc, tanh_prog, kind, fmt):
    """The two models differ by the BF16 rounding of P / dS (relative 2^-9
    per term) and FP32 steps: O by at most 2^-8 of the largest |O|, the
    gradients by at most 2^-6 of their largest magnitude."""
    B, H, Hkv, S, D = 1, 2, 1, 40, 16
    q, k, v, do = inputs(B, H, Hkv, S, D, sd=1.5, seed=7)
    kk = ORC_KIND[kind]
    kw = dict(cap=50.0, causal=True, tanh_prog=tanh_prog, tanh_fmt=fmt)
    rows = np.arange(B * H * S)
    o1, l1, _ = orc.attn_fwd_rows(kk, q, k, v, rows, replay=True, **kw)
    o0, l0, _ = orc.attn_fwd_rows(kk, q, k, v, rows, replay=False, **kw)
    close(o1, o0, 2.0 ** -8, "O")
    if "softcap" in kind:
        close(l1, l0, 1e-6, "lse")
    ob = si.to_bf16_bits(o0).reshape(B, H, S, D)
    ov = bf16v(ob)
    lse = l0.reshape(B, H, S)
    krows = np.arange(B * Hkv * S)
    g1 = orc.attn_bwd_rows(kk, q, k, v, ov, do, lse, rows, krows, replay=True, **kw)
    g0 = orc.attn_bwd_rows(kk, q, k, v, ov, do, lse, rows, krows, replay=False, **kw)
    for i, name in enumerate(("dQ", "dK", "dV")):
        close(g1[i], g0[i], 2.0 ** -6, name)


def test_planted_mistake_unrounded_p_is_visible(orc, tanh_prog):
    """The vectorized model with P left unrounded before P V differs from the
    oracle's replay far above the comparison's 1e-12: the pin would catch an
    oracle that skipped the BF16 rounding."""
    B, H, Hkv, S, D = 1, 2, 2, 37, 16
    q, k, v, do = inputs(B, H, Hkv, S, D, sd=2.0, seed=3)
    tr = Transform(orc, "softcap_poly", 50.0, D, S, tanh_prog, "bf16", 0)
    Q, K, V = (torch.from_numpy(bf16v(a)) for a in (q, k, v))
    S32 = r32(Q @ K.transpose(-1, -2))
    t, _ = tr.softcap_t(S32, Exact())
    P = r32(torch.exp2(r32(t * tr.c2 - tr.mref))).masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), 0.0)
    O_unrounded = ((P @ V) / P.sum(-1, keepdim=True)).numpy().reshape(-1, D)
    o, _, _ = orc.attn_fwd_rows(1, q, k, v, np.arange(B * H * S), cap=50.0, causal=True,
                                tanh_prog=tanh_prog, tanh_fmt="bf16", replay=True)
    err = np.abs(o - O_unrounded).max() / np.abs(o).max()
    assert err > 1e-5, err


def ulp_bf16(a):
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -126)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -16)


@pytest.mark.parametrize("kind,fmt,core", TRANSFORMS)
@pytest.mark.parametrize("cap", [50.0, 100.0])
def test_admissible_alternatives_lie_within_the_spread(orc, tanh_prog, kind, fmt, core, cap):
    """Every output of the replay model run with other admissible choices for
    its open rounding decisions (dot products at the edge of the stated
    accumulation radius, exponentials and comparator functions off by their
    admissible ulps) lies within the oracle's spread of the primary result,
    and the choices do flip decisions (the spread is not vacuous: some
    outputs move).  The spread stays small where no decision is close: its
    median is below a tenth of the output's BF16 ulp."""
    if "sigmoid" in kind and cap != 50.0:
        pytest.skip("no cap")
    B, H, Hkv, S, D, causal = 1, 4, 2, 48, 16, False
    sd = 2.0 if "softcap" in kind else 1.5
    q, k, v, do = inputs(B, H, Hkv, S, D, sd=sd, seed=11 + core + int(cap))
    tr = Transform(orc, kind, cap, D, S, tanh_prog, fmt, core)
    O, lse, Ob, lse32, dQ, dK, dV = replay_torch(tr, q, k, v, do, causal)
    o_b = Ob.reshape(B, H, S, D)
    lse_in = None if lse32 is None else lse32.reshape(B, H, S)
    prim, spr = replay_oracle(orc, tr, tanh_prog, q, k, v, do, o_b, lse_in, causal, spreads=True)
    moved = 0
    for seed in range(4):
        alt = replay_torch(tr, q, k, v, do, causal, Alternative(seed))
        # the backward of the alternative from the same O and lse inputs
        altb = replay_torch_bwd_only(tr, q, k, v, do, causal, o_b, lse_in, Alternative(100 + seed))
        for got, ref, sp, name in ((alt[0], prim[0], spr[0], "O"), (altb[0], prim[2], spr[1], "dQ"),
                                   (altb[1], prim[3], spr[2], "dK"), (altb[2], prim[4], spr[3], "dV")):
            got = got.reshape(ref.shape)
            err = np.abs(got - ref)
            slack = 1e-3 * sp + 1e-12 * np.abs(ref).max()
            bad = err > sp + slack
            assert not bad.any(), f"{name}: {bad.sum()} outputs beyond the spread, worst {np.max(err - sp):.3e}"
            moved += int(np.sum(err > 1e-12 * np.abs(ref).max()))
    assert moved > 0
    for sp, ref in ((spr[0], prim[0]), (spr[1], prim[2])):
        assert np.median(sp / ulp_bf16(ref)) < 0.1


def replay_torch_bwd_only(tr, q, k, v, do, causal, o_b, lse32, ch):
    """Backward of the replay model from given O (BF16 values) and FP32 lse."""
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    Q, K, V, dO = (torch.from_numpy(bf16v(a)) for a in (q, k, v, do))
    Kg, Vg = K.repeat_interleave(G, 1), V.repeat_interleave(G, 1)
    vis = torch.ones(S, S, dtype=torch.bool)
    if causal:
        vis = vis.tril()
    Ob = torch.from_numpy(o_b)
    S32 = ch.dot(Q @ Kg.transpose(-1, -2), Q.abs() @ Kg.abs().transpose(-1, -2), 8)
    dP = ch.dot(dO @ Vg.transpose(-1, -2), dO.abs() @ Vg.abs().transpose(-1, -2), 8)
    if "softcap" in tr.kind:
        t, dq_ = tr.softcap_t(S32, ch)
        lse = torch.from_numpy(lse32.astype(np.float64)).unsqueeze(-1)
        nl = -r32(lse * LOG2E32)
        z = r32(t * tr.c2 + nl)
        Pb_ = tr.exp2(z, 0.0) if tr.core else ch.fn(r32(torch.exp2(z)), 1)
        delta = ch.dot((dO * Ob).sum(-1, keepdim=True), (dO * Ob).abs().sum(-1, keepdim=True), 128)
        dS = r32(dq_ * r32(Pb_ * r32(dP - delta)))
    else:
        Pb_, g = tr.sigmoid(S32, ch)
        dS = r32(dP * g)
    Pb = rbf(Pb_).masked_fill(~vis, 0.0)
    dSb = rbf(dS).masked_fill(~vis, 0.0)
    dQ = (dSb @ Kg) * tr.rsd32
    dK = (dSb.transpose(-1, -2) @ Q).reshape(B, Hkv, G, S, D).sum(2) * tr.rsd32
    dV = (Pb.transpose(-1, -2) @ dO).reshape(B, Hkv, G, S, D).sum(2)
    return dQ.numpy(), dK.numpy(), dV.numpy()
