"""Helpers of the attention parity tests: tolerance checks and oracle inputs.

Tolerance of one BF16 output g against the oracle's FP64 value r, derived from
the arithmetic the kernels perform: the MFMA operands P (and, backward, dS)
are rounded to BF16 (unit roundoff u = 2^-8) while everything else runs in
FP32 (relative 2^-24); the oracle returns, per output, the noise scale
n = sqrt(sum of squared terms of the sum that forms r).  Independent uniform
relative roundings of the terms give a standard deviation (u / sqrt 3) n, so

    |g - r| <= ulp_bf16(r) + 7 (u / sqrt 3) n + 2^-20,

the first term for the final BF16 rounding of g, the last for FP32 rounding
of results near zero.  Backward, dS = P (dP - Delta) ds/dS (softcap) or
dP dP/ds (sigmoid) is formed from FP32 sums of D products; their rounding
errs by at most D 2^-24 times the sum of the absolute products, which the
oracle propagates into a cancellation scale c per dQ / dK output (it matters
where dP and Delta cancel, e.g. a causal row that sees one key, where the
exact gradient is 0); the bound then gains D 2^-24 c.  The comparators form
the transform's derivative g from a rounded FP32 value (1 - t^2 from tanhf,
sigma (1 - sigma)), off by at most 2^-21 in absolute terms (two ulps of t
doubled, plus the roundings of t^2 and of the difference), which matters
where 1 - t^2 is tiny; with the oracle's sensitivity s = sum |dS / g| |K|
the comparator bound gains 2^-21 s.  The programs' derivative values are
exact (the oracle replays them).
"""
import json
import os

import numpy as np

import synth_inputs as si

U = 2.0 ** -8
HERE = os.path.dirname(os.path.abspath(__file__))


def bf16v(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(a):
    a = np.abs(a)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check(got_bits, ref, noise, label, cancel=None, dsens=None, D=128):
    got = bf16v(got_bits)
    err = np.abs(got - ref)
    tol = ulp_bf16(ref) + 7 * (U / np.sqrt(3)) * noise + 2.0 ** -20
    if cancel is not None:
        tol = tol + D * 2.0 ** -24 * cancel
    if dsens is not None:
        tol = tol + 2.0 ** -21 * dsens
    within1 = np.mean(err <= ulp_bf16(ref))
    ratio = float(np.max(err / tol))
    print(f"[attn] {label}: max err/tol {ratio:.3f}, within 1 ulp {within1:.4%}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert ratio <= 1.0, label
    return ratio


def tanh_prog(orc):
    g = [p for p in json.load(open(os.path.join(HERE, "golden", "programs.json")))["programs"]
         if p["name"] == "tanh_fwd_d4"][0]
    return orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])


def sig_prog(orc):
    return orc.sig_prog_from_golden(json.load(open(os.path.join(HERE, "golden",
                                                                "sigmoid_attn_b3.json"))))


def fwd_for_bwd(orc, kind, q, k, v, causal, cap=50.0, **kw):
    """The backward's O (BF16) and lse (FP32) inputs, from the oracle's
    forward over every row: (o_bits [B, H, S, D], lse_f32 [B, H, S])."""
    B, H, S, D = q.shape
    o, lse, _ = orc.attn_fwd_rows(kind, q, k, v, np.arange(B * H * S), cap=cap, causal=causal, **kw)
    return (si.to_bf16_bits(o).reshape(B, H, S, D),
            lse.astype(np.float32).reshape(B, H, S))
