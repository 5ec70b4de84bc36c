"""Helpers of the attention parity tests: the gate and oracle inputs.

The oracle's replay model performs the method's own rounding steps (FP32
scores, exponent arguments and backward scalars; P and dS rounded to BF16
before the products; Fast Polynomial Transcendentals for LLMs, section 3.4
and section 5.2.2) and returns each output in FP64 with its spread: the
largest change admissible alternatives of the replay's rounding decisions can
cause (the pages leave the accumulation order of an FP32 dot product and the
last bit of an FP32 exponential open).  The gate for one BF16 output g
against the oracle's r:

    |g - r| <= u(r) + spread,    u(r) = max(ulp_bf16(r), 2^-16),

one BF16 ulp of the oracle's value, floored at 2^-16 for |r| < 2^-8 (the
final rounding of g and the FP32 accumulation of the sums), plus the spread,
which is zero unless a rounding decision is close.  Every comparison prints
how many outputs are within 1 ulp and how many needed the spread, and the
latter are capped (ALT_CAP of the outputs): the spread explains individual
decisions, it is not a tolerance for a whole tensor.
"""
import json
import os

import numpy as np

import synth_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))
ALT_CAP = 5e-3   # largest share of outputs that may need the spread (at least 16)


def bf16v(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_floor(a):
    """One BF16 ulp of |a|, floored at 2^-16."""
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -126)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -16)


def check(got_bits, ref, spread, label):
    got = bf16v(got_bits)
    err = np.abs(got - ref)
    u = ulp_floor(ref)
    within1 = err <= u
    needed = int(np.sum(~within1))
    worst = float(np.max(err / u)) if err.size else 0.0
    over = err - u - spread
    print(f"[attn] {label}: {err.size} outputs, within 1 ulp {np.mean(within1):.6%}, "
          f"needed the spread {needed}, max err {worst:.2f} ulp, "
          f"not covered {int(np.sum(over > 0))}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert np.all(over <= 0), f"{label}: {int(np.sum(over > 0))} outputs beyond 1 ulp + spread"
    assert needed <= max(16, ALT_CAP * err.size), f"{label}: {needed} outputs needed the spread"
    return needed


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
