"""Mutation tests of the rotary-embedding parity comparison: a plausible
mistake planted in the oracle (on the CPU, never in a kernel) must change
its output against the GPU's.

Mutants: each of the seven BF16 coefficients moved by one unit in the last
place; the Q15 coordinate rounded to nearest instead of truncated; the
rotation with its product and sum rounded separately instead of one FMA;
the cosine's last stage split the same way; the pairs rotated the other way
(y0 = x0 c + x1 s).  The unmutated replay reproduces the GPU bit for bit.
Inputs: one query head (compared) and one key head of 512 positions x 128,
N(0, 1) FP16 (seeds 9, 10).
"""
import ctypes as C

import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import note, to_bits, to_dev

pytestmark = pytest.mark.gpu
S, D, BASE = 512, 128, 10000.0
NEG0 = 0x8000


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def case(pa):
    q = si.to_f16_bits(si.normal(9, S * D)).reshape(1, S, 1, D)
    k = si.to_f16_bits(si.normal(10, S * D)).reshape(1, S, 1, D)
    note("rope mutations: poly_rope 1 x 512 x 1 (1) x 128")
    qo, _ = pa.poly_rope(to_dev(q, torch.float16), to_dev(k, torch.float16), BASE)
    torch.cuda.synchronize()
    return q.reshape(S, D), to_bits(qo).reshape(S, D)


def replay(orc, rp, x, coord=None, rot=None, cos_last=None):
    """The oracle's rotary embedding composed from its FP16 primitives, with
    one step optionally replaced."""
    fma = orc.lib().orc_fma_f16
    f16 = lambda b: orc.lib().orc_f64_to_f16(float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]))  # noqa: E731
    a1, a3, a5 = (f16(b) for b in rp.sin_c)
    b0, b2, b4, b6 = (f16(b) for b in rp.cos_c)
    inc = orc.rope_inc(D, BASE)
    y = np.empty_like(x)
    for s in range(S):
        for i in range(D // 2):
            ph = (s * int(inc[i])) % 2 ** 32
            u = coord(ph) if coord else int(orc.rope_coord(ph)[0])
            w = fma(u, u, NEG0)
            sn = fma(fma(fma(a5, w, a3), w, a1), u, NEG0)
            c = fma(fma(b6, w, b4), w, b2)
            c = cos_last(c, w, b0) if cos_last else fma(c, w, b0)
            x0, x1 = int(x[s, 2 * i]), int(x[s, 2 * i + 1])
            if rot:
                y[s, 2 * i], y[s, 2 * i + 1] = rot(x0, x1, sn, c)
            else:
                y[s, 2 * i] = fma(x0, c, fma(x1, sn, NEG0) ^ 0x8000)
                y[s, 2 * i + 1] = fma(x1, c, fma(x0, sn, NEG0))
    return y


def differing(got, want):
    return int(np.sum(got != want))


def test_unmutated_replay_matches(orc, case):
    x, got = case
    rp = orc.rope_prog()
    assert differing(got, replay(orc, rp, x)) == 0
    assert differing(got, orc.rope_rows(rp, orc.rope_inc(D, BASE), x, np.arange(S))) == 0


@pytest.mark.parametrize("which", ["sin0", "sin1", "sin2", "cos0", "cos1", "cos2", "cos3"])
@pytest.mark.parametrize("step", [1, -1])
def test_coefficient_ulp_mutants_detected(orc, case, which, step):
    x, got = case
    rp = orc.rope_prog()
    m = orc.RopeProg()
    C.memmove(C.byref(m), C.byref(rp), C.sizeof(orc.RopeProg))
    arr = m.sin_c if which.startswith("sin") else m.cos_c
    j = int(which[3])
    arr[j] = (arr[j] + step) & 0xFFFF
    ref = orc.rope_rows(m, orc.rope_inc(D, BASE), x, np.arange(S))
    assert differing(got, ref) > 0, f"{which} {step:+d} ulp not detected"


def test_order_mutants_detected(orc, case):
    x, got = case
    rp = orc.rope_prog()
    fma = orc.lib().orc_fma_f16
    f64 = orc.lib().orc_f16_to_f64
    to16 = orc.lib().orc_f64_to_f16

    def coord_round(ph):      # nearest instead of truncation
        v = ((((ph + (1 << 15)) % 2 ** 32) >> 16) ^ 0x8000) - 0x8000
        return to16(v / 32768.0)

    def rot_split(x0, x1, sn, c):   # product and sum rounded separately
        y0 = to16(f64(fma(x0, c, NEG0)) - f64(fma(x1, sn, NEG0)))
        y1 = to16(f64(fma(x1, c, NEG0)) + f64(fma(x0, sn, NEG0)))
        return y0, y1

    def rot_reverse(x0, x1, sn, c):  # the opposite sense of rotation
        return fma(x0, c, fma(x1, sn, NEG0)), fma(x1, c, fma(x0, sn, NEG0) ^ 0x8000)

    def cos_split(c, w, b0):
        return to16(f64(fma(c, w, NEG0)) + f64(b0))

    for name, kw in (("coordinate rounded", {"coord": coord_round}),
                     ("rotation split", {"rot": rot_split}),
                     ("rotation reversed", {"rot": rot_reverse}),
                     ("cosine last stage split", {"cos_last": cos_split})):
        assert differing(got, replay(orc, rp, x, **kw)) > 0, f"{name} not detected"
