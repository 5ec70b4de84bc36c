"""Bit-exact readback of the softcap tanh program and of its analytic
derivative inside the attention kernels, in BF16 and in FP16, over every
value x of the program's input format with x_min <= |x| <= 1.5 Lc (x_min =
2^-12 in BF16, 2^-9 in FP16; Eq. 1, section 3.3, section 5.2.2).

Every query row sees exactly one key (S = 1, one head per tested x): head h
has q = (a, b, 0, ...) and k = (1, 1, 0, ...) with BF16 a, b chosen on the
host so that the kernels' scaled score RN_fmt(RN_f32(RN_f32(a + b) *
RN_f32(1 / (cap sqrt D)))) is the tested x (a + b is exact in FP32, so the
MFMA's sum is too).

* forward: the row's log-sum-exp is (m + log2 P) ln 2 with P = 2^z,
  z = RN_f32(t RN_f32(cap log2 e) - m): it identifies t, since the lse of the
  two neighbouring program values lies about 8x further away than the FP32
  error of exp2 / log2 / ln 2 (about 1e-5; x_min keeps neighbours apart), and
  the test asserts the measured error stays below a quarter of that gap;
* backward: dO = V = e_0 and O = 0 give dP - Delta = 1; the lse passed in is
  RN_f32(RN_f32(t c2) / log2 e), so P = 2^z with z = RN_f32(t c2 -
  RN_f32(lse log2 e)) close to 0 (replayed on the host), dS =
  RN_bf16(RN_f32(q'(x) P)) and dQ[0] = RN_bf16(RN_f32(dS RN_f32(1 / sqrt D))).
  The expected dQ is formed from the oracle's q'(x) with that P and its FP32
  neighbours (the hardware exponential is within an ulp); any of the three
  is accepted (for BF16 q' all three agree).  Beyond the clamp q'(x) = 0, so
  dQ = 0.

The expected t and q' are the oracle's program and derivative-program
values at x.
"""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from attn_util import tanh_prog
from gpu_util import note, to_bits, to_dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
CAP, D = 50.0, 128
SCALE = np.float32(1.0 / (CAP * math.sqrt(D)))
C2 = np.float32(CAP * math.log2(math.e))
MREF = math.ceil(float(np.float32(C2 - np.float32(40.0))))
LOG2E = np.float32(math.log2(math.e))
RSD = np.float32(1.0 / math.sqrt(D))


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def tp(orc):
    return tanh_prog(orc)


def fmt_values(fmt, lo, hi):
    """Bits and values of every positive and negative value of the format
    with lo <= |x| <= hi."""
    allb = np.arange(0x8000, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        v = bits_to_f64(allb, fmt)
    keep = np.isfinite(v) & (v >= lo) & (v <= hi)
    b = allb[keep]
    return np.concatenate([b, b | 0x8000])


def bits_to_f64(b, fmt):
    b = np.asarray(b, np.uint16)
    if fmt == "f16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_fmt(xs32, fmt):
    if fmt == "f16":
        return xs32.astype(np.float16).view(np.uint16)
    return si.to_bf16_bits(xs32.astype(np.float64))


def inputs_for(xbits, fmt):
    """(q, k bits [1, N, 1, 128], hit mask): a + b with a, b BF16 close to
    x / scale, kept where the kernels' rounding chain lands on x."""
    x = bits_to_f64(xbits, fmt)
    target = x / np.float64(SCALE)
    a = si.to_bf16_bits(target)
    av = bits_to_f64(a, "bf16")
    b = si.to_bf16_bits(target - av)
    bv = bits_to_f64(b, "bf16")
    # keep b only where a + b is exact in FP32 (then the MFMA's sum is too)
    exact = (av + bv).astype(np.float32).astype(np.float64) == av + bv
    b = np.where(exact, b, 0).astype(np.uint16)
    bv = np.where(exact, bv, 0.0)
    s32 = (av + bv).astype(np.float32)
    xs = (s32 * SCALE).astype(np.float32)
    hit = to_fmt(xs, fmt) == xbits
    n = xbits.size
    q = np.zeros((1, n, 1, D), np.uint16)
    q[0, :, 0, 0], q[0, :, 0, 1] = a, b
    k = np.zeros((1, n, 1, D), np.uint16)
    k[0, :, 0, :2] = 0x3F80
    return q, k, hit


def lse_of(t):
    """The forward's lse for program value t (FP64 after the FP32 exponent)."""
    z = (np.asarray(t, np.float64) * np.float64(C2) - MREF).astype(np.float32).astype(np.float64)
    return (MREF + z) * math.log(2.0)


def neighbours(tbits, fmt):
    """Adjacent format values of t (one step up and down in magnitude)."""
    mag = tbits & 0x7FFF
    sign = tbits & 0x8000
    up = (mag + 1) | sign
    dn = np.where(mag > 0, (mag - 1) | sign, tbits)
    return bits_to_f64(up, fmt), bits_to_f64(dn, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_softcap_program_and_derivative_bit_exact_in_kernels(pa, orc, tp, fmt):
    Lc = tp.Lc
    xbits = fmt_values(fmt, 2.0 ** (-12 if fmt == "bf16" else -9), 1.5 * Lc)
    q, k, hit = inputs_for(xbits, fmt)
    assert hit.mean() > 0.95
    xbits, q, k = xbits[hit], q[:, hit], k[:, hit]
    n = xbits.size
    order = orc.TANH_ORDERS[fmt]
    tbits = orc.act_fwd(tp, xbits, order)
    t = bits_to_f64(tbits, fmt)
    dq_ = bits_to_f64(orc.dtanh_prog(tp, xbits, fmt), fmt)
    v = np.zeros((1, n, 1, D), np.uint16)
    v[0, :, 0, 0] = 0x3F80
    note(f"softcap readback fmt={fmt}: {n} program inputs, one head each")

    # forward: lse identifies t
    qd, kd, vd = to_dev(q, BF), to_dev(k, BF), to_dev(v, BF)
    _, lse = pa.poly_softcap_attn_fwd(qd, kd, vd, CAP, True, with_lse=True, fmt=fmt)
    lse = lse.cpu().numpy().ravel().astype(np.float64)
    want = lse_of(t)
    up, dn = neighbours(tbits, fmt)
    gap = np.minimum(np.abs(lse_of(up) - want), np.abs(lse_of(dn) - want))
    err = np.abs(lse - want)
    assert np.all(err < 0.25 * gap), f"{int(np.sum(err >= 0.25 * gap))} program values differ"
    print(f"[readback] {fmt} forward: {n} program values identified, max lse error "
          f"{err.max():.2e} (closest neighbour {gap.min():.2e})", flush=True)

    # backward: dQ[0] = RN_bf16(RN_f32(RN_bf16(RN_f32(q' P)) rsd)) with
    # P = 2^RN_f32(t c2 - RN_f32(lse log2 e)) near 1 (t c2 is exact in FP64;
    # the exponential within an ulp)
    tc2 = t * np.float64(C2)
    lse_in = (tc2 / np.float64(LOG2E)).astype(np.float32)
    nl = -(lse_in * LOG2E).astype(np.float32).astype(np.float64)
    z = (tc2 + nl).astype(np.float32).astype(np.float64)
    p0 = np.exp2(z).astype(np.float32)
    assert np.all(np.abs(p0 - 1.0) < 2.0 ** -12)
    do = v.copy()
    o = np.zeros_like(q)
    dq, dk, dv = pa.poly_softcap_attn_bwd(qd, kd, vd, to_dev(o, BF), to_dev(do, BF),
                                          torch.from_numpy(lse_in.reshape(1, n, 1)).cuda(), CAP,
                                          True, fmt=fmt)
    dq0 = to_bits(dq).reshape(n, D)[:, 0]
    ok = np.zeros(n, bool)
    for p in (p0, np.nextafter(p0, np.float32(2.0)), np.nextafter(p0, np.float32(0.0))):
        ds = si.to_bf16_bits((dq_.astype(np.float32) * p).astype(np.float32).astype(np.float64))
        dsv = bits_to_f64(ds, "bf16").astype(np.float32)
        ok |= si.to_bf16_bits((dsv * RSD).astype(np.float32).astype(np.float64)) == dq0
    beyond = np.abs(bits_to_f64(xbits, fmt)) > Lc
    print(f"[readback] {fmt} backward: {int(ok.sum())} of {n} dQ bit-exact "
          f"({int(beyond.sum())} beyond the clamp, q' = 0)", flush=True)
    assert np.all(ok), f"{int((~ok).sum())} derivative values differ, e.g. x bits " \
                       f"{[hex(b) for b in xbits[~ok][:5]]}"
    assert np.all(dq0[beyond] & 0x7FFF == 0)
