"""Pins for the oracle's binary formats and correctly rounded operations.

The oracle (oracle/orc_fp.c) decodes FP16/BF16, rounds to nearest-even and
computes single-rounded fused multiply-adds.  These tests check it against
things other than itself:
  * numpy's float16 conversions and torch's float32 -> bfloat16 conversion
    (independent implementations of the same IEEE / bfloat16 rounding);
  * exact rational arithmetic (fractions.Fraction) with rounding done by
    brute force: a binary search over the sorted table of all 65,536 values
    of the format, the nearest one kept, ties to the even bit pattern.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f16_value(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


class _Table:
    """All finite values of a 16-bit format, sorted, for brute-force rounding."""

    def __init__(self, decode, inf_bits, max_bits):
        vals = []
        for b in range(65536):
            v = decode(b)
            if math.isfinite(v):
                vals.append((v, b))
        vals.sort(key=lambda t: (t[0], t[1]))
        # keep one entry per value (+0 wins over -0; sign of zero decided apart)
        self.vals, self.bits = [], []
        for v, b in vals:
            if self.vals and self.vals[-1] == v:
                continue
            self.vals.append(v)
            self.bits.append(b)
        self.inf_bits = inf_bits
        self.max = decode(max_bits)
        below_max = self.vals[-2]
        self.overflow = Fraction(self.max) + (Fraction(self.max) - Fraction(below_max)) / 2

    def round(self, v: Fraction, neg_zero_hint=False):
        if v == 0:
            return 0x8000 if neg_zero_hint else 0
        if abs(v) >= self.overflow:
            return self.inf_bits | (0x8000 if v < 0 else 0)
        i = bisect.bisect_left(self.vals, v)
        if i < len(self.vals) and self.vals[i] == v:
            b = self.bits[i]
        else:
            lo, hi = i - 1, i
            dl = v - Fraction(self.vals[lo])
            dh = Fraction(self.vals[hi]) - v
            if dl < dh:
                b = self.bits[lo]
            elif dh < dl:
                b = self.bits[hi]
            else:
                b = self.bits[lo] if (self.bits[lo] & 1) == 0 else self.bits[hi]
        if self.vals[self.bits.index(b)] == 0:
            return 0x8000 if v < 0 else 0   # underflow keeps the sign
        return b


@pytest.fixture(scope="module")
def f16_table():
    return _Table(_f16_value, 0x7C00, 0x7BFF)


@pytest.fixture(scope="module")
def bf16_table(orc):
    return _Table(lambda b: orc.lib().orc_bf16_to_f64(b), 0x7F80, 0x7F7F)


def test_decode_all_patterns(orc):
    L = orc.lib()
    f16 = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(65536):
        a, r = L.orc_f16_to_f64(b), f16[b]
        assert (math.isnan(a) and math.isnan(r)) or (a == r and math.copysign(1, a) == math.copysign(1, r)), b
        a, r = L.orc_bf16_to_f64(b), bf[b]
        assert (math.isnan(a) and math.isnan(r)) or (a == r and math.copysign(1, a) == math.copysign(1, r)), b


def test_f64_to_f16_matches_numpy(orc):
    L = orc.lib()
    rng = np.random.default_rng(11)
    # random doubles across the FP16 range, exact ties, subnormals, overflow edge
    xs = list(rng.standard_normal(20000) * np.exp2(rng.integers(-30, 17, 20000)))
    halfs = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.arange(1, 0x7C01, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    xs += list((halfs + nxt) / 2)                      # exact midpoints
    xs += [65504.0, 65519.99, 65520.0, 65536.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26,
           2.0**-26, -0.0, 0.0, 1e-300, -1e300]
    for x in xs:
        for s in (1.0, -1.0):
            v = s * x
            ref = int(np.array([v]).astype(np.float16).view(np.uint16)[0])
            assert L.orc_f64_to_f16(v) == ref, v


def test_f32_to_bf16_matches_torch(orc):
    L = orc.lib()
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, np.arange(0, 1 << 20, 3, dtype=np.uint32),   # subnormals
                           (np.arange(0, 65536, dtype=np.uint32) << 16) | 0x8000,  # ties
                           np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF], dtype=np.uint32)])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, r in zip(f[::7], ref[::7]):
        assert L.orc_f32_to_bf16(float(x)) == r, (x, hex(r))
    for x, r in zip(f[-70000:], ref[-70000:]):
        assert L.orc_f32_to_bf16(float(x)) == r, (x, hex(r))


def _triples(rng, n, max_finite):
    t = rng.integers(0, 65536, (n, 3)).astype(np.int64)
    # bias towards interesting magnitudes: subnormals, near-cancellation
    t[: n // 4, 0] &= 0x83FF
    t[n // 4: n // 2, 2] = t[n // 4: n // 2, 0] ^ 0x8000
    return [tuple(int(v) for v in row) for row in t]


def test_fma_f16_exact(orc, f16_table):
    L = orc.lib()
    rng = np.random.default_rng(13)
    cases = _triples(rng, 6000, 0x7BFF)
    cases += [(0x0001, 0x0001, 0x0000), (0x0001, 0x0001, 0x8000), (0x8001, 0x0001, 0x0000),
              (0x7BFF, 0x7BFF, 0xFBFF), (0x3C00, 0x3C01, 0xBC00), (0x0200, 0x3800, 0x0000),
              (0x0001, 0x3800, 0x0000), (0x0003, 0x3800, 0x0000), (0x3C00, 0x0000, 0x8000),
              (0x8000, 0x3C00, 0x8000), (0x5BFF, 0x5BFF, 0x0001)]
    for a, b, c in cases:
        va, vb, vc = _f16_value(a), _f16_value(b), _f16_value(c)
        if not all(math.isfinite(v) for v in (va, vb, vc)):
            continue
        exact = Fraction(va) * Fraction(vb) + Fraction(vc)
        if exact == 0:
            negp = ((a ^ b) >> 15) & 1
            negz = (va * vb == 0) and vc == 0 and negp and (c >> 15)
            ref = 0x8000 if negz else 0
        else:
            ref = f16_table.round(exact)
        assert L.orc_fma_f16(a, b, c) == ref, (hex(a), hex(b), hex(c), hex(ref))


def test_fma_bf16_exact(orc, bf16_table):
    L = orc.lib()
    rng = np.random.default_rng(14)
    cases = _triples(rng, 6000, 0x7F7F)
    # wide exponent gaps, where one double addition would round
    cases += [(0x7F00, 0x3F80, 0x0001), (0x0001, 0x0001, 0x3F80), (0x3F81, 0x3F81, 0xB3A0),
              (0x4000, 0x3F80, 0x8001), (0x7F7F, 0x3F80, 0x7F7F)]
    for a, b, c in cases:
        va, vb, vc = (L.orc_bf16_to_f64(v) for v in (a, b, c))
        if not all(math.isfinite(v) for v in (va, vb, vc)):
            continue
        exact = Fraction(va) * Fraction(vb) + Fraction(vc)
        if exact == 0:
            continue
        ref = bf16_table.round(exact)
        assert L.orc_fma_bf16(a, b, c) == ref, (hex(a), hex(b), hex(c), hex(ref))


def _round_f32_exact(v: Fraction):
    """RNE of an exact rational to binary32, by the definition (test helper)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, -126) - 23
    s = a / Fraction(2) ** q
    n = s.numerator // s.denominator
    fr = s - n
    if fr > Fraction(1, 2) or (fr == Fraction(1, 2) and n % 2):
        n += 1
    r = n * Fraction(2) ** q
    return r if v > 0 else -r


def test_fma_f32_then_bf16(orc, bf16_table):
    """The two-rounding BF16 order: RN_bf16(RN_f32(a*b + c))."""
    L = orc.lib()
    rng = np.random.default_rng(15)
    n_diff_from_single = 0
    for a, b, c in _triples(rng, 4000, 0x7F7F):
        va, vb, vc = (L.orc_bf16_to_f64(v) for v in (a, b, c))
        if not all(math.isfinite(v) for v in (va, vb, vc)):
            continue
        exact = Fraction(va) * Fraction(vb) + Fraction(vc)
        if exact == 0:
            continue
        r32 = _round_f32_exact(exact)
        if abs(r32) >= Fraction(2) ** 128:
            continue
        ref = bf16_table.round(r32)
        got = L.orc_fma_f32_bf16(a, b, c)
        assert got == ref, (hex(a), hex(b), hex(c))
        n_diff_from_single += got != L.orc_fma_bf16(a, b, c)
    # double rounding differs from single rounding only rarely
    assert n_diff_from_single < 40
