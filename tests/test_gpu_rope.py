"""GPU parity of the rotary embedding ("Fast Polynomial Transcendentals for
LLMs", Appendix B.2) through the C ABI.

* poly_rope against the oracle's replay, bit for bit: ragged sizes, every
  supported head-dimension class, special values, positions past the phase
  wraparound, and sampled positions of the Llama-3-8B-like geometry the
  bench times (1 x 4096 x 32 query / 8 key heads x 128);
* the comparator: pa_rope_table's (cos, sin) within one FP16 ulp of the
  exact values at the same angle, native_rope bit-identical to
  native_rope_table, and both equal to the oracle's rotation applied with
  the table's values.
Inputs: N(0, 1) FP16 from the seeded generator (seed 9 for Q, 10 for K).
"""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import note, to_bits, to_dev

pytestmark = pytest.mark.gpu
F16 = torch.float16
BASE = 10000.0


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def rp(orc):
    return orc.rope_prog()


def inputs(B, S, Hq, Hkv, D):
    q = si.to_f16_bits(si.normal(9, B * S * Hq * D)).reshape(B, S, Hq, D)
    k = si.to_f16_bits(si.normal(10, B * S * Hkv * D)).reshape(B, S, Hkv, D)
    return q, k


def oracle(orc, rp, x, D, pos_rows=None):
    """Expected [B, H, S, D] bits of x [B, S, H, D] (or of the positions
    pos_rows only, as [B, H, len, D])."""
    B, S, H, _ = x.shape
    s_idx = np.arange(S) if pos_rows is None else np.asarray(pos_rows)
    rows = x[:, s_idx].transpose(0, 2, 1, 3).reshape(-1, D)      # (b, h, s) order
    pos = np.tile(s_idx, B * H).astype(np.int64)
    y = orc.rope_rows(rp, orc.rope_inc(D, BASE), rows, pos)
    return y.reshape(B, H, s_idx.size, D)


def same_bits(got, want, label):
    """Bit-exact except that NaN matches NaN (payloads are not compared)."""
    gn = np.isnan(got.view(np.float16))
    wn = np.isnan(want.view(np.float16))
    assert np.array_equal(gn, wn), label
    bad = (got != want) & ~gn
    assert not bad.any(), f"{label}: {int(bad.sum())} of {got.size} differ"


@pytest.mark.parametrize("shape", [(2, 67, 4, 2, 128), (1, 1, 3, 1, 64), (1, 300, 2, 2, 8),
                                   (1, 5, 1, 1, 512), (3, 33, 2, 1, 136), (1, 9, 5, 3, 16)])
def test_poly_rope_bit_exact(pa, orc, rp, shape):
    B, S, Hq, Hkv, D = shape
    note(f"poly_rope {shape}")
    q, k = inputs(B, S, Hq, Hkv, D)
    qo, ko = pa.poly_rope(to_dev(q, F16), to_dev(k, F16), BASE)
    torch.cuda.synchronize()
    same_bits(to_bits(qo), oracle(orc, rp, q, D), f"q {shape}")
    same_bits(to_bits(ko), oracle(orc, rp, k, D), f"k {shape}")


def test_poly_rope_special_values(pa, orc, rp):
    B, S, Hq, Hkv, D = 1, 16, 2, 1, 64
    q, k = inputs(B, S, Hq, Hkv, D)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00,
                         0x7E00, 0x3C00, 0xBC00], dtype=np.uint16)
    q.reshape(-1)[: specials.size * 8] = np.repeat(specials, 8)
    k.reshape(-1)[1::7] = specials[np.arange(k.size)[1::7] % specials.size]
    note("poly_rope special values")
    qo, ko = pa.poly_rope(to_dev(q, F16), to_dev(k, F16), BASE)
    torch.cuda.synchronize()
    same_bits(to_bits(qo), oracle(orc, rp, q, D), "q specials")
    same_bits(to_bits(ko), oracle(orc, rp, k, D), "k specials")


def test_poly_rope_long_sequence_sampled(pa, orc, rp):
    """Positions up to 70,000: every frequency's phase wraps many times."""
    B, S, Hq, Hkv, D = 1, 70000, 1, 1, 128
    note("poly_rope S = 70000")
    q, k = inputs(B, S, Hq, Hkv, D)
    qo, ko = pa.poly_rope(to_dev(q, F16), to_dev(k, F16), BASE)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, S, 97), np.arange(S - 40, S)]))
    same_bits(to_bits(qo)[:, :, rows], oracle(orc, rp, q, D, rows), "q long")
    same_bits(to_bits(ko)[:, :, rows], oracle(orc, rp, k, D, rows), "k long")


def test_poly_rope_bench_geometry_sampled(pa, orc, rp):
    B, S, Hq, Hkv, D = 1, 4096, 32, 8, 128
    note("poly_rope 1 x 4096 x 32 (8) x 128")
    q, k = inputs(B, S, Hq, Hkv, D)
    qo, ko = pa.poly_rope(to_dev(q, F16), to_dev(k, F16), BASE)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, S, 61), [S - 1]]))
    same_bits(to_bits(qo)[:, :, rows], oracle(orc, rp, q, D, rows), "q bench")
    same_bits(to_bits(ko)[:, :, rows], oracle(orc, rp, k, D, rows), "k bench")


def test_native_table_values(pa, orc):
    S, D = 3000, 128
    note("pa_rope_table")
    t = pa.rope_table(S, D, BASE)
    torch.cuda.synchronize()
    w = t.cpu().numpy().view(np.uint32)
    cs = (w & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    sn = (w >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    inc = orc.rope_inc(D, BASE).astype(np.uint64)
    ph = (np.arange(S, dtype=np.uint64)[:, None] * inc[None, :]) & 0xFFFFFFFF
    v = ((ph >> 16).astype(np.int64) ^ 0x8000) - 0x8000
    th = (v.astype(np.float32) * np.float32(math.pi / 32768)).astype(np.float64)   # the FP32 angle
    for got, want in ((cs, np.cos(th)), (sn, np.sin(th))):
        ref = want.astype(np.float16).astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp), float(np.max(np.abs(got - ref) / ulp))
        assert np.mean(got == ref) > 0.999


def test_native_rope_equals_table_and_oracle_rotation(pa, orc):
    B, S, Hq, Hkv, D = 2, 129, 3, 1, 64
    note("native_rope / native_rope_table")
    q, k = inputs(B, S, Hq, Hkv, D)
    qd, kd = to_dev(q, F16), to_dev(k, F16)
    qn, kn = pa.native_rope(qd, kd, BASE)
    t = pa.rope_table(S, D, BASE)
    qt, kt = pa.native_rope_table(qd, kd, t)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(qn), to_bits(qt)) and np.array_equal(to_bits(kn), to_bits(kt))
    w = t.cpu().numpy().view(np.uint32).reshape(S, D // 2)
    x = q[1, 5, 2]
    y = np.array([orc.rope_rotate(x[2 * i], x[2 * i + 1], int(w[5, i] >> 16), int(w[5, i] & 0xFFFF))
                  for i in range(D // 2)], dtype=np.uint16).reshape(-1)
    assert np.array_equal(to_bits(qt)[1, 2, 5], y)
