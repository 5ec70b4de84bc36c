"""Bit-exact readback of the two-region sigmoid program inside the attention
kernels, over every finite BF16 score (section 3.4; Eq. 14 at n = 4096).

The inputs make each program value land, untouched, in one output element:

* forward: K and V rows 0..127 are the unit vectors e_j (the other keys are
  zero), so S[i][j] = Q[i][j] exactly and O[i][j] = 1 * P(Q[i][j]) for
  j < 128 (masked keys give 0);
* backward: query row 0 of every head is e_0, dO row 0 is e_0, the other
  query and dO rows are zero, K[j] = x_j e_0 and V[j] = e_0, so
  dV[j][0] = P(x_j) and dK[j][0] = g(x_j) / sqrt(D), where g is the
  program's factored derivative surrogate; every other element of dK and dV
  is zero.

The expected P and g come from the oracle's program evaluated at the BF16
input x = RN_bf16(RN_f32(s * RN_f32(1 / sqrt D))), the same FP32 product the
kernels form.  dK's last step (the FP32 product of g and 1 / sqrt D, then a
BF16 rounding) is the kernels' stated order and is taken the same way here.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from attn_util import bf16v, sig_prog
from gpu_util import diff_report, note, to_bits, to_dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
S, D = 4096, 128


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def tables(orc):
    sp = sig_prog(orc)
    p, g = orc.sig_prog_eval(sp, np.arange(65536, dtype=np.uint16))
    return p, g


def finite_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b[(b & 0x7F80) == 0x7F80] = 0          # the 256 infinities and NaNs
    return b


SCALE = np.float32(1.0 / np.sqrt(float(D)))


def x_bits(s_bits):
    prod = bf16v(s_bits).astype(np.float32) * SCALE      # FP32 product, RNE
    return si.to_bf16_bits(prod.astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_forward_program_every_score(pa, tables, causal):
    p_tab, _ = tables
    rng = np.random.default_rng(71)
    pat = finite_patterns()
    q = np.concatenate([rng.permutation(pat) for _ in range(S * D // pat.size)]).reshape(S, D)
    eye = np.zeros((S, D), np.uint16)
    eye[np.arange(D), np.arange(D)] = 0x3F80                # BF16 1.0
    note(f"sigmoid readback fwd causal={causal}")
    o = pa.poly_sigmoid_attn_fwd(to_dev(q[None, None], BF), to_dev(eye[None, None], BF),
                                 to_dev(eye[None, None], BF), causal)
    got = to_bits(o).reshape(S, D)
    ref = p_tab[x_bits(q)]
    if causal:
        ref = np.where(np.arange(D)[None, :] <= np.arange(S)[:, None], ref, np.uint16(0))
    assert np.array_equal(got, ref), diff_report(got.ravel(), ref.ravel(), q.ravel())


def test_backward_program_every_score(pa, tables):
    p_tab, g_tab = tables
    H = 16                                                  # 16 heads x 4096 keys
    xs = np.random.default_rng(72).permutation(finite_patterns()).reshape(H, S)
    q = np.zeros((1, H, S, D), np.uint16)
    q[0, :, 0, 0] = 0x3F80
    do = q.copy()
    k = np.zeros((1, H, S, D), np.uint16)
    k[0, :, :, 0] = xs
    v = np.zeros((1, H, S, D), np.uint16)
    v[0, :, :, 0] = 0x3F80
    note("sigmoid readback bwd H=16 S=4096 causal=False")
    dq, dk, dv = pa.poly_sigmoid_attn_bwd(to_dev(q, BF), to_dev(k, BF), to_dev(v, BF),
                                          to_dev(do, BF), False)
    dk, dv = to_bits(dk).reshape(H * S, D), to_bits(dv).reshape(H * S, D)
    xb = x_bits(xs.ravel())
    p_ref = p_tab[xb]
    g32 = bf16v(g_tab[xb]).astype(np.float32) * SCALE       # FP32 product, RNE
    dk_ref = si.to_bf16_bits(g32.astype(np.float64))
    assert np.array_equal(dv[:, 0], p_ref), diff_report(dv[:, 0], p_ref, xs.ravel())
    assert np.array_equal(dk[:, 0], dk_ref), diff_report(dk[:, 0], dk_ref, xs.ravel())
    # nothing leaks into the other columns (+0 or -0 only)
    assert not np.any(dv[:, 1:] & 0x7FFF) and not np.any(dk[:, 1:] & 0x7FFF)
    dq = to_bits(dq).reshape(H, S, D)
    assert not np.any(dq[:, 1:] & 0x7FFF) and not np.any(dq[:, 0, 1:] & 0x7FFF)
