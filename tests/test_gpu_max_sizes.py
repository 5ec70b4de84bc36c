"""GPU parity beyond 2^32 elements: 64-bit indexing of the streaming, the
SwiGLU and the rotary-embedding kernels.

Each input element is a hash of its own 64-bit index, so a kernel that
computed an address from a wrapped 32-bit index would read a different
value than the one at the sampled position and fail the comparison.  The
arrays are drawn on the GPU; outputs are compared with the oracle (bit-exact;
NaN against NaN for SwiGLU) on samples around 2^31 and 2^32, the first and
last elements (ragged tail) and a stride through the whole range.
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import bwd_prog_name, diff_report, fwd_prog_name, note, programs, to_bits

pytestmark = pytest.mark.gpu

MULT_X = 0x9E3779B97F4A7C1
MULT_G = 0x5851F42D4C957F3


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


def hashed(n, mult, dtype):
    """Element i = bits 40..55 of i * mult (mod 2^64), as a 16-bit value."""
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    step = 1 << 27
    for s in range(0, n, step):
        e = min(s + step, n)
        i = torch.arange(s, e, dtype=torch.int64, device="cuda")
        v = ((i * mult) >> 40) & 0xFFFF
        out[s:e] = torch.where(v >= 32768, v - 65536, v).to(torch.int16)
        del i, v
    return out.view(dtype)


def sample_index(n, width=2048, stride=999_983):
    parts = [np.arange(0, width), np.arange(n - width, n), np.arange(0, n, stride)]
    for b in (1 << 31, 1 << 32):
        if b < n:
            parts.append(np.arange(b - width, min(b + width, n)))
    return np.unique(np.concatenate(parts))


def free():
    gc.collect()
    torch.cuda.empty_cache()


def test_elementwise_beyond_2_32(pa, orc):
    """2^32 + 4,099 FP16 elements (a ragged tail): sigmoid D3 forward and
    sigmoid' D4 backward."""
    progs = programs(orc)
    n = (1 << 32) + 4099
    note(f"max size elementwise draw n={n}")
    xt = hashed(n, MULT_X, torch.float16)
    gt = hashed(n, MULT_G, torch.float16)
    idx = sample_index(n)
    it = torch.from_numpy(idx).cuda()
    xs, gs = to_bits(xt[it]), to_bits(gt[it])
    note("max size sigmoid fwd")
    y = pa.poly_act_fwd(xt, "sigmoid")
    got = to_bits(y[it])
    del y
    ref = orc.act_fwd(progs[fwd_prog_name("sigmoid")], xs, 1)
    assert np.array_equal(got, ref), diff_report(got, ref, xs)
    note("max size sigmoid bwd")
    dx = pa.poly_act_bwd(xt, gt, "sigmoid")
    got = to_bits(dx[it])
    del dx, xt, gt
    free()
    ref = orc.act_bwd(progs[bwd_prog_name("sigmoid")], xs, gs, 1)
    assert np.array_equal(got, ref), diff_report(got, ref, xs)


def test_swiglu_beyond_2_32(pa, orc):
    """Dense BF16 SwiGLU forward over 65,537 x 65,544 = 4,295,557,128
    elements, compared on whole rows around the 2^31 and 2^32 elements."""
    sig = programs(orc)["sigmoid_fwd_d3"]
    R, C = 65537, 65544
    note(f"max size swiglu draw {R}x{C}")
    gt = hashed(R * C, MULT_X, torch.bfloat16).view(R, C)
    ut = hashed(R * C, MULT_G, torch.bfloat16).view(R, C)
    note("max size swiglu fwd")
    h = pa.poly_swiglu_fwd(gt, ut)
    rows = sorted({0, R - 1, (1 << 31) // C, (1 << 31) // C + 1, (1 << 32) // C,
                   (1 << 32) // C + 1, R // 2})
    rt = torch.tensor(rows, dtype=torch.int64, device="cuda")
    g, u, got = to_bits(gt[rt]), to_bits(ut[rt]), to_bits(h[rt])
    del gt, ut, h
    free()
    ref = orc.swiglu_fwd(sig, g, u)
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    ok = (got == ref) | (nan_g & nan_r)
    assert bool(ok.all()), diff_report(got.ravel(), ref.ravel())


def test_rope_beyond_2_32(pa, orc):
    """Rotary embedding of Q [1, 2^21 + 3, 16, 128] (2^32 + 6,144 elements)
    and K [1, 2^21 + 3, 4, 128]: positions around the 2^31 and 2^32 input
    elements and the last one, every head (the outputs of heads >= 8 lie
    beyond 2^31 in the transposed layout), compared with the oracle."""
    S, Hq, Hkv, D = (1 << 21) + 3, 16, 4, 128
    note(f"max size rope draw S={S}")
    qt = hashed(S * Hq * D, MULT_X, torch.float16).view(1, S, Hq, D)
    kt = hashed(S * Hkv * D, MULT_G, torch.float16).view(1, S, Hkv, D)
    note("max size rope")
    qo, ko = pa.poly_rope(qt, kt, 10000.0)
    pos = np.unique(np.array([0, 1, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 21) - 1, 1 << 21,
                              S - 1] + list(range(0, S, 262_147))))
    pt = torch.from_numpy(pos).cuda()
    rp = orc.rope_prog()
    inc = orc.rope_inc(D, 10000.0)
    for x, y, H in ((qt, qo, Hq), (kt, ko, Hkv)):
        xs = to_bits(x[:, pt])                                   # [1, len, H, D]
        got = to_bits(y[:, :, pt])                               # [1, H, len, D]
        rows = xs.transpose(0, 2, 1, 3).reshape(-1, D)
        ref = orc.rope_rows(rp, inc, rows, np.tile(pos, H).astype(np.int64)).reshape(got.shape)
        nan_g = (got & 0x7FFF) > 0x7C00
        nan_r = (ref & 0x7FFF) > 0x7C00
        ok = (got == ref) | (nan_g & nan_r)
        assert bool(ok.all()), f"{int((~ok).sum())} of {got.size} differ"
    del qt, kt, qo, ko
    free()
