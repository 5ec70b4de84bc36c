"""The attention backward's two forms give the same bits.

With the dS blocks stored (the default while they fit
pa_attn_bwd_ds_limit) the dK/dV kernel writes the BF16 dS it forms
and dQ is a product over those blocks; with the limit at 0 a dQ kernel
recomputes S, dP and the transform.  Both use the same products in the same
order, so dQ, dK and dV must agree bit for bit, for every score transform,
both causal settings, grouped heads and ragged lengths.  (Each form is also
checked against the oracle by the parity tests.)  Inputs: the seeded
N(0, 1) BF16 Q, K, V, dO; O and lse from the library's forward.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


def bits(t):
    return t.view(torch.int16).cpu().numpy()


def both_forms(pa, run):
    """run() under the default limit, then with the limit at 0; the limit is
    restored whatever happens."""
    lim = pa.attn_bwd_ds_limit()
    assert lim > 0
    stored = [bits(t) for t in run()]
    torch.cuda.synchronize()
    pa.attn_bwd_ds_limit(0)
    try:
        recomputed = [bits(t) for t in run()]
        torch.cuda.synchronize()
    finally:
        pa.attn_bwd_ds_limit(lim)
    return stored, recomputed


SHAPES = [(1, 2, 2, 300, True), (2, 3, 3, 257, False), (1, 4, 1, 130, True), (1, 4, 2, 200, False),
          (1, 1, 1, 1, True), (1, 2, 2, 64, True), (1, 2, 1, 515, True)]
SOFTCAP = [("bf16", None), ("f16", None), ("native", None), ("bf16", "d1"), ("bf16", "pwl2")]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("variant", SOFTCAP)
def test_softcap_forms_agree(pa, shape, variant):
    B, H, Hkv, S, causal = shape
    fmt, core = variant
    note(f"softcap backward forms {fmt} core={core} {shape}")
    q, k, v = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    do = si.t_attn_grad(B, H, S)
    if fmt == "native":
        o, lse = pa.native_softcap_attn_fwd(q, k, v, 50.0, causal, with_lse=True)
        run = lambda: pa.native_softcap_attn_bwd(q, k, v, o, do, lse, 50.0, causal)  # noqa: E731
    elif core is not None:
        o, lse = pa.poly_softcap_attn_fwd_exp2(q, k, v, 50.0, causal, core=core, with_lse=True)
        run = lambda: pa.poly_softcap_attn_bwd(q, k, v, o, do, lse, 50.0, causal, core=core)  # noqa: E731
    else:
        o, lse = pa.poly_softcap_attn_fwd(q, k, v, 50.0, causal, fmt=fmt, with_lse=True)
        run = lambda: pa.poly_softcap_attn_bwd(q, k, v, o, do, lse, 50.0, causal, fmt=fmt)  # noqa: E731
    stored, recomputed = both_forms(pa, run)
    for name, a, b in zip(("dq", "dk", "dv"), stored, recomputed):
        assert np.array_equal(a, b), f"{name}: {int(np.sum(a != b))} of {a.size} differ"


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_softcap_forms_agree_at_scale(pa, fmt):
    """A longer causal run (1 x 16 x 4096, 2048 workgroups per kernel), where
    waves drift far out of step: a missing wait or barrier shows up as bits
    that differ between the forms or between repeats."""
    B, H, S = 1, 16, 4096
    note(f"softcap backward forms at scale {fmt}")
    q, k, v = si.t_attn_inputs(B, H, S)
    do = si.t_attn_grad(B, H, S)
    o, lse = pa.poly_softcap_attn_fwd(q, k, v, 50.0, True, fmt=fmt, with_lse=True)
    run = lambda: pa.poly_softcap_attn_bwd(q, k, v, o, do, lse, 50.0, True, fmt=fmt)  # noqa: E731
    first = [bits(t) for t in run()]
    stored, recomputed = both_forms(pa, run)
    for name, a, b, c in zip(("dq", "dk", "dv"), first, stored, recomputed):
        assert np.array_equal(a, b), f"{name}: repeat differs in {int(np.sum(a != b))} of {a.size}"
        assert np.array_equal(b, c), f"{name}: {int(np.sum(b != c))} of {b.size} differ"


@pytest.mark.parametrize("shape", [(1, 4, 2, 4096, True), (1, 2, 2, 4096, False)])
@pytest.mark.parametrize("poly", [True, False])
def test_sigmoid_forms_agree(pa, shape, poly):
    B, H, Hkv, S, causal = shape
    note(f"sigmoid backward forms poly={poly} {shape}")
    q, k, v = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    do = si.t_attn_grad(B, H, S)
    f = pa.poly_sigmoid_attn_bwd if poly else pa.native_sigmoid_attn_bwd
    stored, recomputed = both_forms(pa, lambda: f(q, k, v, do, causal))
    for name, a, b in zip(("dq", "dk", "dv"), stored, recomputed):
        assert np.array_equal(a, b), f"{name}: {int(np.sum(a != b))} of {a.size} differ"


def test_sigmoid_without_workspace_takes_the_recompute_form(pa):
    """H == Hkv: a NULL workspace is allowed and gives the same bits."""
    B, H, S = 1, 2, 333
    q, k, v = si.t_attn_inputs(B, H, S)
    do = si.t_attn_grad(B, H, S)
    note("native sigmoid backward, NULL workspace")
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    L = pa.lib()
    st = L.native_sigmoid_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), None, B, H, H, S, 128, 1,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref = pa.native_sigmoid_attn_bwd(q, k, v, do, True)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert np.array_equal(bits(a), bits(b))
