"""GPU parity of the attention backwards against the CPU oracle.

The backward entry points take the forward's O and log-sum-exp; here those
inputs come from the oracle's forward (O rounded to BF16, lse to FP32), and
the oracle's backward receives exactly the same values, so the comparison
isolates the backward.  dQ, dK and dV are checked against the oracle's replay
of the method's rounding steps (P and dS are the BF16 MFMA operands) with
the gate of attn_util: one BF16 ulp plus the oracle's spread.  Softcap: the
analytic derivative of the D4 tanh program in BF16 or FP16 (0 beyond the
clamp), with the hardware exponential or a software exp2 core, or 1 - tanh^2
(comparator); sigmoid: the factored surrogate (poly, at the fitted length
4096) or sigma (1 - sigma).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from attn_util import bf16v, check, fwd_for_bwd, sig_prog, tanh_prog
from gpu_util import note, to_bits, to_dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def tp(orc):
    return tanh_prog(orc)


@pytest.fixture(scope="module")
def sp(orc):
    return sig_prog(orc)


def draw(B, H, Hkv, S, seed, sd=1.0):
    rng = np.random.default_rng(seed)
    q = si.to_bf16_bits(rng.standard_normal((B, H, S, 128)) * sd)
    k, v = (si.to_bf16_bits(rng.standard_normal((B, Hkv, S, 128)) * sd) for _ in range(2))
    do = si.to_bf16_bits(rng.standard_normal((B, H, S, 128)))
    return q, k, v, do


def compare(orc, kind, q, k, v, o, do, lse, dq, dk, dv, qrows, krows, causal, label, **kw):
    D = q.shape[3]
    rq, rk, rv, sq, sk, sv = orc.attn_bwd_rows(
        kind, q, k, v, None if o is None else bf16v(o), do,
        None if lse is None else lse.astype(np.float64), qrows, krows, causal=causal, **kw)
    check(dq.reshape(-1, D)[qrows], rq, sq, f"{label} dQ")
    check(dk.reshape(-1, D)[krows], rk, sk, f"{label} dK")
    check(dv.reshape(-1, D)[krows], rv, sv, f"{label} dV")


FMTS = ("bf16", "f16", "native")


def softcap_variant(pa, orc, fmt, core=None):
    """(backward call, oracle kind, oracle keywords) of a softcap variant."""
    if fmt == "native":
        return (lambda *a: pa.native_softcap_attn_bwd(*a)), orc.ATTN_SOFTCAP_EXACT, {}
    kw = dict(tanh_fmt=fmt)
    if core is not None:
        kw["exp2_core"] = pa.EXP2_CORES[core]
    return ((lambda *a: pa.poly_softcap_attn_bwd(*a, fmt=fmt, core=core)), orc.ATTN_SOFTCAP_POLY, kw)


def softcap_case(pa, orc, tp, B, H, Hkv, S, causal, fmt, seed, qrows=None, krows=None, sd=1.0,
                 core=None, cap=50.0):
    q, k, v, do = draw(B, H, Hkv, S, seed, sd)
    call, kind, kw = softcap_variant(pa, orc, fmt, core)
    o, lse = fwd_for_bwd(orc, kind, q, k, v, causal, cap=cap, tanh_prog=tp, **kw)
    label = f"softcap bwd B={B} H={H} Hkv={Hkv} S={S} causal={causal} fmt={fmt} core={core} cap={cap}"
    note(label)
    dq, dk, dv = call(to_dev(q, BF), to_dev(k, BF), to_dev(v, BF), to_dev(o, BF), to_dev(do, BF),
                      torch.from_numpy(lse).cuda(), cap, causal)
    dq, dk, dv = to_bits(dq), to_bits(dk), to_bits(dv)
    qrows = np.arange(B * H * S) if qrows is None else qrows
    krows = np.arange(B * Hkv * S) if krows is None else krows
    compare(orc, kind, q, k, v, o, do, lse, dq, dk, dv, qrows, krows, causal, label, cap=cap,
            tanh_prog=tp, **kw)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [64, 200, 384])
def test_softcap_small(pa, orc, tp, S, causal, fmt):
    softcap_case(pa, orc, tp, 1, 2, 2, S, causal, fmt, S * 3 + 1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [True, False])
def test_softcap_grouped_query(pa, orc, tp, causal, fmt):
    softcap_case(pa, orc, tp, 2, 4, 2, 300, causal, fmt, 61)


@pytest.mark.parametrize("fmt", FMTS)
def test_softcap_large_logits(pa, orc, tp, fmt):
    """Scores past the clamp: the differentiated program is 0 there (the
    clamped forward program is constant)."""
    softcap_case(pa, orc, tp, 1, 1, 1, 256, True, fmt, 62, sd=40.0)


@pytest.mark.parametrize("core", ["d1", "pwl2", "d2", "d3"])
@pytest.mark.parametrize("S,causal,cap", [(200, True, 50.0), (300, False, 100.0)])
def test_softcap_exp2_cores(pa, orc, tp, core, S, causal, cap):
    """P recomputed through the forward's software exp2 core (Appendix B.1)."""
    softcap_case(pa, orc, tp, 1, 4, 2, S, causal, "bf16", 64 + S, core=core, cap=cap,
                 sd=3.0 if cap > 50 else 1.0)


def test_softcap_full_size_sampled(pa, orc, tp):
    """B=1 H=16 S=8192 D=128 causal, the benchmark's launch.  Heads are
    independent, so the oracle's forward supplies O and lse for every row of
    two heads only (the others get lse = 1e4, i.e. P = 0); 40 query rows and
    40 key rows of those heads are recomputed."""
    B, H, S = 1, 16, 8192
    heads = (0, 11)
    note("softcap bwd full size draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S)
    dot = si.t_attn_grad(B, H, S)
    q, k, v, do = to_bits(qt), to_bits(kt), to_bits(vt), to_bits(dot)
    rng = np.random.default_rng(63)
    qrows = np.unique(np.concatenate([[h * S, h * S + 1, h * S + S - 1, h * S + 5000] for h in heads]
                                     + [heads[1] * S + rng.integers(0, S, 32)]))
    krows = np.unique(np.concatenate([[h * S, h * S + S - 1, h * S + S - 2, h * S + 77] for h in heads]
                                     + [heads[0] * S + rng.integers(0, S, 32)]))
    for fmt in FMTS:
        call, kind, kw = softcap_variant(pa, orc, fmt)
        o = np.zeros((B, H, S, 128), np.uint16)
        lse = np.full((B, H, S), 1e4, np.float32)
        for h in heads:
            note(f"softcap bwd full size fmt={fmt}: oracle forward of head {h}")
            sl = slice(h, h + 1)
            o[:, sl], lse[:, sl] = fwd_for_bwd(orc, kind, q[:, sl], k[:, sl], v[:, sl], True,
                                               tanh_prog=tp, **kw)
        note(f"softcap bwd full size fmt={fmt}: kernel")
        dq, dk, dv = call(qt, kt, vt, to_dev(o, BF), dot, torch.from_numpy(lse).cuda(), 50.0, True)
        dq, dk, dv = to_bits(dq), to_bits(dk), to_bits(dv)
        compare(orc, kind, q, k, v, o, do, lse, dq, dk, dv, qrows, krows, True,
                f"softcap bwd full fmt={fmt}", cap=50.0, tanh_prog=tp, **kw)


def test_softcap_b2_geometry_sampled(pa, orc, tp):
    """The pages' B2 geometry, 1 x 32 query heads on 8 key/value heads x
    4096 x 128, causal, BF16 program: the grouped dK/dV kernel with FP32
    partials and their sum, and the dQ pass over stored dS blocks.  Query
    heads 1 and 13 get the oracle's O and lse (the others lse = 1e4, P = 0,
    in the kernel and the oracle alike); sampled query rows of both and key
    rows of their key/value heads 0 and 3."""
    B, H, Hkv, S = 1, 32, 8, 4096
    heads = (1, 13)
    note("softcap bwd B2 geometry draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    dot = si.t_attn_grad(B, H, S)
    q, k, v, do = to_bits(qt), to_bits(kt), to_bits(vt), to_bits(dot)
    rng = np.random.default_rng(65)
    qrows = np.unique(np.concatenate([[h * S, h * S + S - 1] for h in heads] + [heads[1] * S + rng.integers(0, S, 24)]))
    krows = np.unique(np.concatenate([[g * S, g * S + S - 1] for g in (0, 3)] + [3 * S + rng.integers(0, S, 24)]))
    call, kind, kw = softcap_variant(pa, orc, "bf16")
    o = np.zeros((B, H, S, 128), np.uint16)
    lse = np.full((B, H, S), 1e4, np.float32)
    for h in heads:
        note(f"softcap bwd B2 geometry: oracle forward of head {h}")
        g = h // (H // Hkv)
        o[:, h:h + 1], lse[:, h:h + 1] = fwd_for_bwd(orc, kind, q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1],
                                                     True, tanh_prog=tp, **kw)
    note("softcap bwd B2 geometry: kernel")
    dq, dk, dv = call(qt, kt, vt, to_dev(o, BF), dot, torch.from_numpy(lse).cuda(), 50.0, True)
    dq, dk, dv = to_bits(dq), to_bits(dk), to_bits(dv)
    compare(orc, kind, q, k, v, o, do, lse, dq, dk, dv, qrows, krows, True, "softcap bwd B2 geometry",
            cap=50.0, tanh_prog=tp, **kw)


def sigmoid_case(pa, orc, sp, B, H, Hkv, S, causal, poly, seed, qrows=None, krows=None):
    q, k, v, do = draw(B, H, Hkv, S, seed)
    kind = orc.ATTN_SIGMOID_POLY if poly else orc.ATTN_SIGMOID_EXACT
    label = f"sigmoid bwd B={B} H={H} Hkv={Hkv} S={S} causal={causal} poly={poly}"
    note(label)
    entry = pa.poly_sigmoid_attn_bwd if poly else pa.native_sigmoid_attn_bwd
    dq, dk, dv = entry(to_dev(q, BF), to_dev(k, BF), to_dev(v, BF), to_dev(do, BF), causal)
    dq, dk, dv = to_bits(dq), to_bits(dk), to_bits(dv)
    qrows = np.arange(B * H * S) if qrows is None else qrows
    krows = np.arange(B * Hkv * S) if krows is None else krows
    compare(orc, kind, q, k, v, None, do, None, dq, dk, dv, qrows, krows, causal, label, sig=sp)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [64, 200, 384])
def test_sigmoid_native_small(pa, orc, sp, S, causal):
    sigmoid_case(pa, orc, sp, 2, 4, 2, S, causal, False, S + 71)


@pytest.mark.parametrize("causal", [True, False])
def test_sigmoid_poly_fitted_length(pa, orc, sp, causal):
    rng = np.random.default_rng(72)
    S = 4096
    qrows = np.unique(np.concatenate([[0, 127, 128, S - 1, S, 2 * S - 1], rng.integers(0, 2 * S, 40)]))
    krows = np.unique(np.concatenate([[0, 127, 128, S - 1], rng.integers(0, S, 40)]))
    sigmoid_case(pa, orc, sp, 1, 2, 1, S, causal, True, 73, qrows, krows)


def test_sigmoid_full_size_sampled(pa, orc, sp):
    """B=1, 32 query heads on 8 key/value heads, S = 4096, causal."""
    B, H, Hkv, S = 1, 32, 8, 4096
    note("sigmoid bwd full size draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    dot = si.t_attn_grad(B, H, S)
    q, k, v, do = to_bits(qt), to_bits(kt), to_bits(vt), to_bits(dot)
    rng = np.random.default_rng(74)
    qrows = np.unique(np.concatenate([[0, S - 1, H * S - 1], rng.integers(0, H * S, 30)]))
    krows = np.unique(np.concatenate([[0, S - 1, Hkv * S - 1], rng.integers(0, Hkv * S, 30)]))
    for poly in (True, False):
        kind = orc.ATTN_SIGMOID_POLY if poly else orc.ATTN_SIGMOID_EXACT
        note(f"sigmoid bwd full size poly={poly}")
        entry = pa.poly_sigmoid_attn_bwd if poly else pa.native_sigmoid_attn_bwd
        dq, dk, dv = entry(qt, kt, vt, dot, True)
        dq, dk, dv = to_bits(dq), to_bits(dk), to_bits(dv)
        compare(orc, kind, q, k, v, None, do, None, dq, dk, dv, qrows, krows, True,
                f"sigmoid bwd full poly={poly}", sig=sp)


@pytest.mark.parametrize("S", [1, 65, 129])
def test_edge_lengths_and_wide_groups(pa, orc, tp, sp, S):
    """Sequences shorter than, or one past, a tile; eight query heads on one
    key/value head (the summing pass over a group of eight)."""
    for causal in (True, False):
        for fmt in FMTS:
            softcap_case(pa, orc, tp, 1, 8, 1, S, causal, fmt, 95 + S)
        sigmoid_case(pa, orc, sp, 1, 8, 1, S, causal, False, 96 + S)


def test_workspace_must_be_contiguous(pa):
    import synth_inputs as si
    q, k, v = si.t_attn_inputs(1, 2, 64, 128)
    dout = si.t_attn_grad(1, 2, 64, 128)
    o, lse = pa.poly_softcap_attn_fwd(q, k, v, 50.0, True, with_lse=True)
    need = pa.attn_bwd_workspace(True, 1, 2, 2, 64, 128, device=q.device).numel()
    strided = torch.empty(2 * need, dtype=torch.float32, device=q.device)[::2]
    with pytest.raises(ValueError):
        pa.poly_softcap_attn_bwd(q, k, v, o, dout, lse, 50.0, True, workspace=strided)
