"""GPU parity of the attention forwards against the CPU oracle.

Softcap attention (Eq. 1; the D4 tanh program in BF16 as the pages run it,
or in packed FP16, or accurate tanhf; the softmax's exp2 by the hardware or
a software core) and sigmoid attention (Eq. 14; the two-region BF16 cubic at
the fitted length 4096, or accurate sigma), multi-head and grouped-query
layouts, causal or not, ragged sequence lengths, the fixed and the running
softmax reference.  The oracle replays the method's rounding steps from the
same BF16 inputs; the gate is one BF16 ulp plus the oracle's spread
(attn_util).  The log-sum-exp the softcap forward writes for the backward is
compared too: the kernel forms it in FP32 from the reference and the row sum
of up to S terms, so
    |lse - lse_ref| <= 2^-14 (1 + |lse_ref|)
(S 2^-24 relative for the sum at S = 8192, plus the FP32 rounding of the log
and of the reference).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from attn_util import check, sig_prog, tanh_prog
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


def check_lse(got, ref, label):
    err = np.abs(got.astype(np.float64) - ref)
    ratio = float(np.max(err / (2.0 ** -14 * (1 + np.abs(ref)))))
    print(f"[attn] {label} lse: max err/tol {ratio:.3f}", flush=True)
    assert ratio <= 1.0, label


def draw(B, H, Hkv, S, seed, sd=1.0):
    rng = np.random.default_rng(seed)
    q = si.to_bf16_bits(rng.standard_normal((B, H, S, 128)) * sd)
    k, v = (si.to_bf16_bits(rng.standard_normal((B, Hkv, S, 128)) * sd) for _ in range(2))
    return q, k, v


FMTS = ("bf16", "f16", "native")


def softcap_entry(pa, fmt, core=None):
    """(kernel call, oracle kind, oracle keywords) of a softcap variant."""
    if core is not None:
        cid = pa.EXP2_CORES[core]
        return ((lambda q, k, v, cap, causal: pa.poly_softcap_attn_fwd_exp2(
            q, k, v, cap, causal, core=core, with_lse=True)), 1, dict(tanh_fmt="bf16", exp2_core=cid))
    if fmt == "native":
        return ((lambda q, k, v, cap, causal: pa.native_softcap_attn_fwd(q, k, v, cap, causal,
                                                                         with_lse=True)), 2, {})
    return ((lambda q, k, v, cap, causal: pa.poly_softcap_attn_fwd(q, k, v, cap, causal,
                                                                   with_lse=True, fmt=fmt)),
            1, dict(tanh_fmt=fmt))


def softcap_case(pa, orc, tp, q, k, v, causal, fmt, rows=None, label="", cap=50.0, core=None):
    B, H, S, D = q.shape
    note(f"softcap fwd {label} B={B} H={H} Hkv={k.shape[1]} S={S} causal={causal} fmt={fmt} "
         f"core={core} cap={cap}")
    call, kind, kw = softcap_entry(pa, fmt, core)
    o, lse = call(to_dev(q, BF), to_dev(k, BF), to_dev(v, BF), cap, causal)
    o, lse = to_bits(o).reshape(-1, D), lse.cpu().numpy().ravel()
    if rows is None:
        rows = np.arange(B * H * S)
    ref, ref_lse, spread = orc.attn_fwd_rows(kind, q, k, v, rows, cap=cap, causal=causal,
                                             tanh_prog=tp, **kw)
    lab = f"{label} S={S} causal={causal} fmt={fmt} core={core} cap={cap}"
    check(o[rows], ref, spread, lab)
    check_lse(lse[rows], ref_lse, lab)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [64, 128, 200, 384])
def test_softcap_small(pa, orc, tp, S, causal, fmt):
    q, k, v = draw(1, 2, 2, S, S * 7 + 2)
    softcap_case(pa, orc, tp, q, k, v, causal, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("causal", [True, False])
def test_softcap_grouped_query(pa, orc, tp, causal, fmt):
    """Four query heads on two key/value heads, two batches, ragged S."""
    q, k, v = draw(2, 4, 2, 300, 41)
    softcap_case(pa, orc, tp, q, k, v, causal, fmt, label="gqa")


@pytest.mark.parametrize("fmt", FMTS)
def test_softcap_large_logits(pa, orc, tp, fmt):
    """Scores beyond the softcap's clamp (|x| > Lc) and saturated tails."""
    q, k, v = draw(2, 1, 1, 256, 43, sd=40.0)
    softcap_case(pa, orc, tp, q, k, v, True, fmt, label="large")


def test_softcap_one_hot_v_readback(pa, orc, tp):
    """V = identity rows (V[j][d] = [d == j]): O[i][j] is the probability P_ij
    itself, so the softmax inside the kernel is compared directly."""
    S = 128
    rng = np.random.default_rng(31)
    q, k = (si.to_bf16_bits(rng.standard_normal((1, 1, S, 128)) * 2) for _ in range(2))
    v = si.to_bf16_bits(np.eye(S, 128)[None, None])
    for fmt in FMTS:
        softcap_case(pa, orc, tp, q, k, v, True, fmt, label="one-hot")


def test_softcap_full_size_sampled(pa, orc, tp):
    """B=1 H=16 S=8192 D=128 causal, alpha = 50, the benchmark's launch; the
    oracle recomputes 48 sampled rows (first and last rows of heads, random)."""
    B, H, S = 1, 16, 8192
    note("softcap full size draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S)
    rng = np.random.default_rng(32)
    rows = np.unique(np.concatenate([[0, 1, 2, S - 1, 5 * S + 4095, H * S - 1],
                                     rng.integers(0, B * H * S, 42)]))
    q, k, v = to_bits(qt), to_bits(kt), to_bits(vt)
    for fmt in FMTS:
        note(f"softcap full size fmt={fmt}")
        call, kind, kw = softcap_entry(pa, fmt)
        o, lse = call(qt, kt, vt, 50.0, True)
        o, lse = to_bits(o).reshape(-1, 128), lse.cpu().numpy().ravel()
        ref, ref_lse, spread = orc.attn_fwd_rows(kind, q, k, v, rows, tanh_prog=tp, **kw)
        check(o[rows], ref, spread, f"full fmt={fmt}")
        check_lse(lse[rows], ref_lse, f"full fmt={fmt}")


def test_softcap_b2_geometry_sampled(pa, orc, tp):
    """The pages' B2 geometry: 1 x 32 query heads on 8 key/value heads x
    4096 x 128, causal, alpha = 50, BF16 program and comparator; 40 sampled
    rows (every key/value group's first and last rows, random)."""
    B, H, Hkv, S = 1, 32, 8, 4096
    note("softcap B2 geometry draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([np.arange(0, H, 4) * S, np.arange(3, H, 4) * S + S - 1,
                                     rng.integers(0, B * H * S, 24)]))
    q, k, v = to_bits(qt), to_bits(kt), to_bits(vt)
    for fmt in ("bf16", "native"):
        note(f"softcap B2 geometry fmt={fmt}")
        call, kind, kw = softcap_entry(pa, fmt)
        o, lse = call(qt, kt, vt, 50.0, True)
        o, lse = to_bits(o).reshape(-1, 128), lse.cpu().numpy().ravel()
        ref, ref_lse, spread = orc.attn_fwd_rows(kind, q, k, v, rows, tanh_prog=tp, **kw)
        check(o[rows], ref, spread, f"B2 geometry fmt={fmt}")
        check_lse(lse[rows], ref_lse, f"B2 geometry fmt={fmt}")


def sigmoid_case(pa, orc, sp, q, k, v, causal, poly, rows=None, label=""):
    B, H, S, D = q.shape
    note(f"sigmoid fwd {label} B={B} H={H} Hkv={k.shape[1]} S={S} causal={causal} poly={poly}")
    entry = pa.poly_sigmoid_attn_fwd if poly else pa.native_sigmoid_attn_fwd
    o = to_bits(entry(to_dev(q, BF), to_dev(k, BF), to_dev(v, BF), causal)).reshape(-1, D)
    if rows is None:
        rows = np.arange(B * H * S)
    kind = orc.ATTN_SIGMOID_POLY if poly else orc.ATTN_SIGMOID_EXACT
    ref, _, spread = orc.attn_fwd_rows(kind, q, k, v, rows, causal=causal, sig=sp)
    check(o[rows], ref, spread, f"sigmoid {label} S={S} causal={causal} poly={poly}")


def sample_rows(B, H, S, n, seed):
    rng = np.random.default_rng(seed)
    heads = np.arange(B * H) * S
    return np.unique(np.concatenate([heads, heads + S - 1, heads + 127, heads + 128,
                                     rng.integers(0, B * H * S, n)]))


@pytest.mark.parametrize("causal", [True, False])
def test_sigmoid_poly_fitted_length(pa, orc, sp, causal):
    """The program holds for S = 4096 only; two query heads on one key/value
    head, sampled rows."""
    q, k, v = draw(1, 2, 1, 4096, 51)
    sigmoid_case(pa, orc, sp, q, k, v, causal, True, rows=sample_rows(1, 2, 4096, 120, 52))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [64, 200, 384])
def test_sigmoid_native_small(pa, orc, sp, S, causal):
    q, k, v = draw(2, 4, 2, S, S + 53)
    sigmoid_case(pa, orc, sp, q, k, v, causal, False)


def test_sigmoid_length_guard(pa):
    q = torch.zeros((1, 1, 2048, 128), dtype=BF, device="cuda")
    with pytest.raises(pa.PolyActError):
        pa.poly_sigmoid_attn_fwd(q, q, q, True)


def test_sigmoid_full_size_sampled(pa, orc, sp):
    """B=1, 32 query heads on 8 key/value heads, S = 4096, causal: the
    sigmoid-attention geometry of the paper's B3 measurement."""
    B, H, Hkv, S = 1, 32, 8, 4096
    note("sigmoid full size draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S, Hkv=Hkv)
    q, k, v = to_bits(qt), to_bits(kt), to_bits(vt)
    rows = sample_rows(1, 1, B * H * S, 60, 54)
    for poly in (True, False):
        note(f"sigmoid full size poly={poly}")
        entry = pa.poly_sigmoid_attn_fwd if poly else pa.native_sigmoid_attn_fwd
        o = to_bits(entry(qt, kt, vt, True)).reshape(-1, 128)
        kind = orc.ATTN_SIGMOID_POLY if poly else orc.ATTN_SIGMOID_EXACT
        ref, _, spread = orc.attn_fwd_rows(kind, q, k, v, rows, sig=sp)
        check(o[rows], ref, spread, f"sigmoid full poly={poly}")


@pytest.mark.parametrize("core", ["hw", "d1", "pwl2", "d2", "d3"])
@pytest.mark.parametrize("S,causal,cap", [(200, True, 50.0), (384, False, 50.0), (300, True, 100.0)])
def test_softcap_exp2_cores(pa, orc, tp, core, S, causal, cap):
    """The softmax's exponentials by a software exp2 core, with the fixed
    reference (cap 50) and the running integer reference (cap 100, where
    cap log2 e > 80): the oracle forms the same weights 2^floor(z) p(z -
    floor(z)) with the core in target precision."""
    cid = pa.EXP2_CORES[core]
    q, k, v = draw(1, 4, 2, S, 81 + cid, sd=3.0 if cap > 50 else 1.0)
    softcap_case(pa, orc, tp, q, k, v, causal, "bf16", label="exp2", cap=cap, core=core)


def test_softcap_exp2_cores_full_size_sampled(pa, orc, tp):
    B, H, S = 1, 16, 8192
    note("softcap exp2 full size draw")
    qt, kt, vt = si.t_attn_inputs(B, H, S)
    q, k, v = to_bits(qt), to_bits(kt), to_bits(vt)
    rows = sample_rows(1, 1, B * H * S, 40, 82)
    for core in ("d1", "pwl2", "d2", "d3"):
        note(f"softcap exp2 full size core={core}")
        o = to_bits(pa.poly_softcap_attn_fwd_exp2(qt, kt, vt, 50.0, True, core=core)).reshape(-1, 128)
        ref, _, spread = orc.attn_fwd_rows(orc.ATTN_SOFTCAP_POLY, q, k, v, rows, tanh_prog=tp,
                                           exp2_core=pa.EXP2_CORES[core])
        check(o[rows], ref, spread, f"exp2 full {core}")


@pytest.mark.parametrize("S", [1, 65, 129])
def test_edge_lengths_and_wide_groups(pa, orc, tp, sp, S):
    """Sequences shorter than, or one past, a tile; eight query heads on one
    key/value head; causal and not."""
    q, k, v = draw(1, 8, 1, S, 90 + S)
    for causal in (True, False):
        for fmt in FMTS:
            softcap_case(pa, orc, tp, q, k, v, causal, fmt, label="edge")
        sigmoid_case(pa, orc, sp, q, k, v, causal, False, label="edge")


@pytest.mark.parametrize("fmt", FMTS)
def test_softcap_large_cap_running_max(pa, orc, tp, fmt):
    """cap = 100 (cap log2 e > 80): the logits' range no longer fits a fixed
    reference, so the kernel tracks an integer running reference (lazy
    rescale by exact powers of two) and evaluates 2^z as 2^floor(z)
    2^(z - floor(z))."""
    q, k, v = draw(1, 2, 1, 300, 97, sd=3.0)
    softcap_case(pa, orc, tp, q, k, v, True, fmt, label="cap=100", cap=100.0)
