"""poly_softcap_attn_bwd_static (no workspace, the library's device scratch)
against poly_softcap_attn_bwd (caller workspace), through the C ABI: the same
kernels on the same inputs, so the gradients must agree bit for bit.  Two
calls in a row, the second on a smaller grouped-head shape (the scratch keeps
the first call's contents), then a third equal-size call again; a shape
whose scratch would exceed the array is rejected on the host."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import note, to_bits, to_dev

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


def case(pa, B, H, Hkv, S, seed):
    rng = np.random.default_rng(seed)
    q = to_dev(si.to_bf16_bits(rng.standard_normal((B, H, S, 128))), BF)
    k, v = (to_dev(si.to_bf16_bits(rng.standard_normal((B, Hkv, S, 128))), BF) for _ in range(2))
    do = to_dev(si.to_bf16_bits(rng.standard_normal((B, H, S, 128))), BF)
    o, lse = pa.poly_softcap_attn_fwd(q, k, v, 50.0, True, with_lse=True)
    note(f"static scratch backward B={B} H={H} Hkv={Hkv} S={S}")
    ref = pa.poly_softcap_attn_bwd(q, k, v, o, do, lse, 50.0, True)
    outs = tuple(torch.full_like(t, float("nan")) for t in ref)
    got = pa.poly_softcap_attn_bwd_static(q, k, v, o, do, lse, 50.0, True, *outs)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gb, rb = to_bits(g), to_bits(r)
        assert np.array_equal(gb, rb), f"{name}: {(gb != rb).sum()} differing outputs"


def test_static_scratch_backward_matches_workspace_backward(pa):
    assert pa.lib().pa_attn_bwd_static_scratch_bytes() == 8 << 20
    case(pa, 1, 4, 4, 1000, 1)      # plain heads: Delta and -lse log2 e in the scratch
    case(pa, 1, 2, 1, 300, 2)       # smaller, grouped heads: FP32 partials too
    case(pa, 2, 3, 3, 129, 3)


def test_static_scratch_rejects_shapes_beyond_the_array(pa):
    B, H, Hkv, S = 1, 16, 4, 1024   # grouped: 2 * 16384 + 2 * 16384 * 128 floats > 2 Mi
    assert pa.lib().pa_attn_bwd_workspace_bytes(1, B, H, Hkv, S, 128) > \
        pa.lib().pa_attn_bwd_static_scratch_bytes()
    q = torch.zeros((B, H, S, 128), dtype=BF, device="cuda")
    k = torch.zeros((B, Hkv, S, 128), dtype=BF, device="cuda")
    lse = torch.zeros((B, H, S), dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PolyActError) as e:
        pa.poly_softcap_attn_bwd_static(q, k, k, q, q, lse, 50.0, True)
    assert e.value.status == 2
