"""Host-side checks of bench.py's contract (no GPU).

- More than one GPU is refused with a message and exit status 2, before any
  GPU work.
- The committed HBM-traffic profile belongs to the committed streaming
  kernels (same source digest) and equals the algorithmic bytes of each
  program at 268,435,456 elements (4 bytes per element forward, 6 backward)
  to 0.01 %; bench.py reports it only when the digest matches.
- The CPU-baseline leg (the oracle on a bounded sample) returns the fields
  the bench line carries.
"""
import json
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_traffic_profile_matches_kernels():
    from elementwise_symmetry_range_amd._build import source_digest
    import bench
    tr = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert tr["source_digest"] == source_digest(), "profile taken from other kernel sources"
    algorithmic = {f"{f}_fwd": 4 * bench.N_HBM for f in bench.FWD}
    algorithmic.update({f"{f}_bwd": 6 * bench.N_HBM for f in bench.BWD})
    assert set(tr["kernels"]) == set(algorithmic)
    for name, by in tr["kernels"].items():
        assert abs(by / algorithmic[name] - 1.0) < 1e-4, (name, by)


def test_cpu_baseline_fields():
    """The CPU leg's fields: all-core and one-core rates of the six programs
    (median of 5 after 1 warm-up), the oracle's SwiGLU and softcap-attention
    rates, each with its sample; small sizes here."""
    import bench
    import synth_inputs as si
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.integers(0, 65536, 1 << 16).astype(np.uint16).view(np.int16)).view(torch.float16)
    g = torch.from_numpy(rng.integers(0, 65536, 1 << 16).astype(np.uint16).view(np.int16)).view(torch.float16)
    bits = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    swi = tuple(bits(a) for a in si.swiglu_inputs(8, 256))
    q, k, v = (bits(a) for a in si.attn_inputs(1, 2, 64, 128))
    cb = bench.cpu_baseline(x, g, swi=swi, attn=(q, k, v), n=1 << 14, n1=1 << 12, attn_rows=8,
                            runs=5)
    assert {"value", "unit", "cores", "kind", "sample", "value_1core", "sample_1core",
            "timing", "swiglu", "softcap_attention"} <= set(cb)
    assert cb["value"] > 0 and cb["unit"] == "Gelem/s" and cb["kind"] == "oracle"
    assert cb["cores"] >= 1 and cb["value_1core"] > 0
    assert "median of 5" in cb["timing"]
    assert cb["swiglu"]["fwd_gelem_s"] > 0 and cb["swiglu"]["bwd_gelem_s"] > 0
    assert cb["softcap_attention"]["fwd_scores_s"] > 0
    import oracle
    assert oracle.threads() == cb["cores"]          # the one-core leg restores the thread count


def test_program_table_carries_printed_bounds():
    import bench
    t = bench.program_table()
    assert t["sigmoid_bwd_d4"]["meets_printed_bound"] is True       # reproduced exactly
    assert t["gelu_fwd_d5"]["meets_printed_bound"] is False         # unreachable (tested)
    assert t["tanh_bwd_d4"]["printed_bound"] is None
