"""bench.py end to end on the GPU, with the short timing protocol: the step,
every SwiGLU / attention component and the JSON line it prints (the default
run times the same calls, only longer).  Guards the benchmark's own calls
(argument shapes, workspace sizes) against drifting from the library's."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_quick_run_prints_its_line():
    print("[gpu] bench.py --protocol quick --no-cpu --steps 2 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--protocol", "quick",
                        "--no-cpu", "--steps", "2", "--warmup", "1"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["value"] > 0
    assert line["roofline"]["frac"] > 0
    comp = line["components"]
    for key in ("swiglu_dense_fwd", "swiglu_dense_bwd", "swiglu_routed_fwd", "swiglu_routed_bwd",
                "softcap_attn_fwd", "softcap_attn_fwd_f16", "softcap_attn_exp2_cores",
                "softcap_attn_bwd", "softcap_attn_bwd_f16", "sigmoid_attn_fwd", "sigmoid_attn_bwd",
                "rope_fused_4096x32x8x128"):
        assert key in comp, key
    assert set(comp["softcap_attn_exp2_cores"]) == {"d1", "pwl2", "d2", "d3"}
    assert comp["rope_fused_4096x32x8x128"]["table_ms"] > 0
    assert line["detail_cfg1"]["elements"] == 4_194_304 + 65_536
    assert line["programs"]["sigmoid_fwd_d3"]["Lc"] == 5.28125
