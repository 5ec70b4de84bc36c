"""Helpers shared by the GPU parity tests (host <-> device bit moves, oracle
programs from the golden table)."""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden", "programs.json")
FUNC_ID = {"sigmoid": 1, "tanh": 2, "silu": 3, "gelu": 4}


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(dev()).view(dtype)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def programs(orc):
    out = {}
    for g in json.load(open(GOLD))["programs"]:
        out[g["name"]] = orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])
    return out


def fwd_prog_name(func):
    return {"sigmoid": "sigmoid_fwd_d3", "tanh": "tanh_fwd_d4", "silu": "silu_fwd_d3",
            "gelu": "gelu_fwd_d5"}[func]


def bwd_prog_name(func):
    return {"sigmoid": "sigmoid_bwd_d4", "tanh": "tanh_bwd_d4", "silu": "silu_bwd_d3",
            "gelu": "gelu_bwd_d5"}[func]


def diff_report(got, ref, x=None, limit=5):
    bad = np.nonzero(got != ref)[0]
    msg = f"{bad.size} differing of {got.size}"
    for i in bad[:limit]:
        msg += f"\n  i={i} got={got[i]:#06x} ref={ref[i]:#06x}"
        if x is not None:
            msg += f" x={x[i]:#06x}"
    return msg
