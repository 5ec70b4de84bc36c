"""Mutation tests: the parity comparison must detect a plausible mistake.

The mistakes are planted in the oracle, on the CPU, never in a kernel: each
program's GPU output over all 65,536 bit patterns of its format (and a fixed
seeded upstream gradient for the backward programs) is compared with an
oracle whose program has one coefficient moved by one unit in the last place
or whose clamp is moved by one unit of the format.  A mutant that changes no
output of the oracle itself is equivalent (the same function after rounding:
only clamp moves of the SiLU' program are) and is reported, not required;
every other mutant must change outputs against the GPU.  For BF16 the
rounding order is mutated too: a split multiply / add must be detected,
while the pages' single-rounding BF16 FMA reproduces the GPU output exactly
(the deployed FP32 FMA + BF16 rounding never double-rounds differently for
these programs).
"""
import ctypes as C

import numpy as np
import pytest
import torch

from gpu_util import note, programs, to_bits, to_dev

pytestmark = pytest.mark.gpu
ALL = np.arange(65536, dtype=np.uint16)
DT = {"f16": torch.float16, "bf16": torch.bfloat16}
ORDER = {"f16": 1, "bf16": 3}
FWD = {"sigmoid": "sigmoid_fwd_d3", "tanh": "tanh_fwd_d4", "silu": "silu_fwd_d3",
       "gelu": "gelu_fwd_d5"}
BWD = {"sigmoid": "sigmoid_bwd_d4", "tanh": "tanh_bwd_d4", "silu": "silu_bwd_d3",
       "gelu": "gelu_bwd_d5"}


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    assert torch.cuda.is_available()
    pa.lib()
    return pa


@pytest.fixture(scope="module")
def progs(orc):
    return programs(orc)


def clone(orc, p):
    q = orc.Prog()
    C.memmove(C.byref(q), C.byref(p), C.sizeof(orc.Prog))
    return q


def grads():
    return np.random.default_rng(77).integers(0, 65536, 65536).astype(np.uint16)


def gpu_out(pa, fmt, func, bwd):
    x = to_dev(ALL, DT[fmt])
    if bwd:
        return to_bits(pa.poly_act_bwd(x, to_dev(grads(), DT[fmt]), func))
    return to_bits(pa.poly_act_fwd(x, func))


def oracle_out(orc, p, order, bwd):
    return orc.act_bwd(p, ALL, grads(), order) if bwd else orc.act_fwd(p, ALL, order)


def mutants(orc, p, fmt):
    """(label, mutated program) pairs: every coefficient the chain reads +-1
    ULP of its BF16 value, and the clamp +-1 ULP of the format."""
    out = []
    c0_used = p.c[0] != 0
    for j in range(0 if c0_used else 1, p.degree + 1):
        for d in (1, -1):
            q = clone(orc, p)
            q.c[j] = (int(p.c[j]) + d) & 0xFFFF
            out.append((f"c{j}{d:+d}ulp", q))
    for d in (1, -1):
        q = clone(orc, p)
        if fmt == "f16":
            b = int(np.array([p.Lc], np.float16).view(np.uint16)[0]) + d
            q.Lc = float(np.array([b], np.uint16).view(np.float16)[0])
        else:
            b = (int(np.array([p.Lc], np.float32).view(np.uint32)[0]) >> 16) + d
            q.Lc = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        out.append((f"Lc{d:+d}ulp", q))
    return out


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("bwd", [False, True])
@pytest.mark.parametrize("func", ["sigmoid", "tanh", "silu", "gelu"])
def test_program_mutations_detected(pa, orc, progs, fmt, bwd, func):
    p = progs[(BWD if bwd else FWD)[func]]
    note(f"mutations {fmt} {'bwd' if bwd else 'fwd'} {func}")
    got = gpu_out(pa, fmt, func, bwd)
    assert np.array_equal(got, oracle_out(orc, p, ORDER[fmt], bwd)), "unmutated oracle must agree"
    base = oracle_out(orc, p, ORDER[fmt], bwd)
    missed, equivalent = [], []
    for label, q in mutants(orc, p, fmt):
        mo = oracle_out(orc, q, ORDER[fmt], bwd)
        n = int((mo != got).sum())
        note(f"  {label}: {n} differing outputs")
        if not (mo != base).any():
            equivalent.append(label)
        elif n == 0:
            missed.append(label)
    assert not missed, f"mutations the comparison would not see: {missed}"
    assert all(e.startswith("Lc") for e in equivalent), equivalent
    if equivalent:
        note(f"  equivalent mutants (no output changes): {equivalent}")


@pytest.mark.parametrize("bwd", [False, True])
@pytest.mark.parametrize("func", ["sigmoid", "tanh", "silu", "gelu"])
def test_bf16_rounding_orders(pa, orc, progs, bwd, func):
    """The GPU's BF16 output against two other rounding orders: a split
    multiply / add must differ; the pages' single-rounding BF16 FMA must not."""
    p = progs[(BWD if bwd else FWD)[func]]
    got = gpu_out(pa, "bf16", func, bwd)
    n_split = int((oracle_out(orc, p, orc.ORDER_BF16_SPLIT, bwd) != got).sum())
    n_fma = int((oracle_out(orc, p, orc.ORDER_BF16_FMA, bwd) != got).sum())
    note(f"bf16 {'bwd' if bwd else 'fwd'} {func}: split {n_split}, single-rounding FMA {n_fma} "
         "differing outputs")
    assert n_split > 0
    assert n_fma == 0
