"""CPU tests of the C-ABI library: it loads, exports every declared entry
point, reports the program table the oracle derives, and rejects bad
arguments on the host before touching the device (no GPU needed: every call
here returns before any HIP call)."""
import ctypes as C
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "polyact.h")


@pytest.fixture(scope="module")
def pa():
    import elementwise_symmetry_range_amd as pa
    pa.lib()
    return pa


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|pa_status\s|int32_t\s)\s*(\w+)\s*\(",
                                 src, flags=re.M)))


def test_exports_every_declared_symbol(pa):
    names = declared_functions()
    assert len(names) == 13, names
    L = pa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.pa_abi_version() == 1


def test_program_table_matches_oracle(pa, orc):
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "programs.json")))["programs"]
    names = {1: "sigmoid", 2: "tanh", 3: "silu", 4: "gelu"}
    for g in gold:
        for dt in ("f16", "bf16"):
            info = pa.program_info(names[g["func"]], g["deriv"], dt)
            assert info["coeff_bits"] == g["coeff_bits"], g["name"]
            assert (info["Li"], info["Lc"], info["degree"]) == (g["Li"], g["Lc"], g["degree"])
            assert info["order"] == (1 if dt == "f16" else 3)
        # and the oracle, fitting now, agrees
        p = orc.make_prog(g["func"], g["deriv"], g["degree"], g["Li"], g["Lc"])
        assert p.coeff_bits() == g["coeff_bits"]
    out = pa.PaProgram()
    assert pa.lib().poly_program_info(9, 0, 1, C.byref(out)) == 4   # no such function
    assert pa.lib().poly_program_info(1, 0, 5, C.byref(out)) == 3   # no such dtype


FAKE = 0x10000  # never dereferenced: validation fails (or n == 0) first


def test_error_paths_unary(pa):
    L = pa.lib()
    assert L.poly_act_fwd(1, 1, None, FAKE, 8, None) == 1            # NULL
    assert L.poly_act_fwd(1, 1, FAKE, FAKE + 2, -1, None) == 2       # negative n
    assert L.poly_act_fwd(1, 7, FAKE, FAKE, 8, None) == 3            # dtype
    assert L.poly_act_fwd(9, 1, FAKE, FAKE + 64, 8, None) == 4       # func
    assert L.poly_act_fwd(1, 1, FAKE, FAKE + 2, 8, None) == 5        # partial overlap
    assert L.poly_act_fwd(1, 1, FAKE + 1, FAKE + 64, 8, None) == 7   # odd address
    assert L.poly_act_fwd(1, 1, FAKE, FAKE, 0, None) == 0            # n = 0: no launch
    assert L.poly_act_fwd(1, 2, FAKE, FAKE + 64, 0, None) == 0
    assert L.poly_act_bwd(5, 1, FAKE, FAKE + 64, FAKE + 128, 8, None) == 4   # no such function
    assert L.native_act_bwd(2, 3, 1, FAKE, FAKE + 64, FAKE + 128, 8, None) == 4  # SiLU' from y
    assert L.poly_act_bwd(1, 1, FAKE, FAKE + 64, FAKE + 66, 8, None) == 5    # dx over dy
    assert L.native_act_bwd(5, 1, 1, FAKE, FAKE + 64, FAKE + 128, 8, None) == 4
    assert L.native_act_fwd(0, 1, FAKE, FAKE + 64, 8, None) == 4
    assert L.pa_status_str(5) == b"output partially overlaps another buffer"


def test_error_paths_swiglu(pa):
    L = pa.lib()
    f = L.poly_swiglu_fwd
    assert f(1, FAKE, FAKE, FAKE, 4, 8, 8, 8, 8, None, 0, None) == 3          # FP16 unsupported
    assert f(2, FAKE, FAKE + 1024, FAKE + 4096, 4, 8, 4, 8, 8, None, 0, None) == 2   # ld < cols
    assert f(2, None, FAKE, FAKE, 4, 8, 8, 8, 8, None, 0, None) == 1
    assert f(2, FAKE, FAKE + 1024, FAKE + 2, 4, 8, 8, 8, 8, None, 0, None) == 5  # h over gate
    assert f(2, FAKE, FAKE + 1024, FAKE + 4096, 0, 8, 8, 8, 8, None, 0, None) == 0  # rows = 0
    assert f(2, FAKE, FAKE + 1024, FAKE + 4096, 4, 8, 8, 8, 8, FAKE + 3, 2, None) == 7  # offsets
    b = L.poly_swiglu_bwd
    # dgate and dup overlapping each other
    assert b(2, FAKE, FAKE + 1024, FAKE + 2048, FAKE + 4096, FAKE + 4100, 4, 8, 8, 8, 8, 8, 8,
             None, 0, None) == 5
    assert b(2, FAKE, FAKE + 1024, FAKE + 2048, FAKE + 4096, FAKE + 8192, 0, 8, 8, 8, 8, 8, 8,
             None, 0, None) == 0


def test_error_paths_attention(pa):
    L = pa.lib()
    a = L.poly_softcap_attn_fwd
    big = 1 << 30
    assert a(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 2, 64, 64, 50.0, 1, None) == 2
    assert a(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 2, 64, 128, -1.0, 1, None) == 2
    assert a(FAKE + 2, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 1, 2, 64, 128, 50.0, 1, None) == 7
    assert a(FAKE, FAKE + big, FAKE + 2 * big, FAKE, 1, 2, 64, 128, 50.0, 1, None) == 5
    assert a(None, FAKE, FAKE, FAKE, 1, 2, 64, 128, 50.0, 1, None) == 1
    assert a(FAKE, FAKE + big, FAKE + 2 * big, FAKE + 3 * big, 0, 2, 64, 128, 50.0, 1, None) == 0
