"""CPU oracle for the polynomial activation programs (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does, and the
two share no code: the oracle fits its own coefficients (paper section 3.2,
Eqs. 7-8) and replays each program with correctly rounded operations written
from the definitions of FP16, BF16 and FP32 (``orc_fp.c``).

This module only marshals numpy arrays to the plain C library ``liborc.so``
built from ``orc_*.c`` by :func:`build`.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liborc.so")
SOURCES = ["orc_fp.c", "orc_fit.c", "orc_eval.c"]

SIGMOID, TANH, SILU, GELU = 1, 2, 3, 4
FUNC_NAMES = {SIGMOID: "sigmoid", TANH: "tanh", SILU: "silu", GELU: "gelu"}
ORDER_F16_FMA, ORDER_BF16_FMA, ORDER_F32FMA_BF16, ORDER_BF16_SPLIT = 1, 2, 3, 4


def build(verbose: bool = False) -> str:
    """Compile liborc.so with gcc (strict IEEE: no contraction, no fast-math)."""
    cmd = ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", LIB_PATH + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class Prog(C.Structure):
    _fields_ = [("func", C.c_int32), ("deriv", C.c_int32), ("degree", C.c_int32),
                ("reserved", C.c_int32), ("Li", C.c_double), ("Lc", C.c_double),
                ("c", C.c_uint16 * 8)]

    def coeff_bits(self):
        return [int(self.c[j]) for j in range(self.degree + 1)]

    def __repr__(self):
        return (f"Prog({FUNC_NAMES[self.func]}{'_bwd' if self.deriv else ''} "
                f"D{self.degree} Li={self.Li} Lc={self.Lc} "
                f"c={[hex(b) for b in self.coeff_bits()]})")


_lib = None


def lib():
    global _lib
    if _lib is None:
        srcs = [os.path.join(HERE, f) for f in SOURCES + ["orc.h"]]
        if not os.path.exists(LIB_PATH) or \
                max(os.path.getmtime(f) for f in srcs) > os.path.getmtime(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        u16, f64, i32, i64 = C.c_uint16, C.c_double, C.c_int32, C.c_int64
        P = C.POINTER
        sig = {
            "orc_f16_to_f64": (f64, [u16]), "orc_bf16_to_f64": (f64, [u16]),
            "orc_f64_to_f16": (u16, [f64]), "orc_f64_to_bf16": (u16, [f64]),
            "orc_f32_to_bf16": (u16, [C.c_float]),
            "orc_fma_f16": (u16, [u16, u16, u16]), "orc_fma_bf16": (u16, [u16, u16, u16]),
            "orc_fma_f32_bf16": (u16, [u16, u16, u16]),
            "orc_ref": (f64, [C.c_int, C.c_int, f64]),
            "orc_residual": (f64, [C.c_int, C.c_int, f64]),
            "orc_fit": (C.c_int, [C.c_int, C.c_int, C.c_int, f64, P(f64)]),
            "orc_make_prog": (C.c_int, [C.c_int, C.c_int, C.c_int, f64, f64, P(Prog)]),
            "orc_prog_real": (f64, [P(Prog), f64]),
            "orc_table2_metric": (f64, [P(Prog)]),
            "orc_search_objective": (f64, [P(Prog), C.c_int, P(C.c_int)]),
            "orc_search": (C.c_int, [C.c_int, C.c_int, C.c_int, f64, f64, C.c_int,
                                     P(Prog), P(f64), P(f64)]),
            "orc_prog_eval": (u16, [P(Prog), u16, C.c_int]),
            "orc_prog_bwd": (u16, [P(Prog), u16, u16, C.c_int]),
            "orc_act_fwd": (None, [P(Prog), C.c_int, C.c_void_p, C.c_void_p, i64]),
            "orc_act_bwd": (None, [P(Prog), C.c_int, C.c_void_p, C.c_void_p,
                                   C.c_void_p, i64]),
            "orc_swiglu_fwd": (None, [P(Prog), C.c_void_p, C.c_void_p, C.c_void_p,
                                      i64, i64, i64, i64, i64, i64]),
            "orc_swiglu_bwd": (None, [P(Prog), C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p, i64, i64, i64, i64,
                                      i64, i64, i64, i64]),
            "orc_softcap_attn_rows": (None, [P(Prog), C.c_int, C.c_void_p, C.c_void_p,
                                             C.c_void_p, i32, i32, i32, i32, C.c_float,
                                             i32, C.c_void_p, i64, C.c_void_p,
                                             C.c_void_p]),
            "orc_threads": (C.c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ---- thin wrappers ---------------------------------------------------------

def fit(func: int, deriv: int, degree: int, Li: float) -> np.ndarray:
    c = (C.c_double * 8)()
    rc = lib().orc_fit(func, deriv, degree, Li, c)
    if rc:
        raise RuntimeError(f"orc_fit failed: {rc}")
    return np.array(c[: degree + 1])


def make_prog(func: int, deriv: int, degree: int, Li: float, Lc: float) -> Prog:
    p = Prog()
    rc = lib().orc_make_prog(func, deriv, degree, Li, Lc, C.byref(p))
    if rc:
        raise RuntimeError(f"orc_make_prog failed: {rc}")
    return p


def table2_metric(p: Prog) -> float:
    return lib().orc_table2_metric(C.byref(p))


def search_objective(p: Prog, order: int = ORDER_F32FMA_BF16):
    ok = C.c_int(0)
    v = lib().orc_search_objective(C.byref(p), order, C.byref(ok))
    return v, bool(ok.value)


def search(func, deriv, degree, Lc_fixed=0.0, bound=0.0, order=ORDER_F32FMA_BF16):
    p = Prog()
    obj, met = C.c_double(), C.c_double()
    rc = lib().orc_search(func, deriv, degree, Lc_fixed, bound, order, C.byref(p),
                          C.byref(obj), C.byref(met))
    if rc:
        raise RuntimeError(f"orc_search failed: {rc}")
    return p, obj.value, met.value


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def act_fwd(p: Prog, x_bits, order: int) -> np.ndarray:
    x = _u16(x_bits)
    y = np.empty_like(x)
    lib().orc_act_fwd(C.byref(p), order, _ptr(x), _ptr(y), x.size)
    return y


def act_bwd(p: Prog, x_bits, g_bits, order: int) -> np.ndarray:
    x, g = _u16(x_bits), _u16(g_bits)
    assert x.shape == g.shape
    dx = np.empty_like(x)
    lib().orc_act_bwd(C.byref(p), order, _ptr(x), _ptr(g), _ptr(dx), x.size)
    return dx


def swiglu_fwd(sig: Prog, gate, up, row_begin=0, row_end=None):
    g, u = _u16(gate), _u16(up)
    rows, cols = g.shape
    row_end = rows if row_end is None else row_end
    h = np.zeros_like(g)
    lib().orc_swiglu_fwd(C.byref(sig), _ptr(g), _ptr(u), _ptr(h), row_begin, row_end,
                         cols, cols, cols, cols)
    return h


def swiglu_bwd(sig: Prog, gate, up, dh, row_begin=0, row_end=None):
    g, u, d = _u16(gate), _u16(up), _u16(dh)
    rows, cols = g.shape
    row_end = rows if row_end is None else row_end
    dg = np.zeros_like(g)
    du = np.zeros_like(g)
    lib().orc_swiglu_bwd(C.byref(sig), _ptr(g), _ptr(u), _ptr(d), _ptr(dg), _ptr(du),
                         row_begin, row_end, cols, cols, cols, cols, cols, cols)
    return dg, du


def softcap_attn_rows(tanh_prog: Prog, poly: bool, q, k, v, cap: float, causal: bool,
                      rows):
    """q, k, v: uint16 (BF16 bits) [B, H, S, D].  Returns (O, noise) as float64
    [len(rows), D] for the requested flat query rows (b*H + h)*S + i."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, S, D = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, D), dtype=np.float64)
    noise = np.zeros((rows.size, D), dtype=np.float64)
    lib().orc_softcap_attn_rows(C.byref(tanh_prog), int(poly), _ptr(q), _ptr(k), _ptr(v),
                                B, H, S, D, cap, int(causal), _ptr(rows), rows.size,
                                _ptr(out), _ptr(noise))
    return out, noise


def threads() -> int:
    return lib().orc_threads()
