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
SOURCES = ["orc_fp.c", "orc_fit.c", "orc_eval.c", "orc_exp2.c", "orc_rope.c"]

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


class SigProg(C.Structure):
    """Two-region sigmoid-attention program (BF16 bit patterns)."""
    _fields_ = [("n", C.c_int32), ("thr", C.c_uint16), ("lo", C.c_uint16),
                ("hi", C.c_uint16), ("c", (C.c_uint16 * 4) * 2), ("a", C.c_uint16 * 2),
                ("b", C.c_uint16 * 2)]


class Attn(C.Structure):
    _fields_ = [("kind", C.c_int32), ("B", C.c_int32), ("H", C.c_int32), ("Hkv", C.c_int32),
                ("S", C.c_int32), ("D", C.c_int32), ("causal", C.c_int32),
                ("order", C.c_int32), ("exp2_core", C.c_int32), ("cap", C.c_float),
                ("tanh_prog", C.POINTER(Prog)),
                ("sig", C.POINTER(SigProg)), ("tanh_order", C.c_int32), ("replay", C.c_int32)]


class RopeProg(C.Structure):
    """Paired sine / cosine program of the rotary embedding (BF16 bit patterns):
    sin(pi u) ~ u (a1 + a3 u^2 + a5 u^4), cos(pi u) ~ b0 + b2 u^2 + b4 u^4 + b6 u^6."""
    _fields_ = [("sin_c", C.c_uint16 * 3), ("cos_c", C.c_uint16 * 4)]


ATTN_SOFTCAP_POLY, ATTN_SOFTCAP_EXACT, ATTN_SIGMOID_POLY, ATTN_SIGMOID_EXACT = 1, 2, 3, 4
EXP2_EXACT, EXP2_D1, EXP2_PWL2, EXP2_D2, EXP2_D3 = 0, 1, 2, 3, 4

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
            "orc_attn_fwd_rows": (C.c_int, [P(Attn), C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_void_p, i64, C.c_void_p, C.c_void_p,
                                            C.c_void_p]),
            "orc_attn_bwd_rows": (C.c_int, [P(Attn)] + [C.c_void_p] * 7 + [i64, C.c_void_p, i64]
                                  + [C.c_void_p] * 6),
            "orc_dtanh_prog_f16": (u16, [P(Prog), u16]),
            "orc_dtanh_prog": (u16, [P(Prog), u16, C.c_int]),
            "orc_exp2_core": (f64, [C.c_int, f64, f64]),
            "orc_exp2_errors": (None, [C.c_int, f64, P(f64), P(f64)]),
            "orc_exp2_fit": (f64, [C.c_int, C.c_int]),
            "orc_exp2_core_target": (C.c_float, [C.c_int, C.c_float]),
            "orc_sig_prog_eval": (u16, [P(SigProg), u16, C.c_int, P(u16)]),
            "orc_lsq": (C.c_int, [C.c_int, C.c_int, P(f64), P(f64), P(f64)]),
            "orc_rope_fit": (C.c_int, [P(f64), P(f64)]),
            "orc_rope_prog": (C.c_int, [P(RopeProg)]),
            "orc_rope_inc": (None, [C.c_int, f64, P(C.c_uint32)]),
            "orc_rope_coord": (u16, [C.c_uint32]),
            "orc_rope_sincos": (None, [P(RopeProg), C.c_uint32, P(u16), P(u16)]),
            "orc_rope_rotate": (None, [u16, u16, u16, u16, P(u16), P(u16)]),
            "orc_rope_rows": (None, [P(RopeProg), P(C.c_uint32), C.c_int, C.c_void_p, C.c_void_p,
                                     i64, C.c_void_p]),
            "orc_threads": (C.c_int, []),
            "orc_set_threads": (C.c_int, [C.c_int]),
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


def sig_prog_from_golden(d: dict) -> SigProg:
    """SigProg from the golden description (hex strings of BF16 bit patterns)."""
    sp = SigProg()
    sp.n = int(d["n"])
    sp.thr, sp.lo, sp.hi = (int(d[k], 16) for k in ("threshold", "clamp_lo", "clamp_hi"))
    for r, name in enumerate(("region_lo", "region_hi")):
        reg = d[name]
        for j in range(4):
            sp.c[r][j] = int(reg[f"c{j}"], 16)
        sp.a[r] = int(reg["a"], 16)
        sp.b[r] = int(reg["b"], 16)
    return sp


TANH_ORDERS = {"bf16": ORDER_F32FMA_BF16, "f16": ORDER_F16_FMA}


def _attn(kind, q, k, cap, causal, tanh_prog, sig, order, exp2_core=0, tanh_fmt="bf16",
          replay=True):
    B, H, S, D = q.shape
    a = Attn()
    a.kind, a.B, a.H, a.Hkv, a.S, a.D = kind, B, H, k.shape[1], S, D
    a.causal, a.order, a.cap, a.exp2_core = int(causal), order, cap, exp2_core
    a.tanh_order = TANH_ORDERS[tanh_fmt]
    a.replay = int(bool(replay))
    a._keep = (tanh_prog, sig)
    if tanh_prog is not None:
        a.tanh_prog = C.pointer(tanh_prog)
    if sig is not None:
        a.sig = C.pointer(sig)
    return a


def attn_fwd_rows(kind: int, q, k, v, rows, cap: float = 50.0, causal: bool = True,
                  tanh_prog: Prog = None, sig: SigProg = None, order: int = 0,
                  exp2_core: int = 0, tanh_fmt: str = "bf16", replay: bool = True):
    """q: uint16 BF16 bits [B, H, S, D]; k, v: [B, Hkv, S, D].  Returns (O, lse,
    spread) in float64 for the flat query rows (b H + h) S + i: O and spread
    [len(rows), D], lse [len(rows)] (NaN for sigmoid attention).  exp2_core
    (softcap poly only): the softmax's exponentials by that fractional core.
    tanh_fmt: format of the softcap program ("bf16", the pages' path, or
    "f16").  replay: the method's FP32 steps and BF16 rounding of P (True) or
    real arithmetic around the programs (False).  spread: per output, the
    largest change that admissible alternatives of the replay's rounding
    decisions can cause (0 without replay)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    D = q.shape[3]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, D))
    lse = np.zeros(rows.size)
    spread = np.zeros((rows.size, D))
    a = _attn(kind, q, k, cap, causal, tanh_prog, sig, order, exp2_core, tanh_fmt, replay)
    rc = lib().orc_attn_fwd_rows(C.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(rows), rows.size,
                                 _ptr(out), _ptr(lse), _ptr(spread))
    if rc:
        raise ValueError(f"orc_attn_fwd_rows: {rc}")
    return out, lse, spread


def attn_bwd_rows(kind: int, q, k, v, o, dout, lse, qrows, krows, cap: float = 50.0,
                  causal: bool = True, tanh_prog: Prog = None, sig: SigProg = None,
                  order: int = 0, exp2_core: int = 0, tanh_fmt: str = "bf16",
                  replay: bool = True):
    """Gradients of sum(O * dout) for the flat query rows (dQ) and key rows
    (b Hkv + hk) S + j (dK, dV).  o: float64 [B, H, S, D] (the forward output
    the backward is given), lse: float64 [B, H, S] (softcap only).  Returns
    (dq, dk, dv, sp_dq, sp_dk, sp_dv), float64 [rows, D] each: the gradients
    and their spreads (as attn_fwd_rows).  tanh_fmt, replay, exp2_core: as
    attn_fwd_rows."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    D = q.shape[3]
    o = np.ascontiguousarray(o, dtype=np.float64)
    lse = np.ascontiguousarray(np.zeros(1) if lse is None else lse, dtype=np.float64)
    qrows = np.ascontiguousarray(qrows, dtype=np.int64)
    krows = np.ascontiguousarray(krows, dtype=np.int64)
    res = [np.zeros((n, D)) for n in (qrows.size, krows.size, krows.size) * 2]
    a = _attn(kind, q, k, cap, causal, tanh_prog, sig, order, exp2_core, tanh_fmt, replay)
    rc = lib().orc_attn_bwd_rows(C.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                 _ptr(lse), _ptr(qrows), qrows.size, _ptr(krows), krows.size,
                                 *[_ptr(r) for r in res])
    if rc:
        raise ValueError(f"orc_attn_bwd_rows: {rc}")
    return tuple(res)


def exp2_errors(core: int, a: float = 0.0):
    mx, rms = C.c_double(), C.c_double()
    lib().orc_exp2_errors(core, a, C.byref(mx), C.byref(rms))
    return mx.value, rms.value


def exp2_fit(core: int, minimax: bool) -> float:
    return lib().orc_exp2_fit(core, int(minimax))


def exp2_core_target(core: int, f) -> np.ndarray:
    return np.array([lib().orc_exp2_core_target(core, float(x)) for x in np.atleast_1d(f)],
                    dtype=np.float32)


def dtanh_prog(tanh_prog: Prog, x_bits, tanh_fmt: str = "bf16") -> np.ndarray:
    """The analytic derivative of the tanh program at x (bits of tanh_fmt)."""
    x = np.atleast_1d(np.asarray(x_bits, dtype=np.uint16))
    order = TANH_ORDERS[tanh_fmt]
    return np.array([lib().orc_dtanh_prog(C.byref(tanh_prog), int(b), order) for b in x],
                    dtype=np.uint16)


def dtanh_prog_f16(tanh_prog: Prog, x_bits) -> np.ndarray:
    return dtanh_prog(tanh_prog, x_bits, "f16")


def sig_prog_eval(sp: SigProg, x_bits, order: int = ORDER_F32FMA_BF16):
    """(P~, surrogate derivative) BF16 bit arrays at BF16 inputs x."""
    x = np.atleast_1d(np.asarray(x_bits, dtype=np.uint16))
    p = np.zeros(x.size, np.uint16)
    g = np.zeros(x.size, np.uint16)
    gb = C.c_uint16()
    for i, b in enumerate(x):
        p[i] = lib().orc_sig_prog_eval(C.byref(sp), int(b), order, C.byref(gb))
        g[i] = gb.value
    return p, g


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> int:
    """Threads of the oracle's later parallel loops; returns the previous count."""
    return lib().orc_set_threads(int(n))


# ---- rotary embedding (Appendix B.2) ---------------------------------------

def lsq(A, r) -> np.ndarray:
    """Least squares by the oracle's Householder QR (A: N x m, column-major copy)."""
    A = np.asarray(A, dtype=np.float64)
    N, m = A.shape
    a = np.ascontiguousarray(A.T).ravel().copy()
    rr = np.asarray(r, dtype=np.float64).copy()
    x = np.zeros(m)
    rc = lib().orc_lsq(N, m, a.ctypes.data_as(C.POINTER(C.c_double)),
                       rr.ctypes.data_as(C.POINTER(C.c_double)), x.ctypes.data_as(C.POINTER(C.c_double)))
    assert rc == 0
    return x


def rope_fit():
    """FP64 (a1, a3, a5), (b0, b2, b4, b6) before rounding."""
    s, c = (C.c_double * 3)(), (C.c_double * 4)()
    assert lib().orc_rope_fit(s, c) == 0
    return np.array(list(s)), np.array(list(c))


def rope_prog() -> RopeProg:
    rp = RopeProg()
    assert lib().orc_rope_prog(C.byref(rp)) == 0
    return rp


def rope_inc(D: int, base: float = 10000.0) -> np.ndarray:
    out = (C.c_uint32 * (D // 2))()
    lib().orc_rope_inc(D, base, out)
    return np.array(list(out), dtype=np.uint32)


def rope_coord(phase) -> np.ndarray:
    return np.array([lib().orc_rope_coord(int(p)) for p in np.atleast_1d(phase)], dtype=np.uint16)


def rope_sincos(rp: RopeProg, phase):
    """(sin bits, cos bits) of the programs at each Q0.32 phase."""
    ph = np.atleast_1d(np.asarray(phase, dtype=np.uint64))
    s, c = np.empty(ph.size, np.uint16), np.empty(ph.size, np.uint16)
    a, b = C.c_uint16(), C.c_uint16()
    for j, p in enumerate(ph):
        lib().orc_rope_sincos(C.byref(rp), int(p), C.byref(a), C.byref(b))
        s[j], c[j] = a.value, b.value
    return s, c


def rope_rotate(x0, x1, s, c):
    a, b = C.c_uint16(), C.c_uint16()
    lib().orc_rope_rotate(int(x0), int(x1), int(s), int(c), C.byref(a), C.byref(b))
    return a.value, b.value


def rope_rows(rp: RopeProg, inc, x_bits, pos) -> np.ndarray:
    """Rotary embedding of rows x [n, D] (FP16 bits) at positions pos [n]."""
    x = _u16(x_bits)
    n, D = x.shape
    inc = np.ascontiguousarray(inc, dtype=np.uint32)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    assert pos.size == n and inc.size == D // 2
    y = np.empty_like(x)
    lib().orc_rope_rows(C.byref(rp), inc.ctypes.data_as(C.POINTER(C.c_uint32)), D, _ptr(x),
                        _ptr(pos), n, _ptr(y))
    return y
