"""Python binding of libpolyact.so, the gfx950 polynomial activation library.

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/polyact.h.  Tensors supply device memory and the
current stream; there is no fallback path -- if the library is not built, or a
call fails, an exception is raised.

Programs ("Fast Polynomial Transcendentals for LLMs", arXiv 2610.00049):
sigmoid D3, tanh D4, SiLU D3 and GELU D5 forward; sigmoid' D4 and tanh' D4
direct derivative fits for backward; the D3 sigmoid fused into SwiGLU forward
and backward; the D4 tanh as an attention softcap (forward) and its analytic
derivative (backward); the two-region sigmoid-attention cubic and its
factored derivative surrogate.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from ._build import LIB as LIB_PATH

__all__ = [
    "PolyActError", "lib", "program_info", "poly_act_fwd", "poly_act_bwd", "native_act_fwd",
    "native_act_bwd", "poly_swiglu_fwd", "poly_swiglu_bwd", "native_swiglu_fwd",
    "native_swiglu_bwd", "poly_softcap_attn_fwd", "native_softcap_attn_fwd",
    "poly_softcap_attn_fwd_exp2", "poly_softcap_attn_bwd", "native_softcap_attn_bwd",
    "poly_sigmoid_attn_fwd",
    "native_sigmoid_attn_fwd", "poly_sigmoid_attn_bwd", "native_sigmoid_attn_bwd",
    "sigmoid_attn_program", "attn_bwd_workspace", "attn_bwd_ds_limit", "stream_copy", "FUNCS",
    "poly_rope",
    "native_rope", "native_rope_table", "rope_table", "rope_program",
]

FUNCS = {"sigmoid": 1, "tanh": 2, "silu": 3, "gelu": 4}
IMPLS = {"poly": 0, "native": 1, "native_from_y": 2}
_DTYPES = {torch.float16: 1, torch.bfloat16: 2}
DTYPE_CODES = {"f16": 1, "bf16": 2}


class PaProgram(C.Structure):
    _fields_ = [("func", C.c_int32), ("deriv", C.c_int32), ("degree", C.c_int32),
                ("dtype", C.c_int32), ("Li", C.c_float), ("Lc", C.c_float),
                ("coeff_bits", C.c_uint16 * 8), ("order", C.c_int32)]


class PaSigmoidAttnProgram(C.Structure):
    _fields_ = [("n", C.c_int32), ("thr", C.c_uint16), ("clamp_lo", C.c_uint16),
                ("clamp_hi", C.c_uint16), ("coeff_bits", (C.c_uint16 * 4) * 2),
                ("a_bits", C.c_uint16 * 2), ("b_bits", C.c_uint16 * 2), ("order", C.c_int32)]


class PaRopeProgram(C.Structure):
    _fields_ = [("sin_bits", C.c_uint16 * 3), ("cos_bits", C.c_uint16 * 4)]


class PolyActError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"polyact status {status}: {message}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        sigs = {
            "poly_act_fwd": [i32, i32, p, p, i64, p],
            "poly_act_bwd": [i32, i32, p, p, p, i64, p],
            "native_act_fwd": [i32, i32, p, p, i64, p],
            "native_act_bwd": [i32, i32, i32, p, p, p, i64, p],
            "poly_swiglu_fwd": [i32, p, p, p, i64, i64, i64, i64, i64, p, i32, p],
            "native_swiglu_fwd": [i32, p, p, p, i64, i64, i64, i64, i64, p, i32, p],
            "poly_swiglu_bwd": [i32, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, i32, p],
            "native_swiglu_bwd": [i32, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, i32,
                                  p],
            "poly_softcap_attn_fwd": [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, p],
            "native_softcap_attn_fwd": [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, p],
            "poly_softcap_attn_fwd_f16": [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, p],
            "poly_softcap_attn_fwd_exp2": [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p],
            "poly_softcap_attn_bwd": [p] * 10 + [i32] * 5 + [f32, i32, p],
            "poly_softcap_attn_bwd_f16": [p] * 10 + [i32] * 5 + [f32, i32, p],
            "poly_softcap_attn_bwd_exp2": [p] * 10 + [i32] * 5 + [f32, i32, i32, p],
            "poly_softcap_attn_bwd_static": [p] * 9 + [i32] * 5 + [f32, i32, p],
            "native_softcap_attn_bwd": [p] * 10 + [i32] * 5 + [f32, i32, p],
            "poly_sigmoid_attn_fwd": [p] * 4 + [i32] * 6 + [p],
            "native_sigmoid_attn_fwd": [p] * 4 + [i32] * 6 + [p],
            "poly_sigmoid_attn_bwd": [p] * 8 + [i32] * 6 + [p],
            "native_sigmoid_attn_bwd": [p] * 8 + [i32] * 6 + [p],
            "poly_sigmoid_attn_program": [C.POINTER(PaSigmoidAttnProgram)],
            "poly_program_info": [i32, i32, i32, C.POINTER(PaProgram)],
            "pa_stream_copy": [p, p, p, i64, p],
            "poly_rope": [p] * 4 + [i32] * 5 + [C.c_double, p],
            "native_rope": [p] * 4 + [i32] * 5 + [C.c_double, p],
            "native_rope_table": [p] * 5 + [i32] * 5 + [p],
            "pa_rope_table": [p, i32, i32, C.c_double, p],
            "poly_rope_program": [C.POINTER(PaRopeProgram)],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_int
        L.pa_status_str.argtypes = [C.c_int]
        L.pa_status_str.restype = C.c_char_p
        L.pa_attn_bwd_workspace_bytes.argtypes = [i32] * 6
        L.pa_attn_bwd_workspace_bytes.restype = C.c_int64
        L.pa_attn_bwd_ds_limit.argtypes = [C.c_int64]
        L.pa_attn_bwd_ds_limit.restype = C.c_int64
        L.pa_attn_bwd_static_scratch_bytes.argtypes = []
        L.pa_attn_bwd_static_scratch_bytes.restype = C.c_int64
        L.pa_abi_version.argtypes = []
        L.pa_abi_version.restype = C.c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise PolyActError(status, lib().pa_status_str(status).decode())


def program_info(func: str, deriv: int, dtype: str = "f16") -> dict:
    """The program the kernels execute (host query, no device work)."""
    out = PaProgram()
    _check(lib().poly_program_info(FUNCS[func], deriv, DTYPE_CODES[dtype], C.byref(out)))
    return {"func": out.func, "deriv": out.deriv, "degree": out.degree, "dtype": out.dtype,
            "Li": out.Li, "Lc": out.Lc, "order": out.order,
            "coeff_bits": [int(out.coeff_bits[j]) for j in range(out.degree + 1)]}


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(entry, *args, on: torch.Tensor, tensors=()):
    """One library call on the device of `on`, made current for the call (the
    library launches on the current device), with that device's current
    stream as the last argument.  Every tensor of the call must live there."""
    for t in tensors:
        if t is not None and t.device != on.device:
            raise ValueError(f"all tensors of a call must be on {on.device}; one is on {t.device}")
    with torch.cuda.device(on.device):
        _check(entry(*args, torch.cuda.current_stream(on.device).cuda_stream))


def _out(out, like):
    if out is None:
        return torch.empty_like(like)
    _dev(out, "out")
    if out.dtype != like.dtype or out.numel() != like.numel():
        raise ValueError("out must match the input's dtype and size")
    return out


def poly_act_fwd(x: torch.Tensor, func: str, out=None) -> torch.Tensor:
    _dev(x, "x")
    y = _out(out, x)
    _call(lib().poly_act_fwd, FUNCS[func], _DTYPES[x.dtype], x.data_ptr(), y.data_ptr(), x.numel(),
          on=x, tensors=(y,))
    return y


def poly_act_bwd(x: torch.Tensor, dy: torch.Tensor, func: str, out=None) -> torch.Tensor:
    _dev(x, "x")
    _dev(dy, "dy")
    if dy.dtype != x.dtype or dy.numel() != x.numel():
        raise ValueError("dy must match x")
    dx = _out(out, x)
    _call(lib().poly_act_bwd, FUNCS[func], _DTYPES[x.dtype], x.data_ptr(), dy.data_ptr(),
          dx.data_ptr(), x.numel(), on=x, tensors=(dy, dx))
    return dx


def native_act_fwd(x: torch.Tensor, func: str, out=None) -> torch.Tensor:
    _dev(x, "x")
    y = _out(out, x)
    _call(lib().native_act_fwd, FUNCS[func], _DTYPES[x.dtype], x.data_ptr(), y.data_ptr(),
          x.numel(), on=x, tensors=(y,))
    return y


def stream_copy(a: torch.Tensor, b: torch.Tensor | None = None, out=None) -> torch.Tensor:
    """The streaming kernels with no arithmetic: out = a, or out = a XOR b
    bitwise when b is given (the elementwise kernels' HBM reference rate)."""
    _dev(a, "a")
    if b is not None:
        _dev(b, "b")
        if b.dtype != a.dtype or b.numel() != a.numel():
            raise ValueError("b must match a")
    y = _out(out, a)
    _call(lib().pa_stream_copy, a.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(),
          a.numel(), on=a, tensors=(b, y))
    return y


def native_act_bwd(x_or_y: torch.Tensor, dy: torch.Tensor, func: str, impl: str = "native",
                   out=None) -> torch.Tensor:
    _dev(x_or_y, "x_or_y")
    _dev(dy, "dy")
    if dy.dtype != x_or_y.dtype or dy.numel() != x_or_y.numel():
        raise ValueError("dy must match x_or_y")
    dx = _out(out, x_or_y)
    _call(lib().native_act_bwd, IMPLS[impl], FUNCS[func], _DTYPES[x_or_y.dtype], x_or_y.data_ptr(),
          dy.data_ptr(), dx.data_ptr(), x_or_y.numel(), on=x_or_y, tensors=(dy, dx))
    return dx


def _mat(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bfloat16 CUDA tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


def _offsets(row_offsets):
    if row_offsets is None:
        return None, 0
    if not row_offsets.is_cuda or row_offsets.dtype != torch.int64 or row_offsets.dim() != 1:
        raise TypeError("row_offsets must be a 1-D int64 CUDA tensor")
    return row_offsets.data_ptr(), row_offsets.numel() - 1


def _swiglu_fwd(entry, gate, up, out, row_offsets):
    ldg, ldu = _mat(gate, "gate"), _mat(up, "up")
    if up.shape != gate.shape:
        raise ValueError("up must match gate")
    h = torch.empty_like(gate) if out is None else out
    ldh = _mat(h, "out")
    if h.shape != gate.shape:   # the kernel writes rows x cols through out
        raise ValueError("out must match gate")
    off, ng = _offsets(row_offsets)
    rows, cols = gate.shape
    _call(entry, 2, gate.data_ptr(), up.data_ptr(), h.data_ptr(), rows, cols, ldg, ldu, ldh, off,
          ng, on=gate, tensors=(up, h, row_offsets))
    return h


def _swiglu_bwd(entry, gate, up, dh, out, row_offsets):
    ldg, ldu, ldd = _mat(gate, "gate"), _mat(up, "up"), _mat(dh, "dh")
    if up.shape != gate.shape or dh.shape != gate.shape:
        raise ValueError("up and dh must match gate")
    dg, du = (torch.empty_like(gate), torch.empty_like(gate)) if out is None else out
    lddg, lddu = _mat(dg, "dgate"), _mat(du, "dup")
    if dg.shape != gate.shape or du.shape != gate.shape:   # written rows x cols
        raise ValueError("dgate and dup must match gate")
    off, ng = _offsets(row_offsets)
    rows, cols = gate.shape
    _call(entry, 2, gate.data_ptr(), up.data_ptr(), dh.data_ptr(), dg.data_ptr(), du.data_ptr(),
          rows, cols, ldg, ldu, ldd, lddg, lddu, off, ng, on=gate,
          tensors=(up, dh, dg, du, row_offsets))
    return dg, du


def poly_swiglu_fwd(gate, up, out=None, row_offsets=None):
    """h = SiLU~(gate) * up (BF16); grouped rows when row_offsets is given."""
    return _swiglu_fwd(lib().poly_swiglu_fwd, gate, up, out, row_offsets)


def poly_swiglu_bwd(gate, up, dh, out=None, row_offsets=None):
    """(dgate, dup) of SwiGLU with the recomputed D3 sigmoid (BF16)."""
    return _swiglu_bwd(lib().poly_swiglu_bwd, gate, up, dh, out, row_offsets)


def native_swiglu_fwd(gate, up, out=None, row_offsets=None):
    return _swiglu_fwd(lib().native_swiglu_fwd, gate, up, out, row_offsets)


def native_swiglu_bwd(gate, up, dh, out=None, row_offsets=None):
    return _swiglu_bwd(lib().native_swiglu_bwd, gate, up, dh, out, row_offsets)


def _bf16_4d(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 \
            or t.dim() != 4 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous bfloat16 CUDA tensor [B, H, S, D]")


def _attn_shapes(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _bf16_4d(t, name)
    B, H, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must be [B, Hkv, S, D] with q's B, S and D")
    return B, H, k.shape[1], S, D


def _like(out, ref, name):
    if out is None:
        return torch.empty_like(ref)
    _bf16_4d(out, name)
    if out.shape != ref.shape:
        raise ValueError(f"{name} must have shape {tuple(ref.shape)}")
    return out


def _softcap_fwd(entry, q, k, v, cap, causal, out, with_lse):
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    o = _like(out, q, "out")
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if with_lse else None
    _call(entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          None if lse is None else lse.data_ptr(), B, H, Hkv, S, D, float(cap), int(bool(causal)),
          on=q, tensors=(k, v, o))
    return (o, lse) if with_lse else o


SOFTCAP_FORMATS = ("bf16", "f16")


def poly_softcap_attn_fwd(q, k, v, cap: float = 50.0, causal: bool = True, out=None,
                          with_lse: bool = False, fmt: str = "bf16"):
    """Softcapped attention forward with the D4 tanh program (BF16 in / out,
    D = 128).  q [B, H, S, D], k and v [B, Hkv, S, D].  fmt: the program's
    format, "bf16" (the pages' path) or "f16" (packed FP16).  Returns O, or
    (O, lse) with with_lse (the natural log-sum-exp per row, FP32 [B, H, S])."""
    if fmt not in SOFTCAP_FORMATS:
        raise ValueError(f"fmt must be one of {SOFTCAP_FORMATS}")
    entry = lib().poly_softcap_attn_fwd if fmt == "bf16" else lib().poly_softcap_attn_fwd_f16
    return _softcap_fwd(entry, q, k, v, cap, causal, out, with_lse)


EXP2_CORES = {"hw": 0, "d1": 1, "pwl2": 2, "d2": 3, "d3": 4}


def _core(core):
    if core not in EXP2_CORES:
        raise ValueError(f"core must be one of {sorted(EXP2_CORES)}")
    return EXP2_CORES[core]


def poly_softcap_attn_fwd_exp2(q, k, v, cap: float = 50.0, causal: bool = True,
                               core: str = "pwl2", out=None, with_lse: bool = False):
    """poly_softcap_attn_fwd (BF16 program) with the softmax's exponentials by
    a software exp2 core: "hw" (v_exp_f32), "d1", "pwl2" (packed FP16), "d2",
    "d3"."""
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    o = _like(out, q, "out")
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if with_lse else None
    _call(lib().poly_softcap_attn_fwd_exp2, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          None if lse is None else lse.data_ptr(), B, H, Hkv, S, D, float(cap), int(bool(causal)),
          _core(core), on=q, tensors=(k, v, o))
    return (o, lse) if with_lse else o


def native_softcap_attn_fwd(q, k, v, cap: float = 50.0, causal: bool = True, out=None,
                            with_lse: bool = False):
    return _softcap_fwd(lib().native_softcap_attn_fwd, q, k, v, cap, causal, out, with_lse)


def _grads(q, k, dq, dk, dv):
    return _like(dq, q, "dq"), _like(dk, k, "dk"), _like(dv, k, "dv")


def attn_bwd_ds_limit(nbytes: int | None = None) -> int:
    """The process-wide limit on the dS blocks an attention backward stores
    (the library's pa_attn_bwd_ds_limit): with nbytes, set it and return the
    previous value; without, return it.  0 makes every backward recompute
    for dQ; size workspaces after a change."""
    return int(lib().pa_attn_bwd_ds_limit(-1 if nbytes is None else int(nbytes)))


def attn_bwd_workspace(softcap: bool, B, H, Hkv, S, D=128, device=None):
    """A workspace tensor of the size the attention backward needs (None if
    it needs none)."""
    n = lib().pa_attn_bwd_workspace_bytes(int(bool(softcap)), B, H, Hkv, S, D)
    if n < 0:
        raise ValueError("invalid attention shape")
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def _ws(workspace, softcap, B, H, Hkv, S, D, device):
    need = lib().pa_attn_bwd_workspace_bytes(int(bool(softcap)), B, H, Hkv, S, D)
    if workspace is None:
        return attn_bwd_workspace(softcap, B, H, Hkv, S, D, device)
    if (workspace.dtype != torch.float32 or workspace.numel() * 4 < need or not workspace.is_cuda
            or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous float32 CUDA tensor of at least {need} bytes")
    return workspace


def _softcap_bwd(entry, q, k, v, o, dout, lse, cap, causal, dq, dk, dv, workspace, extra=()):
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    _bf16_4d(o, "o")
    _bf16_4d(dout, "dout")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, S]")
    dq, dk, dv = _grads(q, k, dq, dk, dv)
    workspace = _ws(workspace, True, B, H, Hkv, S, D, q.device)
    _call(entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, H,
          Hkv, S, D, float(cap), int(bool(causal)), *extra, on=q,
          tensors=(k, v, o, dout, lse, dq, dk, dv, workspace))
    return dq, dk, dv


def poly_softcap_attn_bwd(q, k, v, o, dout, lse, cap: float = 50.0, causal: bool = True,
                          dq=None, dk=None, dv=None, workspace=None, fmt: str = "bf16",
                          core: str | None = None):
    """Backward of poly_softcap_attn_fwd: (dq, dk, dv), with the analytic
    derivative of the D4 tanh program in the forward's format.  core: the
    exp2 core of poly_softcap_attn_fwd_exp2 (BF16 program only)."""
    if fmt not in SOFTCAP_FORMATS:
        raise ValueError(f"fmt must be one of {SOFTCAP_FORMATS}")
    if core is not None:
        if fmt != "bf16":
            raise ValueError("the exp2 cores run with the BF16 program")
        return _softcap_bwd(lib().poly_softcap_attn_bwd_exp2, q, k, v, o, dout, lse, cap, causal,
                            dq, dk, dv, workspace, extra=(_core(core),))
    entry = lib().poly_softcap_attn_bwd if fmt == "bf16" else lib().poly_softcap_attn_bwd_f16
    return _softcap_bwd(entry, q, k, v, o, dout, lse, cap, causal, dq, dk, dv, workspace)


def poly_softcap_attn_bwd_static(q, k, v, o, dout, lse, cap: float = 50.0, causal: bool = True,
                                 dq=None, dk=None, dv=None):
    """poly_softcap_attn_bwd with the library's own device scratch instead of
    a workspace: the call allocates nothing (outputs the caller does not pass
    are created here, before the call).  Calls on one GPU must not overlap."""
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    _bf16_4d(o, "o")
    _bf16_4d(dout, "dout")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, S]")
    dq, dk, dv = _grads(q, k, dq, dk, dv)
    _call(lib().poly_softcap_attn_bwd_static, q.data_ptr(), k.data_ptr(), v.data_ptr(),
          o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
          dv.data_ptr(), B, H, Hkv, S, D, float(cap), int(bool(causal)), on=q,
          tensors=(k, v, o, dout, lse, dq, dk, dv))
    return dq, dk, dv


def native_softcap_attn_bwd(q, k, v, o, dout, lse, cap: float = 50.0, causal: bool = True,
                            dq=None, dk=None, dv=None, workspace=None):
    return _softcap_bwd(lib().native_softcap_attn_bwd, q, k, v, o, dout, lse, cap, causal, dq,
                        dk, dv, workspace)


def _sigmoid_fwd(entry, q, k, v, causal, out):
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    o = _like(out, q, "out")
    _call(entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, Hkv, S, D,
          int(bool(causal)), on=q, tensors=(k, v, o))
    return o


def poly_sigmoid_attn_fwd(q, k, v, causal: bool = True, out=None):
    """Sigmoid attention O = sigma(s - ln S) V with the two-region cubic
    (S must be the program's fitted length, 4096)."""
    return _sigmoid_fwd(lib().poly_sigmoid_attn_fwd, q, k, v, causal, out)


def native_sigmoid_attn_fwd(q, k, v, causal: bool = True, out=None):
    return _sigmoid_fwd(lib().native_sigmoid_attn_fwd, q, k, v, causal, out)


def _sigmoid_bwd(entry, q, k, v, dout, causal, dq, dk, dv, workspace):
    B, H, Hkv, S, D = _attn_shapes(q, k, v)
    _bf16_4d(dout, "dout")
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    dq, dk, dv = _grads(q, k, dq, dk, dv)
    workspace = _ws(workspace, False, B, H, Hkv, S, D, q.device)
    _call(entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
          dk.data_ptr(), dv.data_ptr(), None if workspace is None else workspace.data_ptr(), B, H,
          Hkv, S, D, int(bool(causal)), on=q, tensors=(k, v, dout, dq, dk, dv, workspace))
    return dq, dk, dv


def poly_sigmoid_attn_bwd(q, k, v, dout, causal: bool = True, dq=None, dk=None, dv=None,
                          workspace=None):
    """Backward of poly_sigmoid_attn_fwd with the factored derivative surrogate."""
    return _sigmoid_bwd(lib().poly_sigmoid_attn_bwd, q, k, v, dout, causal, dq, dk, dv,
                        workspace)


def native_sigmoid_attn_bwd(q, k, v, dout, causal: bool = True, dq=None, dk=None, dv=None,
                            workspace=None):
    return _sigmoid_bwd(lib().native_sigmoid_attn_bwd, q, k, v, dout, causal, dq, dk, dv,
                        workspace)


def sigmoid_attn_program() -> dict:
    """The sigmoid-attention program the kernels execute (host query)."""
    out = PaSigmoidAttnProgram()
    _check(lib().poly_sigmoid_attn_program(C.byref(out)))
    return {"n": out.n, "thr": out.thr, "clamp_lo": out.clamp_lo, "clamp_hi": out.clamp_hi,
            "coeff_bits": [[int(out.coeff_bits[r][j]) for j in range(4)] for r in range(2)],
            "a_bits": [int(x) for x in out.a_bits], "b_bits": [int(x) for x in out.b_bits],
            "order": out.order}


# ---- rotary position embedding ---------------------------------------------

def _rope_io(q, k, q_out, k_out):
    _dev(q, "q")
    _dev(k, "k")
    if q.dtype != torch.float16 or k.dtype != torch.float16:
        raise TypeError("q and k must be float16")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, S, Hq, D] and k [B, S, Hkv, D]")
    B, S, Hq, D = q.shape
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError("k must be [B, S, Hkv, D] with q's B, S and D")
    Hkv = k.shape[2]
    if q_out is None:
        q_out = torch.empty((B, Hq, S, D), dtype=q.dtype, device=q.device)
    if k_out is None:
        k_out = torch.empty((B, Hkv, S, D), dtype=k.dtype, device=k.device)
    for t, name, shape in ((q_out, "q_out", (B, Hq, S, D)), (k_out, "k_out", (B, Hkv, S, D))):
        _dev(t, name)
        if tuple(t.shape) != shape or t.dtype != torch.float16:
            raise ValueError(f"{name} must be float16 {list(shape)}")
    return q_out, k_out, (B, S, Hq, Hkv, D)


def poly_rope(q, k, base: float = 10000.0, q_out=None, k_out=None):
    """Rotary embedding with the paired D5 sine / D6 cosine programs
    (Appendix B.2): q [B, S, Hq, D], k [B, S, Hkv, D] FP16 -> q_out
    [B, Hq, S, D], k_out [B, Hkv, S, D]."""
    q_out, k_out, (B, S, Hq, Hkv, D) = _rope_io(q, k, q_out, k_out)
    _call(lib().poly_rope, q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), B, S, Hq,
          Hkv, D, float(base), on=q, tensors=(k, q_out, k_out))
    return q_out, k_out


def native_rope(q, k, base: float = 10000.0, q_out=None, k_out=None):
    """The same rotation with accurate sinf / cosf computed on the fly."""
    q_out, k_out, (B, S, Hq, Hkv, D) = _rope_io(q, k, q_out, k_out)
    _call(lib().native_rope, q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), B, S,
          Hq, Hkv, D, float(base), on=q, tensors=(k, q_out, k_out))
    return q_out, k_out


def rope_table(S: int, D: int, base: float = 10000.0, device=None) -> torch.Tensor:
    """The comparator's (cos, sin) table: int32 [S, D / 2] words (two FP16 values)."""
    t = torch.empty((S, D // 2), dtype=torch.int32, device=device or "cuda")
    _call(lib().pa_rope_table, t.data_ptr(), S, D, float(base), on=t)
    return t


def native_rope_table(q, k, table: torch.Tensor, q_out=None, k_out=None):
    """The same rotation with (cos, sin) read from a rope_table."""
    q_out, k_out, (B, S, Hq, Hkv, D) = _rope_io(q, k, q_out, k_out)
    if not table.is_cuda or table.numel() != S * (D // 2) or not table.is_contiguous():
        raise ValueError("table must be a contiguous device tensor of S * D / 2 words")
    _call(lib().native_rope_table, q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(),
          table.data_ptr(), B, S, Hq, Hkv, D, on=q, tensors=(k, q_out, k_out, table))
    return q_out, k_out


def rope_program() -> dict:
    """BF16 bits of the sine (a1, a3, a5) and cosine (b0, b2, b4, b6) programs."""
    out = PaRopeProgram()
    _check(lib().poly_rope_program(C.byref(out)))
    return {"sin_bits": [int(x) for x in out.sin_bits], "cos_bits": [int(x) for x in out.cos_bits]}

