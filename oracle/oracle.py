"""ctypes front end of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg.  The HIP library and its binding never import it.

Arrays cross as numpy (bf16 as uint16 bit patterns).  ``build()`` compiles the
C source with gcc; ``load()`` builds only when no library is present.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, MXFP4, FP8, NVFP4 = 0, 1, 2, 3, 4
_FMT = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "fp8": FP8, "nvfp4": NVFP4}

_lib = None


def build() -> str:
    # ISO C (-std=c11) keeps floating-point contraction off; no semantic
    # interposition lets the format decoders inline into the per-element loops
    cmd = ["gcc", "-O3", "-fno-fast-math", "-fno-semantic-interposition", "-fopenmp", "-shared",
           "-fPIC", "-std=c11", "-Wall", SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class _Expert(C.Structure):
    _fields_ = [("fmt", C.c_int), ("gate", C.c_void_p), ("up", C.c_void_p),
                ("down", C.c_void_p), ("gate_sc", C.c_void_p), ("up_sc", C.c_void_p),
                ("down_sc", C.c_void_p), ("gate_ts", C.c_void_p), ("up_ts", C.c_void_p),
                ("down_ts", C.c_void_p)]


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    lib = C.CDLL(LIB)
    P = C.c_void_p
    lib.or_mxfp4_value.restype = C.c_double
    lib.or_mxfp4_value.argtypes = [C.c_uint8, C.c_uint8]
    lib.or_fp8_value.restype = C.c_double
    lib.or_fp8_value.argtypes = [C.c_uint8]
    lib.or_nvfp4_value.restype = C.c_double
    lib.or_nvfp4_value.argtypes = [C.c_uint8, C.c_uint8]
    lib.or_bf16_to_f64.restype = C.c_double
    lib.or_bf16_to_f64.argtypes = [C.c_uint16]
    lib.or_f64_to_bf16.restype = C.c_uint16
    lib.or_f64_to_bf16.argtypes = [C.c_double]
    lib.or_router_logits.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, P]
    lib.or_route.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P, P]
    lib.or_align.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P, P, P]
    lib.or_expert_ffn.argtypes = [C.POINTER(_Expert), P, C.c_int, C.c_int, C.c_int, P]
    lib.or_moe_layer.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                 P, P, C.POINTER(_Expert), C.POINTER(_Expert), C.c_int,
                                 C.c_int, P, P, C.c_int, C.c_int]
    lib.or_max_threads.restype = C.c_int
    for name in ("or_table_e2m1", "or_table_pow2", "or_table_fp8"):
        getattr(lib, name).restype = C.c_double
        getattr(lib, name).argtypes = [C.c_uint8]
    _lib = lib
    return lib


def _np(a, dtype=None):
    """torch tensor or numpy array -> contiguous numpy (bf16 -> uint16 bits)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _fmt_of(a: np.ndarray) -> int:
    return F32 if a.dtype == np.float32 else BF16


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ---- scalar helpers ---------------------------------------------------------
def mxfp4_value(code: int, scale: int) -> float:
    return load().or_mxfp4_value(code, scale)


def fp8_value(code: int) -> float:
    return load().or_fp8_value(code)


def nvfp4_value(code: int, scale: int) -> float:
    return load().or_nvfp4_value(code, scale)


def bf16_to_f64(b: int) -> float:
    return load().or_bf16_to_f64(b)


def f64_to_bf16(v: float) -> int:
    return load().or_f64_to_bf16(v)


# ---- layer steps ------------------------------------------------------------
def router_logits(x, wr) -> np.ndarray:
    x, wr = _np(x), _np(wr)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    rc = load().or_router_logits(_ptr(x), _ptr(wr), _fmt_of(x), T, H, E, _ptr(out))
    assert rc == 0
    return out


def route(logits, k: int, bias=None):
    lg = _np(logits, np.float32)
    T, E = lg.shape
    b = None if bias is None else _np(bias, np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = load().or_route(_ptr(lg), None if b is None else _ptr(b), T, E, k, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError(f"or_route failed ({rc})")
    return ids, w


def align(ids, E: int):
    ids = _np(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    rc = load().or_align(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv))
    assert rc == 0
    return counts, offsets, perm, inv


class ExpertSet:
    """Keeps numpy copies of expert weights alive and exposes or_expert structs."""

    def __init__(self, experts: list, wdtype: str):
        self.keep = []
        self.structs = (_Expert * max(1, len(experts)))()
        for i, ex in enumerate(experts):
            s = self.structs[i]
            s.fmt = _FMT[wdtype]
            for name in ("gate", "up", "down"):
                a = _np(ex[name])
                self.keep.append(a)
                setattr(s, name, a.ctypes.data)
                if wdtype in ("mxfp4", "fp8", "nvfp4"):
                    sc = _np(ex[name + "_sc"])
                    self.keep.append(sc)
                    setattr(s, name + "_sc", sc.ctypes.data)
                if wdtype == "nvfp4":
                    ts = np.ascontiguousarray(ex[name + "_ts"], dtype=np.float32).reshape(1)
                    self.keep.append(ts)
                    setattr(s, name + "_ts", ts.ctypes.data)


def expert_ffn(expert: dict, wdtype: str, x_row, H: int, I: int, round_h: bool) -> np.ndarray:
    es = ExpertSet([expert], wdtype)
    xr = np.ascontiguousarray(x_row, dtype=np.float64)
    y = np.empty(H, np.float64)
    load().or_expert_ffn(C.byref(es.structs[0]), _ptr(xr), H, I, int(round_h), _ptr(y))
    return y


def moe_layer(x, ids, w, experts: list, wdtype: str, I: int, shared=None, out_fmt=None,
              tokens=None, nthreads: int = 0) -> np.ndarray:
    """Routed layer output for all tokens (or the rows listed in ``tokens``).

    ``out_fmt`` defaults to the activation format; bf16 output comes back as
    uint16 bit patterns.  h is rounded to bf16 unless weights are fp32."""
    x = _np(x)
    T, H = x.shape
    ids = _np(ids, np.int32)
    w = _np(w, np.float32)
    k = ids.shape[1]
    E = len(experts)
    xf = _fmt_of(x)
    of = xf if out_fmt is None else _FMT[out_fmt]
    es = ExpertSet(experts, wdtype)
    sh = ExpertSet([shared], wdtype) if shared is not None else None
    if tokens is None:
        n = T
        tok = None
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(tok)
    out = np.empty((n, H), np.float32 if of == F32 else np.uint16)
    rc = load().or_moe_layer(_ptr(x), xf, T, H, I, E, k, _ptr(ids), _ptr(w), es.structs,
                             C.byref(sh.structs[0]) if sh else None, int(wdtype != "f32"), of,
                             _ptr(out), None if tok is None else _ptr(tok), n, nthreads)
    assert rc == 0, rc
    return out


def max_threads() -> int:
    return load().or_max_threads()


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
