"""ctypes access to the float64 C reference products (oracle/w4_matvec.c).

Test infrastructure only.  The shared library is built in place from
oracle/w4_matvec.c with gcc (by __graft_entry__.build(), or here on first use).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .moe_oracle import silu

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "w4_matvec.c")
LIB = os.path.join(_DIR, "libw4ref.so")
_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.w4_matvec.argtypes = [P, P, I64, I64, I64, P, I64, P]
        lib.w4_matvec.restype = ctypes.c_int
        lib.w4_dequant_rows.argtypes = [P, P, I64, I64, I64, I64, P]
        lib.w4_dequant_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _group(q, s):
    """Group size from the stored shapes: q [out, in/2], s [out, in/gs]."""
    in_dim = q.shape[1] * 2
    gs = in_dim // s.shape[1]
    if gs not in (64, 128, 256) or gs * s.shape[1] != in_dim or s.shape[0] != q.shape[0]:
        raise ValueError(f"scales {s.shape} do not fit codes {q.shape} with a group of 64/128/256")
    return in_dim, gs


def w4_matvec(q: np.ndarray, s: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_c q[n, c] s[n, c // gs] x[t, c] in float64, from the
    stored arrays q (uint8 [out, in/2]) and s (fp16 [out, in/gs]); the group
    size gs (64, 128 or 256) follows from the shapes."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float16)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
    out_dim = q.shape[0]
    in_dim, gs = _group(q, s)
    assert x.shape[1] == in_dim
    y = np.empty((x.shape[0], out_dim), dtype=np.float64)
    if _load().w4_matvec(q.ctypes.data, s.ctypes.data, out_dim, in_dim, gs, x.ctypes.data,
                         x.shape[0], y.ctypes.data) != 0:
        raise ValueError(f"shape [{out_dim}, {in_dim}] with group {gs} not supported")
    return y


def dequant_rows(q: np.ndarray, s: np.ndarray, r0: int, r1: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float16)
    in_dim, gs = _group(q, s)
    out = np.empty((r1 - r0, in_dim), dtype=np.float64)
    if _load().w4_dequant_rows(q.ctypes.data, s.ctypes.data, in_dim, gs, r0, r1,
                               out.ctypes.data) != 0:
        raise ValueError(f"shape [*, {in_dim}] with group {gs} not supported")
    return out


def expert_ffn_w4_c(X, gate_q, gate_s, up_q, up_s, down_q, down_s) -> np.ndarray:
    """One routed expert's SwiGLU FFN, y = (silu(X Wg^T) * (X Wu^T)) Wd^T, with
    the products evaluated by the C reference (same definition as
    oracle.expert_ffn_w4, without materialising the dequantized matrices)."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    h = silu(w4_matvec(gate_q, gate_s, X)) * w4_matvec(up_q, up_s, X)
    return w4_matvec(down_q, down_s, h)
