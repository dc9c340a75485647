"""ctypes binding of the attention oracle (test infrastructure only).

Takes numpy arrays (bf16 as uint16 bit patterns); imports nothing from the
product package.
"""
from __future__ import annotations

import contextlib
import ctypes as C

import numpy as np

from . import moe_oracle as _mo

MUTANTS = {"window_short": 1, "rope_interleaved": 2, "no_scale": 3, "rope_sign": 4}

_lib = None


def lib():
    global _lib
    if _lib is None:
        L = _mo.lib()  # the same shared library
        p, i32 = C.c_void_p, C.c_int32
        L.attn_oracle_rope.argtypes = [i32, i32, i32, i32, C.c_double, p]
        L.attn_oracle_attention.argtypes = [i32, i32, i32, i32, i32, i32, i32, p, p, p, p]
        L.attn_oracle_set_mutant.argtypes = [C.c_int]
        _lib = L
    return _lib


def rope(x_bits: np.ndarray, pos0: int, theta: float) -> np.ndarray:
    """x [T, H, D] bf16 bits -> rotated copy (bf16 bits)."""
    x = np.ascontiguousarray(x_bits, np.uint16).copy()
    T, H, D = x.shape
    rc = lib().attn_oracle_rope(T, H, D, int(pos0), float(theta), x.ctypes.data)
    assert rc == 0, rc
    return x


def attention(q, k, v, q_pos0: int, window: int) -> np.ndarray:
    """q [Tq, Hq, D], k, v [Tk, Hkv, D] bf16 bits -> o [Tq, Hq, D] float32."""
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    o = np.empty((Tq, Hq, D), np.float32)
    rc = lib().attn_oracle_attention(Tq, Tk, Hq, Hkv, D, int(q_pos0), int(window), q.ctypes.data, k.ctypes.data,
                                     v.ctypes.data, o.ctypes.data)
    assert rc == 0, rc
    return o


@contextlib.contextmanager
def mutant(name: str):
    L = lib()
    L.attn_oracle_set_mutant(MUTANTS[name])
    try:
        yield
    finally:
        L.attn_oracle_set_mutant(0)
