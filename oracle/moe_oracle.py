"""ctypes binding of the C++ oracle (test infrastructure only).

Takes the numpy arrays produced by the seeded input generator; imports nothing
from the product package.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os

import numpy as np

from . import build as _build

ACT = {"f32": 0, "bf16": 1}
WDT = {"f32": 0, "bf16": 1, "fp8": 2, "fp8a16": 3, "u4": 4}
OK, ERR_INVALID, ERR_FORCED_INDEX = 0, -1, -5

MUTANTS = {
    "select_unbiased": 1, "router_bf16": 2, "logits_bf16": 3, "tie_highest": 4, "softmax_all": 5,
    "no_shared": 6, "scale_transposed": 7, "reversed_order": 8, "no_h_quant": 9, "weights_biased": 10,
    "silu_sign": 11, "gate_up_swap": 12, "combine_no_weight": 13, "u4_nibble_swap": 14, "u4_no_bias": 15,
    "u4_group128": 16, "compare_min_pair": 17, "compare_unbiased": 18, "quant_reciprocal": 19,
    "quant_ties_away": 20,
}


class _Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "d", "E", "k", "F", "Fs", "act_dtype", "w_dtype")]


_WEIGHT_FIELDS = ("w_router", "sel_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                  "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down",
                  "b_gate", "b_up", "b_down", "sb_gate", "sb_up", "sb_down")


class _Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _WEIGHT_FIELDS]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        p, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.oracle_e4m3_decode.restype = C.c_float
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [C.c_float]
        L.oracle_f32_to_bf16.restype = C.c_uint16
        L.oracle_f32_to_bf16.argtypes = [C.c_float]
        L.oracle_e4m3_encode_array.argtypes = [p, p, i64]
        L.oracle_f32_to_bf16_array.argtypes = [p, p, i64]
        L.oracle_quant_groups.argtypes = [p, i64, p, p]
        L.oracle_set_mutant.argtypes = [C.c_int]
        L.oracle_route.argtypes = [p, p, p, p, i32, p, p, p]
        L.oracle_route_forced.argtypes = [p, p, p, p, p, i32, p, p, p]
        L.oracle_dispatch.argtypes = [i32, i32, i32, p, p, p, p, p]
        L.oracle_forward.argtypes = [p, p, p, p, p, p, i32, p, p]
        L.oracle_forward_dense_masked.argtypes = [p, p, p, p, p, p]
        L.oracle_expert_ffn.argtypes = [p, p, i32, p, i32, p, p]
        L.oracle_expert_ffn_trace.argtypes = [p, p, i32, p, i32, p, p, p, p, p, p, p]
        L.oracle_route_threads.argtypes = [p, p, p, p, i32, p, p, p, i32]
        L.oracle_forward_threads.argtypes = [p, p, p, p, p, p, i32, p, p, i32]
        L.oracle_route_compare.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


class Layer:
    """Holds contiguous copies of one layer's inputs and the C structs."""

    def __init__(self, inp: dict):
        s = inp["shape"]
        self.s = s
        self._keep = {k: _c(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
        if inp.get("sel_bias") is None:
            self._keep.pop("sel_bias", None)
        self.shape = _Shape(s.T, s.d, s.E, s.k, s.F, s.Fs, ACT[s.act], WDT[s.w])
        self.weights = _Weights(*[_ptr(self._keep.get(n)) for n in _WEIGHT_FIELDS])
        self.x = self._keep["x"]

    def _args(self):
        return C.byref(self.shape), C.byref(self.weights), _ptr(self.x)


def _tokens(s, tokens):
    if tokens is None:
        return None, s.T
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return t, len(t)


def route(layer: Layer, tokens=None):
    """Free routing. Returns (rc, logits [n,E], idx [n,k], w [n,k])."""
    s = layer.s
    tl, n = _tokens(s, tokens)
    logits = np.empty((n, s.E), np.float32)
    idx = np.empty((n, s.k), np.int32)
    w = np.empty((n, s.k), np.float32)
    rc = lib().oracle_route(*layer._args(), _ptr(tl), n, _ptr(logits), _ptr(idx), _ptr(w))
    return rc, logits, idx, w


def route_forced(layer: Layer, forced, tokens=None):
    s = layer.s
    forced = _c(forced, np.int32)
    assert forced.shape == (s.T, s.k)
    tl, n = _tokens(s, tokens)
    logits = np.empty((n, s.E), np.float32)
    idx = np.empty((n, s.k), np.int32)
    w = np.empty((n, s.k), np.float32)
    rc = lib().oracle_route_forced(*layer._args(), _ptr(forced), _ptr(tl), n, _ptr(logits), _ptr(idx), _ptr(w))
    return rc, logits, idx, w


def host_threads() -> int:
    """Threads for the all-cores oracle runs: the host's cores, at most 16
    (a GPU machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


def route_threads(layer: Layer, tokens=None, n_threads=None):
    """route() over contiguous token ranges on n_threads std::threads; bitwise
    the single-threaded result."""
    s = layer.s
    tl, n = _tokens(s, tokens)
    logits = np.empty((n, s.E), np.float32)
    idx = np.empty((n, s.k), np.int32)
    w = np.empty((n, s.k), np.float32)
    rc = lib().oracle_route_threads(*layer._args(), _ptr(tl), n, _ptr(logits), _ptr(idx), _ptr(w),
                                    n_threads or host_threads())
    return rc, logits, idx, w


def dispatch(idx, E: int):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    P = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(P, np.int32)
    inv = np.empty(P, np.int32)
    rc = lib().oracle_dispatch(T, k, E, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv))
    assert rc == OK
    return counts, offsets, perm, inv


def forward(layer: Layer, idx, w, tokens=None):
    """Layer output for the listed tokens (idx, w rows aligned with them).
    Returns (y in the activation dtype: f32 or uint16 bf16 bits, acc f32)."""
    s = layer.s
    tl, n = _tokens(s, tokens)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    assert idx.shape == (n, s.k) and w.shape == (n, s.k)
    y = np.empty((n, s.d), np.float32 if s.act == "f32" else np.uint16)
    acc = np.empty((n, s.d), np.float32)
    rc = lib().oracle_forward(*layer._args(), _ptr(idx), _ptr(w), _ptr(tl), n, _ptr(y), _ptr(acc))
    assert rc == OK, rc
    return y, acc


def forward_threads(layer: Layer, idx, w, tokens=None, n_threads=None):
    """forward() over contiguous token ranges on n_threads std::threads;
    bitwise the single-threaded result."""
    s = layer.s
    tl, n = _tokens(s, tokens)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    assert idx.shape == (n, s.k) and w.shape == (n, s.k)
    y = np.empty((n, s.d), np.float32 if s.act == "f32" else np.uint16)
    acc = np.empty((n, s.d), np.float32)
    rc = lib().oracle_forward_threads(*layer._args(), _ptr(idx), _ptr(w), _ptr(tl), n, _ptr(y), _ptr(acc),
                                      n_threads or host_threads())
    assert rc == OK, rc
    return y, acc


def forward_dense_masked(layer: Layer, idx, w):
    s = layer.s
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    acc = np.empty((s.T, s.d), np.float32)
    rc = lib().oracle_forward_dense_masked(*layer._args(), _ptr(idx), _ptr(w), _ptr(acc))
    assert rc == OK, rc
    return acc


def expert_ffn(layer: Layer, expert: int, t: int):
    """One expert (-1: shared) on token t. Returns (x as the FFN sees it, y)."""
    s = layer.s
    xu = np.empty(s.d, np.float32)
    y = np.empty(s.d, np.float32)
    sp, wp, xp = layer._args()
    rc = lib().oracle_expert_ffn(sp, wp, expert, xp, t, _ptr(xu), _ptr(y))
    assert rc == OK, rc
    return xu, y


def expert_ffn_trace(layer: Layer, expert: int, t: int) -> dict:
    """One expert (-1: shared) on token t, with what the forward quantised
    (FP8 weights): x_codes [d] uint8, x_scales [d/128], h [F] (before
    quantisation), h_codes [F] uint8, h_scales [F/128], x_used [d], y [d]."""
    s = layer.s
    F = s.Fs if expert < 0 else s.F
    out = dict(x_codes=np.zeros(s.d, np.uint8), x_scales=np.zeros(s.d // 128, np.float32),
               h=np.zeros(F, np.float32), h_codes=np.zeros(F, np.uint8), h_scales=np.zeros(F // 128, np.float32),
               x_used=np.zeros(s.d, np.float32), y=np.zeros(s.d, np.float32))
    sp, wp, xp = layer._args()
    rc = lib().oracle_expert_ffn_trace(sp, wp, expert, xp, t, *(_ptr(out[n]) for n in (
        "x_codes", "x_scales", "h", "h_codes", "h_scales", "x_used", "y")))
    assert rc == OK, rc
    return out


def route_compare(logits, ref_logits, idx, ref_idx, sel_bias=None):
    """Routing compared as a distribution. Returns (gap [T] float32, sigma,
    number of disagreeing tokens, largest gap)."""
    logits = _c(logits, np.float32)
    ref_logits = _c(ref_logits, np.float32)
    idx = _c(idx, np.int32)
    ref_idx = _c(ref_idx, np.int32)
    bias = _c(sel_bias, np.float32)
    T, E = logits.shape
    k = idx.shape[1]
    assert ref_logits.shape == (T, E) and ref_idx.shape == (T, k)
    gap = np.empty(T, np.float32)
    sigma = C.c_double()
    nd = C.c_int32()
    mg = C.c_float()
    rc = lib().oracle_route_compare(T, E, k, _ptr(logits), _ptr(ref_logits), _ptr(bias), _ptr(idx), _ptr(ref_idx),
                                    _ptr(gap), C.addressof(sigma), C.addressof(nd), C.addressof(mg))
    assert rc == OK, rc
    return gap, sigma.value, nd.value, mg.value


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e4m3_decode(int(c)) for c in np.asarray(codes).ravel()], np.float32)


def e4m3_encode(v) -> np.ndarray:
    v = _c(np.asarray(v, np.float32).ravel(), np.float32)
    out = np.empty(v.size, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def f32_to_bf16(v) -> np.ndarray:
    v = _c(np.asarray(v, np.float32).ravel(), np.float32)
    out = np.empty(v.size, np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(v), _ptr(out), v.size)
    return out


def quant_groups(v):
    """Per-128-group dynamic E4M3 quantisation: (codes uint8 [n*128], scales f32 [n])."""
    v = _c(np.asarray(v, np.float32).ravel(), np.float32)
    assert v.size % 128 == 0
    g = v.size // 128
    codes = np.empty(v.size, np.uint8)
    scales = np.empty(g, np.float32)
    lib().oracle_quant_groups(_ptr(v), g, _ptr(codes), _ptr(scales))
    return codes, scales


@contextlib.contextmanager
def mutant(name: str):
    """Plant one deliberate bug in the oracle for the duration of the block."""
    L = lib()
    L.oracle_set_mutant(MUTANTS[name])
    try:
        yield
    finally:
        L.oracle_set_mutant(0)
