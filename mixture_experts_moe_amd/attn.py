"""Python binding of include/moe_attn.h (argument marshalling only).

RoPE and causal sliding-window / whole-context attention run in the HIP library
``libmoe.so`` (the same library as the layer); there is no fallback.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import moe

ABI_FUNCTIONS = ("moe_rope", "moe_attn_workspace_bytes", "moe_attention")
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4


class AttnShape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_q_heads", "n_kv_heads", "head_dim", "window")]


_ready = False


def lib() -> C.CDLL:
    global _ready
    L = moe.lib()
    if not _ready:
        p, i32 = C.c_void_p, C.c_int32
        L.moe_rope.argtypes = [i32, i32, i32, i32, C.c_float, p, p]
        L.moe_attn_workspace_bytes.restype = C.c_size_t
        L.moe_attn_workspace_bytes.argtypes = [p, i32, i32, i32]
        L.moe_attention.argtypes = [p, i32, i32, i32, p, p, p, p, p, C.c_size_t, p]
        _ready = True
    return L


class AttnError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: status {rc}")
        self.rc = rc


def _check(rc, what):
    if rc != OK:
        raise AttnError(rc, what)


def rope_(x: torch.Tensor, pos0: int, theta: float, stream=None) -> torch.Tensor:
    """In-place RoPE of x [T, H, D] bf16 (token t at position pos0 + t)."""
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise ValueError("moe_rope: x must be a [T, H, D] bfloat16 tensor")
    T, H, D = x.shape
    _check(lib().moe_rope(T, H, D, int(pos0), float(theta), moe._ptr(x), moe._stream(stream)), "moe_rope")
    return x


def workspace_bytes(shape: AttnShape, Tq: int, Tk: int, q_pos0: int) -> int:
    return int(lib().moe_attn_workspace_bytes(C.byref(shape), Tq, Tk, q_pos0))


class Attention:
    """moe_attention for one call shape, workspace allocated once."""

    def __init__(self, shape: AttnShape, Tq: int, Tk: int, q_pos0: int, device="cuda"):
        self.shape, self.Tq, self.Tk, self.q_pos0 = shape, int(Tq), int(Tk), int(q_pos0)
        self.ws = torch.empty(max(workspace_bytes(shape, Tq, Tk, q_pos0), 256), dtype=torch.uint8, device=device)

    def __call__(self, q, k, v, o, stream=None):
        for t in (q, k, v, o):
            if t.dtype != torch.bfloat16:
                raise ValueError("moe_attention: bfloat16 tensors expected")
        rc = lib().moe_attention(C.byref(self.shape), self.Tq, self.Tk, self.q_pos0, moe._ptr(q), moe._ptr(k),
                                 moe._ptr(v), moe._ptr(o), moe._ptr(self.ws), self.ws.numel(), moe._stream(stream))
        _check(rc, "moe_attention")
        return o


def attention(shape: AttnShape, q, k, v, q_pos0: int, stream=None) -> torch.Tensor:
    o = torch.empty_like(q)
    return Attention(shape, q.shape[0], k.shape[0], q_pos0, q.device)(q, k, v, o, stream)
