"""Python binding of the C ABI in include/moe.h (argument marshalling only).

Every step of the layer runs in the HIP library ``libmoe.so``; this module only
turns torch tensors into device pointers and the current torch stream into the
``stream`` argument.  There is no fallback: if the library is missing or fails
to load, every entry point raises.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_FORCED_INDEX, MOE_ERR_DEVICE_SYNC = -5, -6  # device status word
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "fp8a16": 3, "u4": 4}

# Every function the header declares (checked against include/moe.h by the tests).
ABI_FUNCTIONS = ("moe_workspace_bytes", "moe_plan_bytes", "moe_route", "moe_route_forced", "moe_forward",
                 "moe_forward_noalloc", "moe_forward_stages", "moe_quantize_rows", "moe_pack_weights",
                 "moe_pack_weights_u4", "moe_route_compare_workspace_bytes", "moe_route_compare", "moe_status_string",
                 "moe_router_planes_bytes", "moe_pack_router")
MOE_ERR_SCRATCH_LIMIT = -7
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
LAYOUTS = {"rowmajor": 0, "tiled": 1}
STAGE_GATE_UP, STAGE_DOWN, STAGE_COMBINE, STAGE_ALL = 1, 2, 4, 7
FORWARD_TEST_WAIT_TIMEOUT = 0x100  # error-path test hook of the one-launch expert kernel
N_STAGE_EVENTS = 4


class MoeError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: {status_string(rc)} ({rc})")
        self.rc = rc


class Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "d_model", "n_experts", "top_k", "d_ffn", "d_ffn_shared",
                                         "act_dtype", "w_dtype", "w_layout")]


_WEIGHT_FIELDS = ("w_router", "sel_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                  "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down", "w_router_planes")


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _WEIGHT_FIELDS]


_ROUTING_FIELDS = ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "status", "plan")


class RoutingStruct(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _ROUTING_FIELDS] + [("plan_bytes", C.c_size_t),
                                                             ("forward_status", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    """Load libmoe.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = C.CDLL(LIB_PATH)
        p, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.moe_workspace_bytes.restype = C.c_size_t
        L.moe_workspace_bytes.argtypes = [p]
        L.moe_plan_bytes.restype = C.c_size_t
        L.moe_plan_bytes.argtypes = [p]
        L.moe_route.argtypes = [p, p, p, p, p, C.c_size_t, p]
        L.moe_route_forced.argtypes = [p, p, p, p, p, p, C.c_size_t, p]
        L.moe_forward.argtypes = [p, p, p, p, p, p, C.c_size_t, p]
        L.moe_forward_stages.argtypes = [p, p, p, p, p, p, C.c_size_t, C.c_uint32, p, p]
        L.moe_forward_noalloc.argtypes = [p, p, p, p, p, p]
        L.moe_quantize_rows.argtypes = [i64, i32, i32, p, p, p, p]
        L.moe_pack_weights.argtypes = [i64, i32, i32, p, p, p]
        L.moe_pack_weights_u4.argtypes = [i64, i32, i32, p, p, p, p, p, p]
        L.moe_route_compare_workspace_bytes.restype = C.c_size_t
        L.moe_route_compare_workspace_bytes.argtypes = [i32]
        L.moe_route_compare.argtypes = [i32, i32, i32, p, p, p, p, p, p, p, p, p, p, C.c_size_t, p]
        L.moe_router_planes_bytes.restype = C.c_size_t
        L.moe_router_planes_bytes.argtypes = [i32, i32]
        L.moe_pack_router.argtypes = [i32, i32, p, p, p]
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [C.c_int]
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().moe_status_string(rc).decode()


def make_shape(T, d, E, k, F, Fs, act="bf16", w="fp8", layout="rowmajor") -> Shape:
    return Shape(int(T), int(d), int(E), int(k), int(F), int(Fs), DTYPES[act], DTYPES[w], LAYOUTS[layout])


def shape_of(layer_shape, T=None, layout=None) -> Shape:
    """Shape from any object with attributes T, d, E, k, F, Fs, act, w.  The
    layout defaults to row-major, and to tiled for 4-bit weights (their only
    layout)."""
    s = layer_shape
    if layout is None:
        layout = "tiled" if s.w == "u4" else "rowmajor"
    return make_shape(s.T if T is None else T, s.d, s.E, s.k, s.F, s.Fs, s.act, s.w, layout)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("moe: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("moe: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def weights_struct(w: dict) -> Weights:
    return Weights(*[_ptr(w.get(n)) for n in _WEIGHT_FIELDS])


@dataclasses.dataclass
class Routing:
    """Device buffers of one routing result (see moe_routing in include/moe.h)."""
    logits: torch.Tensor | None
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    inv_perm: torch.Tensor
    status: torch.Tensor
    plan: torch.Tensor  # opaque dispatch plan (at least moe_plan_bytes bytes)
    forward_status: torch.Tensor | None = None  # sticky: MOE_ERR_DEVICE_SYNC of any forward call, until zeroed

    def struct(self) -> RoutingStruct:
        return RoutingStruct(*[_ptr(getattr(self, n)) for n in _ROUTING_FIELDS], self.plan.numel(),
                             _ptr(self.forward_status))


def alloc_routing(shape: Shape, device="cuda", with_logits=True) -> Routing:
    T, E, k = shape.T, shape.n_experts, shape.top_k
    i32 = dict(dtype=torch.int32, device=device)
    return Routing(
        logits=torch.empty((T, E), dtype=torch.float32, device=device) if with_logits else None,
        topk_idx=torch.empty((T, k), **i32), topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
        counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
        perm=torch.empty(T * k, **i32), inv_perm=torch.empty(T * k, **i32), status=torch.empty(1, **i32),
        plan=torch.empty(max(plan_bytes(shape), 256), dtype=torch.uint8, device=device),
        forward_status=torch.zeros(1, **i32))


def workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_workspace_bytes(C.byref(shape)))


def plan_bytes(shape: Shape) -> int:
    return int(lib().moe_plan_bytes(C.byref(shape)))


def alloc_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    n = workspace_bytes(shape)
    if n == 0 and shape.T > 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, "moe_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check(rc, what):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def route(shape: Shape, w: dict, x: torch.Tensor, out: Routing, ws: torch.Tensor, stream=None):
    rc = lib().moe_route(C.byref(shape), C.byref(weights_struct(w)), _ptr(x), C.byref(out.struct()),
                         _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "moe_route")


def route_forced(shape: Shape, w: dict, x: torch.Tensor, forced_idx: torch.Tensor, out: Routing, ws: torch.Tensor,
                 stream=None):
    rc = lib().moe_route_forced(C.byref(shape), C.byref(weights_struct(w)), _ptr(x), _ptr(forced_idx),
                                C.byref(out.struct()), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "moe_route_forced")


def forward(shape: Shape, w: dict, x: torch.Tensor, r: Routing, y: torch.Tensor, ws: torch.Tensor, stream=None):
    rc = lib().moe_forward(C.byref(shape), C.byref(weights_struct(w)), _ptr(x), C.byref(r.struct()), _ptr(y),
                           _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "moe_forward")


def forward_noalloc(shape: Shape, w: dict, x: torch.Tensor, r: Routing, y: torch.Tensor, stream=None):
    """moe_forward without a workspace: the library's static per-device scratch."""
    rc = lib().moe_forward_noalloc(C.byref(shape), C.byref(weights_struct(w)), _ptr(x), C.byref(r.struct()),
                                   _ptr(y), _stream(stream))
    _check(rc, "moe_forward_noalloc")


def _events(events):
    """torch.cuda.Event list -> hipEvent_t[N_STAGE_EVENTS] (or None)."""
    if events is None:
        return None
    assert len(events) == N_STAGE_EVENTS
    for ev in events:
        if ev.cuda_event == 0:  # torch creates the HIP event lazily
            ev.record()
    return (C.c_void_p * N_STAGE_EVENTS)(*[ev.cuda_event for ev in events])


def forward_stages(shape: Shape, w: dict, x: torch.Tensor, r: Routing, y: torch.Tensor, ws: torch.Tensor,
                   stages: int, events=None, stream=None):
    rc = lib().moe_forward_stages(C.byref(shape), C.byref(weights_struct(w)), _ptr(x), C.byref(r.struct()), _ptr(y),
                                  _ptr(ws), ws.numel(), stages, _events(events), _stream(stream))
    _check(rc, "moe_forward_stages")


def quantize_rows(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    act = {torch.float32: DTYPES["f32"], torch.bfloat16: DTYPES["bf16"]}[x.dtype]
    rc = lib().moe_quantize_rows(x.shape[0], x.shape[1], act, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream))
    _check(rc, "moe_quantize_rows")


def pack_weights(w: torch.Tensor, stream=None) -> torch.Tensor:
    """MOE_LAYOUT_TILED copy of a [n, rows, cols] (or [rows, cols]) weight tensor."""
    t = w if w.dim() == 3 else w.unsqueeze(0)
    n, rows, cols = t.shape
    out = torch.empty_like(w)
    rc = lib().moe_pack_weights(n, rows, cols * t.element_size(), _ptr(w), _ptr(out), _stream(stream))
    _check(rc, "moe_pack_weights")
    return out


def pack_weights_u4(codes: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, stream=None):
    """MOE_LAYOUT_TILED codes and group parameters of [n, rows, cols/2] (or
    [rows, cols/2]) 4-bit codes with [.., rows, cols/64] bf16 scales and biases."""
    t = codes if codes.dim() == 3 else codes.unsqueeze(0)
    n, rows, half = t.shape
    if scales.dtype != torch.bfloat16 or biases.dtype != torch.bfloat16:
        raise ValueError("moe: 4-bit group scales and biases must be bfloat16")
    if scales.shape != biases.shape or scales.numel() != n * rows * (2 * half // 64):
        raise ValueError("moe: 4-bit group parameters do not match the codes")
    out = torch.empty_like(codes)
    params = torch.empty(scales.numel() * 4, dtype=torch.uint8, device=codes.device)
    rc = lib().moe_pack_weights_u4(n, rows, 2 * half, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(out),
                                   _ptr(params), _stream(stream))
    _check(rc, "moe_pack_weights_u4")
    return out, params


def pack_router(w_router: torch.Tensor, stream=None) -> torch.Tensor:
    """The [E, d] fp32 router weights as moe_pack_router's three bf16 planes."""
    E, d = w_router.shape
    n = int(lib().moe_router_planes_bytes(E, d))
    if n == 0 or w_router.dtype != torch.float32:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_router_planes_bytes")
    out = torch.empty(n, dtype=torch.uint8, device=w_router.device)
    _check(lib().moe_pack_router(E, d, _ptr(w_router), _ptr(out), _stream(stream)), "moe_pack_router")
    return out


def pack_layer_weights(w: dict, stream=None) -> dict:
    """The weight dict with every expert matrix packed (scales, x untouched) and
    the router's packed planes added as w_router_planes.  4-bit weights
    (recognised by their biases b_*): codes and group parameters packed
    together, the parameters taking the scales' place."""
    out = dict(w)
    if w.get("w_router") is not None:
        out["w_router_planes"] = pack_router(w["w_router"], stream)
    if w.get("b_gate") is not None:
        for c, sc, b in (("w_gate", "s_gate", "b_gate"), ("w_up", "s_up", "b_up"), ("w_down", "s_down", "b_down"),
                         ("sh_gate", "ss_gate", "sb_gate"), ("sh_up", "ss_up", "sb_up"),
                         ("sh_down", "ss_down", "sb_down")):
            if w.get(c) is not None:
                out[c], out[sc] = pack_weights_u4(w[c], w[sc], w[b], stream)
            out.pop(b, None)
        return out
    for k in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        if w.get(k) is not None:
            out[k] = pack_weights(w[k], stream)
    return out


@dataclasses.dataclass
class RouteComparison:
    """Device results of moe_route_compare."""
    gap: torch.Tensor         # [T] float32: -1 where the expert sets agree
    sigma: torch.Tensor       # [1] float64
    n_disagree: torch.Tensor  # [1] int32
    max_gap: torch.Tensor     # [1] float32


class RouteCompare:
    """moe_route_compare with its output and workspace buffers allocated once
    for T tokens (each call is then a single ctypes call)."""

    def __init__(self, T: int, device="cuda"):
        self.T = int(T)
        self.out = RouteComparison(gap=torch.empty(max(self.T, 1), dtype=torch.float32, device=device),
                                   sigma=torch.empty(1, dtype=torch.float64, device=device),
                                   n_disagree=torch.empty(1, dtype=torch.int32, device=device),
                                   max_gap=torch.empty(1, dtype=torch.float32, device=device))
        self.ws = torch.empty(max(int(lib().moe_route_compare_workspace_bytes(self.T)), 256), dtype=torch.uint8,
                              device=device)

    def __call__(self, logits: torch.Tensor, ref_logits: torch.Tensor, idx: torch.Tensor, ref_idx: torch.Tensor,
                 sel_bias: torch.Tensor | None = None, stream=None) -> RouteComparison:
        T, E = logits.shape
        k = idx.shape[1]
        if T != self.T or ref_logits.shape != (T, E) or ref_idx.shape != (T, k):
            raise ValueError("moe_route_compare: mismatched shapes")
        o = self.out
        rc = lib().moe_route_compare(T, E, k, _ptr(logits), _ptr(ref_logits), _ptr(sel_bias), _ptr(idx),
                                     _ptr(ref_idx), _ptr(o.gap), _ptr(o.sigma), _ptr(o.n_disagree), _ptr(o.max_gap),
                                     _ptr(self.ws), self.ws.numel(), _stream(stream))
        _check(rc, "moe_route_compare")
        return o


def route_compare(logits, ref_logits, idx, ref_idx, sel_bias=None, stream=None) -> RouteComparison:
    return RouteCompare(logits.shape[0], logits.device)(logits, ref_logits, idx, ref_idx, sel_bias, stream)


def raw_call(name: str, *args):
    """Call an ABI function with raw ctypes arguments (host-side validation tests)."""
    return getattr(lib(), name)(*args)


class Bound:
    """One layer's arguments marshalled once (structs and pointers prebuilt), for
    launch loops where per-call Python overhead would show: each method is a
    single ctypes call."""

    def __init__(self, shape: Shape, w: dict, x: torch.Tensor, r: Routing, y: torch.Tensor, ws: torch.Tensor,
                 forced_idx: torch.Tensor | None = None, stream=None):
        self._keep = (w, x, r, y, ws, forced_idx)
        self.shape = shape
        self.w = weights_struct(w)
        self.r = r.struct()
        self.args = (C.byref(self.shape), C.byref(self.w), C.c_void_p(_ptr(x)))
        self.y = C.c_void_p(_ptr(y))
        self.ws = (C.c_void_p(_ptr(ws)), ws.numel())
        self.forced = C.c_void_p(_ptr(forced_idx)) if forced_idx is not None else None
        self.stream = _stream(stream)
        self.L = lib()

    def route(self):
        if self.forced is None:
            _check(self.L.moe_route(*self.args, C.byref(self.r), *self.ws, self.stream), "moe_route")
        else:
            _check(self.L.moe_route_forced(*self.args, self.forced, C.byref(self.r), *self.ws, self.stream),
                   "moe_route_forced")

    def forward(self, stages: int = STAGE_ALL, events=None):
        _check(self.L.moe_forward_stages(*self.args, C.byref(self.r), self.y, *self.ws, stages, _events(events),
                                         self.stream), "moe_forward_stages")
