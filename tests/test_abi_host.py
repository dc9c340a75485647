"""The C-ABI library loads, exports every function include/moe.h declares, and
rejects invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from mixture_experts_moe_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return moe.lib()


def header_functions(header="moe.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_]\w*\s*\**\s*(moe_\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_function():
    L = _lib()
    names = header_functions()
    assert set(names) == set(moe.ABI_FUNCTIONS), names
    for n in names:
        assert hasattr(L, n), n
    from mixture_experts_moe_amd import attn
    names = header_functions("moe_attn.h")
    assert set(names) == set(attn.ABI_FUNCTIONS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    _lib()
    for rc in (0, -1, -2, -3, -4, -5, -6, -7):
        assert moe.status_string(rc).startswith("MOE_")
    assert "unknown" in moe.status_string(7)


def test_workspace_bytes():
    _lib()
    s = moe.make_shape(32, 2048, 384, 6, 640, 640)
    n32 = moe.workspace_bytes(s)
    n2048 = moe.workspace_bytes(moe.make_shape(2048, 2048, 384, 6, 640, 640))
    assert 0 < n32 < n2048
    # the per-pair fp32 partials dominate: (P + T) * d * 4 bytes
    assert n2048 >= (2048 * 7) * 2048 * 4
    assert moe.workspace_bytes(moe.make_shape(0, 2048, 384, 6, 640, 640)) >= 0
    for bad in (moe.make_shape(32, 2048, 384, 9, 640, 640),      # k > 8
                moe.make_shape(32, 2048, 4, 6, 640, 640),        # k > E
                moe.make_shape(32, 2000, 384, 6, 640, 640),      # d not a multiple of 128
                moe.make_shape(32, 2048, 384, 6, 640, 640, act="f32", w="fp8"),
                moe.make_shape(32, 2048, 600, 6, 640, 640),      # E > 512
                moe.make_shape(-1, 2048, 384, 6, 640, 640)):
        assert moe.workspace_bytes(bad) == 0



@pytest.mark.parametrize("act,w,layout,d_max,f_max", [("f32", "f32", "rowmajor", 2560, 2560),
                                                       ("bf16", "bf16", "rowmajor", 4736, 4096),
                                                       ("bf16", "fp8", "rowmajor", 4608, 4096),
                                                       ("bf16", "fp8a16", "rowmajor", 4608, 4096),
                                                       ("bf16", "u4", "tiled", 4608, 4096)])
def test_largest_supported_widths(act, w, layout, d_max, f_max):
    """The widths the header states as the largest supported (one 16-row tile's
    activation and h rows in 160 KB of LDS) are accepted, one 128 step more is not."""
    _lib()
    ok = lambda d, F, Fs: moe.workspace_bytes(moe.make_shape(8, d, 16, 2, F, Fs, act, w, layout)) > 0
    assert ok(d_max, 128, 128) and not ok(d_max + 128, 128, 128)
    assert ok(256, f_max, 0) and not ok(256, f_max + 128, 0)
    assert ok(256, 128, f_max) and not ok(256, 128, f_max + 128)

FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below returns before launching


def _routing_struct(plan_bytes=1 << 40, **null):
    vals = {n: 0x2000 for n in moe._ROUTING_FIELDS}
    vals.update({k: None for k in null})
    return moe.RoutingStruct(*[vals[n] for n in moe._ROUTING_FIELDS], plan_bytes, None)


def _weights_struct(**null):
    vals = {n: 0x3000 for n in moe._WEIGHT_FIELDS}
    vals.update({k: None for k in null})
    return moe.Weights(*[vals[n] for n in moe._WEIGHT_FIELDS])


def _route(shape, ws_bytes=1 << 40, w=None, r=None, x=FAKE, ws=FAKE):
    L = _lib()
    w = w or _weights_struct()
    r = r or _routing_struct()
    return L.moe_route(C.byref(shape) if shape is not None else None, C.byref(w), x, C.byref(r), ws, ws_bytes, None)


def test_route_host_validation():
    good = moe.make_shape(32, 2048, 384, 6, 640, 640)
    assert _route(None) == moe.MOE_ERR_INVALID_ARG
    assert _route(moe.make_shape(32, 2048, 4, 6, 640, 640)) == moe.MOE_ERR_INVALID_ARG
    assert _route(moe.make_shape(32, 2048, 384, 9, 640, 640)) == moe.MOE_ERR_UNSUPPORTED
    assert _route(moe.make_shape(32, 2048, 384, 6, 640, 640, act="f32", w="bf16")) == moe.MOE_ERR_UNSUPPORTED
    assert _route(moe.make_shape(32, 2040, 384, 6, 640, 640)) == moe.MOE_ERR_UNSUPPORTED
    assert _route(good, w=_weights_struct(w_router=1)) == moe.MOE_ERR_INVALID_ARG
    assert _route(good, r=_routing_struct(perm=1)) == moe.MOE_ERR_INVALID_ARG
    assert _route(good, r=_routing_struct(status=1)) == moe.MOE_ERR_INVALID_ARG
    assert _route(good, r=_routing_struct(plan=1)) == moe.MOE_ERR_INVALID_ARG
    assert _route(good, x=None) == moe.MOE_ERR_INVALID_ARG
    assert _route(good, ws_bytes=moe.workspace_bytes(good) - 1) == moe.MOE_ERR_WORKSPACE
    assert _route(good, ws=None) == moe.MOE_ERR_INVALID_ARG
    # T = 0: nothing to do, nothing enqueued, and the logits pointer may be NULL
    assert _route(moe.make_shape(0, 2048, 384, 6, 640, 640), ws_bytes=0, ws=None,
                  r=_routing_struct(logits=1)) == moe.MOE_OK


def test_route_forced_requires_ids():
    L = _lib()
    s = moe.make_shape(32, 2048, 384, 6, 640, 640)
    w, r = _weights_struct(), _routing_struct()
    assert L.moe_route_forced(C.byref(s), C.byref(w), FAKE, None, C.byref(r), FAKE, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    s0 = moe.make_shape(0, 2048, 384, 6, 640, 640)
    assert L.moe_route_forced(C.byref(s0), C.byref(w), FAKE, FAKE, C.byref(r), None, 0, None) == moe.MOE_OK


def _forward(shape, w=None, r=None, y=FAKE, ws_bytes=1 << 40):
    L = _lib()
    w = w or _weights_struct()
    r = r or _routing_struct()
    return L.moe_forward(C.byref(shape), C.byref(w), FAKE, C.byref(r), y, FAKE, ws_bytes, None)


def test_undersized_plan_rejected():
    """The plan buffer's size travels with it (moe_routing.plan_bytes): one byte
    short of moe_plan_bytes() is rejected on the host by routing and forward,
    before any launch; T = 0 needs no plan."""
    for s in (moe.make_shape(32, 2048, 384, 6, 640, 640), moe.make_shape(2048, 2048, 384, 6, 640, 640),
              moe.make_shape(64, 256, 16, 2, 128, 128, act="f32", w="f32")):
        n = moe.plan_bytes(s)
        assert n > 0
        assert _route(s, r=_routing_struct(plan_bytes=n - 1)) == moe.MOE_ERR_WORKSPACE
        assert _forward(s, r=_routing_struct(plan_bytes=n - 1)) == moe.MOE_ERR_WORKSPACE
        assert _route(s, r=_routing_struct(plan_bytes=0)) == moe.MOE_ERR_WORKSPACE
    s0 = moe.make_shape(0, 2048, 384, 6, 640, 640)
    assert _route(s0, ws_bytes=0, ws=None, r=_routing_struct(plan_bytes=0)) == moe.MOE_OK
    assert _forward(s0, r=_routing_struct(plan_bytes=0)) == moe.MOE_OK


def test_forward_stage_bits():
    """moe_forward_stages takes the three stage bits and the error-path test bit;
    any other bit is rejected before any launch."""
    L = _lib()
    s = moe.make_shape(0, 2048, 384, 6, 640, 640)
    w, r = _weights_struct(), _routing_struct()
    call = lambda bits: L.moe_forward_stages(C.byref(s), C.byref(w), FAKE, C.byref(r), FAKE, FAKE, 1 << 40, bits,
                                             None, None)
    assert call(moe.STAGE_ALL | moe.FORWARD_TEST_WAIT_TIMEOUT) == moe.MOE_OK
    for bad in (8, 0x80, 0x200, 1 << 31):
        assert call(moe.STAGE_ALL | bad) == moe.MOE_ERR_INVALID_ARG


def test_forward_noalloc_host_validation():
    """moe_forward_noalloc's host checks, none of which touches a GPU: the
    scratch the shape needs against MOE_NOALLOC_SCRATCH_BYTES (the 2048 / 640 /
    top-6 FP8 layer fits up to T = 1083), then the plan size; T = 0 is a no-op;
    missing pointers as for moe_forward."""
    L = _lib()
    w = _weights_struct()

    def call(shape, r=None, y=FAKE):
        r = r or _routing_struct()
        return L.moe_forward_noalloc(C.byref(shape), C.byref(w), FAKE, C.byref(r), y, None)

    assert call(moe.make_shape(1084, 2048, 384, 6, 640, 640)) == moe.MOE_ERR_SCRATCH_LIMIT
    assert call(moe.make_shape(8192, 2048, 384, 6, 640, 640)) == moe.MOE_ERR_SCRATCH_LIMIT
    fits = moe.make_shape(1083, 2048, 384, 6, 640, 640)
    assert call(fits, r=_routing_struct(plan_bytes=moe.plan_bytes(fits) - 1)) == moe.MOE_ERR_WORKSPACE
    assert call(fits, y=None) == moe.MOE_ERR_INVALID_ARG
    assert call(moe.make_shape(0, 2048, 384, 6, 640, 640)) == moe.MOE_OK
    assert call(moe.make_shape(32, 2048, 384, 9, 640, 640)) == moe.MOE_ERR_UNSUPPORTED


def test_forward_host_validation():
    fp8 = moe.make_shape(32, 2048, 384, 6, 640, 640)
    assert _forward(fp8, r=_routing_struct(plan=1)) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, w=_weights_struct(s_gate=1)) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, w=_weights_struct(ss_down=1)) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, w=_weights_struct(sh_up=1)) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, r=_routing_struct(topk_w=1)) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, y=None) == moe.MOE_ERR_INVALID_ARG
    assert _forward(fp8, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    # no shared expert: the shared pointers are not needed
    noshared = moe.make_shape(0, 2048, 384, 6, 640, 0)
    assert _forward(noshared, w=_weights_struct(sh_gate=1, sh_up=1, sh_down=1, ss_gate=1, ss_up=1, ss_down=1)) \
        == moe.MOE_OK
    # bf16 weights need no scales
    bf = moe.make_shape(0, 2048, 384, 6, 640, 640, act="bf16", w="bf16")
    assert _forward(bf, w=_weights_struct(s_gate=1, s_up=1, s_down=1, ss_gate=1, ss_up=1, ss_down=1)) == moe.MOE_OK


def test_quantize_rows_host_validation():
    L = _lib()
    assert L.moe_quantize_rows(4, 100, 1, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_rows(4, 128, 2, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(-1, 128, 1, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(0, 128, 1, None, None, None, None) == moe.MOE_OK
    assert L.moe_quantize_rows(4, 128, 1, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    odd = C.c_void_p(0x1008)  # 8-byte but not 16-byte aligned
    assert L.moe_quantize_rows(4, 128, 1, odd, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows(4, 128, 1, FAKE, odd, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def test_misaligned_activations_rejected():
    good = moe.make_shape(32, 2048, 384, 6, 640, 640)
    odd = C.c_void_p(0x1008)
    assert _route(good, x=odd) == moe.MOE_ERR_INVALID_ARG
    L = _lib()
    w, r = _weights_struct(), _routing_struct()
    for x, y in ((odd, FAKE), (FAKE, odd)):
        assert L.moe_forward(C.byref(good), C.byref(w), x, C.byref(r), y, FAKE, 1 << 40, None) == \
            moe.MOE_ERR_INVALID_ARG


def test_misaligned_weights_rejected():
    """Expert, shared-expert and router weights are read 16 bytes per lane: a
    pointer that is 8- but not 16-byte aligned is rejected before any launch
    (the shared pointers only when the layer has a shared expert)."""
    good = moe.make_shape(32, 2048, 384, 6, 640, 640)
    for field in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        w = _weights_struct()
        setattr(w, field, 0x3008)
        assert _forward(good, w=w) == moe.MOE_ERR_INVALID_ARG, field
    w = _weights_struct()
    w.w_router = 0x3008
    assert _route(good, w=w) == moe.MOE_ERR_INVALID_ARG
    f32 = moe.make_shape(64, 256, 16, 2, 128, 128, act="f32", w="f32")
    w = _weights_struct()
    w.w_down = 0x3004
    assert _forward(f32, w=w) == moe.MOE_ERR_INVALID_ARG
    noshared = moe.make_shape(0, 2048, 384, 6, 640, 0)
    w = _weights_struct()
    w.sh_gate = 0x3008
    assert _forward(noshared, w=w) == moe.MOE_OK  # T = 0, and no shared expert to check


def test_pack_weights_host_validation():
    L = _lib()
    buf = (C.c_uint8 * 8192)()
    a = C.cast(buf, C.c_void_p)
    assert L.moe_pack_weights(1, 16, 100, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED    # row_bytes % 128
    assert L.moe_pack_weights(1, 24, 128, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED    # rows % 16
    assert L.moe_pack_weights(-1, 16, 128, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(1, 0, 128, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(1, 16, 128, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(0, 16, 128, None, None, None) == moe.MOE_OK
    # 2 x 16 x 128 bytes = 4 KB: a and a+2 KB overlap (rejected before any launch)
    assert L.moe_pack_weights(2, 16, 128, a, C.c_void_p(C.addressof(buf) + 2048), None) == moe.MOE_ERR_INVALID_ARG


def test_pack_router_host_validation():
    L = _lib()
    assert L.moe_router_planes_bytes(384, 2048) == 24 * 64 * 3 * 1024
    assert L.moe_router_planes_bytes(17, 256) == 2 * 8 * 3 * 1024      # experts rounded up to 16
    for E, d in ((0, 2048), (513, 2048), (384, 2000), (384, 0)):
        assert L.moe_router_planes_bytes(E, d) == 0
        assert L.moe_pack_router(E, d, FAKE, C.c_void_p(0x100000), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_router(384, 2048, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_router(384, 2048, FAKE, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_router(384, 2048, C.c_void_p(0x1008), C.c_void_p(0x10000000), None) == moe.MOE_ERR_INVALID_ARG
    # w_router [16, 128] fp32 = 8 KB at a; the 12 KB of planes at a + 4 KB overlap it
    assert L.moe_pack_router(16, 128, C.c_void_p(0x100000), C.c_void_p(0x101000), None) == moe.MOE_ERR_INVALID_ARG
    # a routing call rejects misaligned packed planes before any launch
    good = moe.make_shape(2048, 2048, 384, 6, 640, 640)
    w = _weights_struct()
    w.w_router_planes = 0x3008
    assert _route(good, w=w) == moe.MOE_ERR_INVALID_ARG


def test_layout_field_validation():
    _lib()
    assert moe.workspace_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640, layout="tiled")) > 0
    bad = moe.make_shape(32, 2048, 384, 6, 640, 640)
    bad.w_layout = 5
    assert moe.workspace_bytes(bad) == 0
    assert _forward(bad) == moe.MOE_ERR_INVALID_ARG
    f32 = moe.make_shape(32, 2048, 384, 6, 640, 640, act="f32", w="f32", layout="tiled")
    assert _forward(f32) == moe.MOE_ERR_UNSUPPORTED


def test_plan_bytes():
    _lib()
    s32 = moe.make_shape(32, 2048, 384, 6, 640, 640)
    s2k = moe.make_shape(2048, 2048, 384, 6, 640, 640)
    n32, n2k = moe.plan_bytes(s32), moe.plan_bytes(s2k)
    # at least the E4M3 activations, their scales and the per-row info
    assert n32 >= 32 * 2048 + 32 * 16 * 4 + (32 * 7) * 12
    assert n2k >= 2048 * 2048 + 2048 * 16 * 4 + (2048 * 7) * 12 and n2k > n32
    bf = moe.make_shape(32, 2048, 384, 6, 640, 640, act="bf16", w="bf16")
    assert moe.plan_bytes(bf) < n32  # no activation codes with bf16 weights
    assert moe.plan_bytes(moe.make_shape(32, 2048, 384, 9, 640, 640)) == 0


def test_w8a16_shape_and_scales():
    """(bf16 activations, FP8 weights as W8A16) is a supported pair; like the FP8
    mode it needs the block scales, and with no activation codes its workspace
    and plan are those of a layer whose h is bf16."""
    _lib()
    a16 = moe.make_shape(32, 2048, 384, 6, 640, 640, act="bf16", w="fp8a16")
    assert moe.workspace_bytes(a16) > moe.workspace_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640))
    assert moe.workspace_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640, act="f32", w="fp8a16")) == 0
    assert moe.plan_bytes(a16) < moe.plan_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640))  # no x codes
    assert moe.plan_bytes(a16) > 0
    L = _lib()
    r = _routing_struct()
    y = FAKE
    for null in ("s_gate", "s_up", "s_down", "ss_gate"):
        w = _weights_struct(**{null: None})
        rc = L.moe_forward(C.byref(a16), C.byref(w), FAKE, C.byref(r), y, FAKE, 1 << 40, None)
        assert rc == moe.MOE_ERR_INVALID_ARG, null


def test_u4_shape_layout_and_params():
    """(bf16 activations, 4-bit weights) is supported in the tiled layout only;
    the group parameters are required; moe_pack_weights_u4 checks its sizes and
    overlaps before any launch."""
    L = _lib()
    u4 = moe.make_shape(32, 2048, 384, 6, 640, 640, act="bf16", w="u4", layout="tiled")
    assert moe.workspace_bytes(u4) > 0 and moe.plan_bytes(u4) > 0
    assert moe.workspace_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640, act="bf16", w="u4")) == 0  # row-major
    assert moe.workspace_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640, act="f32", w="u4", layout="tiled")) == 0
    assert moe.plan_bytes(u4) < moe.plan_bytes(moe.make_shape(32, 2048, 384, 6, 640, 640))  # no x codes
    r = _routing_struct()
    for null in ("s_gate", "s_up", "s_down", "ss_down"):
        w = _weights_struct(**{null: None})
        rc = L.moe_forward(C.byref(u4), C.byref(w), FAKE, C.byref(r), FAKE, FAKE, 1 << 40, None)
        assert rc == moe.MOE_ERR_INVALID_ARG, null
    P = L.moe_pack_weights_u4
    assert P(1, 24, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED  # rows % 16
    assert P(1, 16, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED   # cols % 128
    assert P(-1, 16, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert P(1, 16, 128, FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert P(0, 16, 128, None, None, None, None, None, None) == moe.MOE_OK
    buf = (C.c_uint8 * 8192)()
    a = C.addressof(buf)
    # 16 x 128 codes = 1 KB at a; params 512 B placed inside the codes' output
    assert P(1, 16, 128, FAKE, FAKE, FAKE, C.c_void_p(a), C.c_void_p(a + 512), None) == moe.MOE_ERR_INVALID_ARG
    assert P(1, 16, 128, C.c_void_p(a), FAKE, FAKE, C.c_void_p(a + 256), C.c_void_p(a + 4096), None) == \
        moe.MOE_ERR_INVALID_ARG


def test_route_compare_host_validation():
    L = _lib()
    f = L.moe_route_compare
    ws = L.moe_route_compare_workspace_bytes(100)
    assert ws >= 100 * 20 and L.moe_route_compare_workspace_bytes(-1) == 0
    args = lambda T, E, k, **kw: [T, E, k] + [kw.get(n, FAKE) for n in (
        "lg", "rl", "bias", "idx", "ridx", "gap", "sigma", "nd", "mg", "ws")] + [kw.get("wsb", 1 << 30), None]
    assert f(*args(100, 8, 9)) == moe.MOE_ERR_INVALID_ARG           # k > E
    assert f(*args(100, 16, 9)) == moe.MOE_ERR_UNSUPPORTED          # k > 8
    assert f(*args(-1, 8, 2)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(100, 8, 2, lg=None)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(100, 8, 2, sigma=None)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(100, 8, 2, wsb=ws - 1)) == moe.MOE_ERR_WORKSPACE
    assert f(*args(0, 8, 2, ws=None)) == moe.MOE_OK
    assert f(*args(100, 8, 2, ws=None)) == moe.MOE_ERR_INVALID_ARG


def test_attention_host_validation():
    from mixture_experts_moe_amd import attn
    L = attn.lib()
    sh = attn.AttnShape(16, 4, 128, 513)
    call = lambda shape, Tq, Tk, q0, **kw: L.moe_attention(
        C.byref(shape), Tq, Tk, q0, kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE), kw.get("o", FAKE),
        kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert call(sh, 10, 5, 0) == attn.ERR_INVALID_ARG            # q_pos0 + Tq > Tk
    assert call(sh, 4, 10, 7) == attn.ERR_INVALID_ARG
    assert call(attn.AttnShape(16, 3, 128, 0), 4, 10, 0) == attn.ERR_INVALID_ARG  # Hkv does not divide Hq
    assert call(attn.AttnShape(16, 4, 64, 0), 4, 10, 0) == attn.ERR_UNSUPPORTED   # head_dim
    assert call(attn.AttnShape(12, 1, 128, 0), 4, 10, 0) == attn.ERR_UNSUPPORTED  # group of 12 does not divide 64
    assert call(attn.AttnShape(16, 4, 128, -1), 4, 10, 0) == attn.ERR_INVALID_ARG
    assert call(sh, 4, 10, 0, q=None) == attn.ERR_INVALID_ARG
    assert call(sh, 0, 10, 0, q=None, ws=None) == attn.OK
    # a decode call splits the keys: it needs a workspace
    need = attn.workspace_bytes(attn.AttnShape(16, 4, 128, 0), 1, 32768, 32767)
    assert need > 0
    assert call(attn.AttnShape(16, 4, 128, 0), 1, 32768, 32767, wsb=need - 1) == attn.ERR_WORKSPACE
    assert attn.workspace_bytes(sh, 10, 5, 0) == 0
    R = L.moe_rope
    assert R(4, 2, 7, 0, 10000.0, FAKE, None) == attn.ERR_INVALID_ARG   # odd head_dim
    assert R(4, 2, 8, 0, 1.0, FAKE, None) == attn.ERR_INVALID_ARG       # theta <= 1
    assert R(4, 2, 8, -1, 10000.0, FAKE, None) == attn.ERR_INVALID_ARG
    assert R(0, 2, 8, 0, 10000.0, None, None) == attn.OK
    assert R(4, 2, 8, 0, 10000.0, None, None) == attn.ERR_INVALID_ARG


def test_missing_library_fails_loudly():
    """Without the built HIP library the bindings raise (no fallback path): a
    fresh interpreter with the library path pointed at a file that does not exist."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from mixture_experts_moe_amd import moe, attn\n"
            "moe.LIB_PATH = '/nonexistent/libmoe.so'  # attn loads through moe\n"
            "for f in (moe.lib, attn.lib):\n"
            "    try:\n"
            "        f(); print('loaded')\n"
            "    except ImportError as e:\n"
            "        print('ImportError', 'is not built' in str(e))\n") % root
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.stdout.split() == ["ImportError", "True", "ImportError", "True"], r.stdout + r.stderr
