"""The router weights packed once per layer (moe_pack_router): the packed planes
against their documented definition, rebuilt on the host, and routing from
them against routing that splits the fp32 weights in every call, bit for bit.

The split is the exact three-way one (w = hi + mid + lo, each a bf16 rounding
to nearest even of what the previous terms leave): the router stays in
float32 ("We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said
No.", part 3 of "Taking it apart")."""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import moe, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def host_planes(w: np.ndarray) -> np.ndarray:
    """The packed bytes of moe_pack_router for w [E, d], built on the host from
    the header's layout: fragment (et, ks, p) at 1024*((et*(d/32) + ks)*3 + p),
    lane l's 8 bf16 at 16*l holding expert 16*et + l%16, K = 32*ks + 8*(l/16) + j."""
    E, d = w.shape
    n_et, nks = (E + 15) // 16, d // 32
    wp = np.zeros((16 * n_et, d), np.float32)
    wp[:E] = w
    hi = synth.bf16_bits(wp)
    r1 = wp - synth.bf16_bits_to_f32(hi)
    mid = synth.bf16_bits(r1)
    r2 = r1 - synth.bf16_bits_to_f32(mid)
    lo = synth.bf16_bits(r2)
    out = np.empty((n_et, nks, 3, 64, 8), np.uint16)
    for p, pl in enumerate((hi, mid, lo)):
        # [et*16 + r][ks*32 + g*8 + j] -> [et][ks][g][r][j]: lane l = 16*g + r
        v = pl.reshape(n_et, 16, nks, 4, 8).transpose(0, 2, 3, 1, 4).reshape(n_et, nks, 64, 8)
        out[:, :, p] = v
    return out.reshape(-1).view(np.uint8)


@pytest.mark.parametrize("E,d", [(40, 256), (384, 2048)])
def test_pack_router_layout(E, d):
    """The planes equal the host-built split and layout byte for byte, and the
    three terms add back to every fp32 weight exactly."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((E, d)) * 0.05).astype(np.float32)
    w[0, :8] = [0.0, -0.0, 1e-30, -3.0, 65504.0, 1.0 + 2.0 ** -23, np.float32(2.0 ** -126), 0.1]
    say(f"pack_router E={E} d={d}")
    got = moe.pack_router(torch.from_numpy(w).to(DEV)).cpu().numpy()
    assert got.size == int(moe.lib().moe_router_planes_bytes(E, d))
    want = host_planes(w)
    assert np.array_equal(got, want)
    planes = want.view(np.uint16).reshape((E + 15) // 16, d // 32, 3, 64, 8)
    terms = [synth.bf16_bits_to_f32(planes[:, :, p]).astype(np.float64)
             .reshape(-1, d // 32, 4, 16, 8).transpose(0, 3, 1, 2, 4).reshape(-1, d)[:E] for p in range(3)]
    assert np.array_equal(terms[0] + terms[1] + terms[2], w.astype(np.float64))


def _route(shape, w, x):
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    moe.route(shape, w, x, r, ws)
    torch.cuda.synchronize()
    assert r.status.item() == moe.MOE_OK
    return r.logits.cpu().numpy(), r.topk_idx.cpu().numpy(), r.topk_w.cpu().numpy()


@pytest.mark.parametrize("case,T", [("prefill_t2048", 171), ("prefill_t2048", 300), ("prefill_t2048", 2048),
                                    ("skew_t8192", 4095), ("skew_t8192", 4096), ("skew_t8192", 8192),
                                    ("skew_t8192", 4133)])
def test_planes_route_bitwise(case, T):
    """Routing with the packed planes gives the logits, ids and weights of
    routing from the fp32 weights, bit for bit (both short- and long-batch
    block shapes, ragged token tiles)."""
    inp = synth.make_inputs(case, T=T)
    s = inp["shape"]
    dev = synth.to_device({k: inp[k] for k in ("x", "w_router", "sel_bias") if inp.get(k) is not None}, DEV)
    shape = moe.shape_of(s)
    say(f"{case} T={T}: planes vs fp32 router weights")
    a = _route(shape, dev, dev["x"])
    dp = dict(dev, w_router_planes=moe.pack_router(dev["w_router"]))
    b = _route(shape, dp, dp["x"])
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


@pytest.mark.parametrize("E", [100, 17])
def test_planes_route_ragged_experts(E):
    """Expert counts that leave the last 64-expert block (and 16-expert tile)
    part empty: the planes path still matches the fp32-weight path bitwise."""
    inp = synth.make_inputs("prefill_t2048", T=1500)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(inp["w_router"][:E])).to(DEV)
    shape = moe.make_shape(1500, 2048, E, 6, 640, 640, act="bf16", w="fp8")
    say(f"T=1500 E={E}: planes vs fp32 router weights")
    a = _route(shape, {"w_router": w}, x)
    b = _route(shape, {"w_router": w, "w_router_planes": moe.pack_router(w)}, x)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])


def test_planes_batch_invariance():
    """The 32 decode tokens alone (K-split router from the fp32 weights) and as
    the first rows of an 8192-token batch routed from the planes: the same
    logits, ids and weights, bit for bit."""
    small = synth.make_inputs("decode_t32")
    big = synth.make_inputs("prefill_t2048", T=8192)
    xb = big["x"].copy()
    xb[:32] = small["x"]
    ds = synth.to_device({"x": small["x"], "w_router": small["w_router"]}, DEV)
    db = synth.to_device({"x": xb, "w_router": big["w_router"]}, DEV)
    db["w_router_planes"] = moe.pack_router(db["w_router"])
    say("decode_t32 alone vs inside T=8192 routed from the planes")
    a = _route(moe.shape_of(small["shape"]), ds, ds["x"])
    b = _route(moe.shape_of(big["shape"], T=8192), db, db["x"])
    assert np.array_equal(a[0].view(np.uint32), b[0][:32].view(np.uint32))
    assert np.array_equal(a[1], b[1][:32])
    assert np.array_equal(a[2].view(np.uint32), b[2][:32].view(np.uint32))
