"""moe_forward_noalloc (the forward without a workspace, for callers that
cannot allocate) against moe_forward, through the C ABI: bitwise the same
output on three calls in a row on one device, each smaller than the one
before (a 1000-token batch in 32-row tiles and separate expert launches, a
300-token and the 32-token decode batch in the one-launch expert kernel), so
the shared static scratch is reused with stale contents from a larger call.
The bar is bitwise equality with moe_forward (the same kernels on the same
inputs), stronger than the oracle bar both already meet."""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import moe, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def test_forward_noalloc_matches_forward_on_shrinking_calls():
    weights = None
    for T in (1000, 300, 32):
        inp = synth.make_inputs("prefill_t2048" if T > 32 else "decode_t32", T=T)
        s = inp["shape"]
        shape = moe.shape_of(s)
        if weights is None:  # both workloads share one layer: upload its weights once
            weights = synth.to_device({k: v for k, v in inp.items() if k not in ("x", "shape")}, DEV)
        dev = dict(weights, x=synth.to_device({"x": inp["x"]}, DEV)["x"])
        say(f"moe_forward_noalloc T={T} ({T * s.k} pairs, scratch limit {moe.NOALLOC_SCRATCH_BYTES} B)")
        r = moe.alloc_routing(shape, DEV)
        ws = moe.alloc_workspace(shape, DEV)
        y_ref = torch.empty((T, s.d), dtype=torch.bfloat16, device=DEV)
        y = torch.full((T, s.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        moe.route(shape, dev, dev["x"], r, ws)
        moe.forward(shape, dev, dev["x"], r, y_ref, ws)
        moe.forward_noalloc(shape, dev, dev["x"], r, y)
        torch.cuda.synchronize()
        assert r.status.item() == moe.MOE_OK and r.forward_status.item() == moe.MOE_OK
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"T={T}: differs from moe_forward"
        assert np.isfinite(y.float().cpu().numpy()).all()
    # one token past the limit is refused on the host, before any launch
    big = moe.make_shape(1084, 2048, 384, 6, 640, 640)
    r = moe.alloc_routing(moe.make_shape(32, 2048, 384, 6, 640, 640), DEV)
    r.plan = torch.empty(moe.plan_bytes(big), dtype=torch.uint8, device=DEV)
    y = torch.empty((1084, 2048), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(big, dev, torch.empty((1084, 2048), dtype=torch.bfloat16, device=DEV), r, y)
    assert e.value.rc == moe.MOE_ERR_SCRATCH_LIMIT
