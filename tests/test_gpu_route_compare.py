"""Routing compared as a distribution (moe_route_compare) on the GPU, through
the C ABI, against the oracle's comparison on the same inputs.

The check is the third part of what "We Ported Aleph Alpha's Kolibri to a
MacBook. Our Own Gate Said No." proposes (section "Taking it apart"), with the
sigma and margin of "We Stopped the Kolibri Benchmark Before Scoring One
Answer" (section "The gate, forced").  Bars: disagreement flags and counts
exact; sigma within 1e-12 relative (both sum in double, in different orders);
gaps within 1e-6 relative.  Cases:

  * the hand-worked examples of the oracle's pins;
  * the library's free routing of a 2048-token prefill against a router whose
    summation order depends on the batch shape (torch's fp32 matmul, over the
    whole batch and in chunks of 64), with and without a selection bias;
  * the 8192-token skewed batch (the bench's size), and a single token;
  * repeatability: the same call twice gives the same bits.
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import moe, synth
from oracle import moe_oracle as O

from test_gpu_parity import DEV, gpu_inputs, say

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(DEV)


def _check(logits, ref_logits, idx, ref_idx, bias=None):
    c = moe.route_compare(_dev(logits, np.float32), _dev(ref_logits, np.float32), _dev(idx, np.int32),
                          _dev(ref_idx, np.int32), None if bias is None else _dev(bias, np.float32))
    torch.cuda.synchronize()
    gap_ref, sigma_ref, nd_ref, mg_ref = O.route_compare(logits, ref_logits, idx, ref_idx, bias)
    gap = c.gap.cpu().numpy()[: len(gap_ref)]
    sigma, nd, mg = c.sigma.item(), c.n_disagree.item(), c.max_gap.item()
    say(f"  T={len(gap_ref)}: sigma {sigma:.6g}, {nd} disagreeing tokens, largest gap {mg:.4g}")
    assert nd == nd_ref
    assert np.array_equal(gap < 0, gap_ref < 0)
    assert abs(sigma - sigma_ref) <= 1e-12 * max(sigma_ref, 1e-300)
    d = gap_ref >= 0
    def close(a, b):  # equal (which also covers +inf), else within 1e-6 relative
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        fin = np.isfinite(a) & np.isfinite(b)
        rel = np.zeros_like(a)
        np.subtract(a, b, out=rel, where=fin)
        return (a == b) | (fin & (np.abs(rel) <= 1e-6 * np.abs(b)))
    assert np.all(close(gap[d], gap_ref[d]))
    assert np.all(gap[~d] == -1.0)
    assert close(np.float32(mg), np.float32(mg_ref))
    return c


def test_compare_worked_examples():
    ref = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -2.0], [0.0, 3.0, 2.5, 2.25, 1.0, 0.0],
                    [1.0, 1.0, 1.0, 1.0, 1.0, 1.0], [5.0, 4.0, 0.0, -1.0, 3.0, 2.0]], np.float32)
    oth = ref.copy()
    oth[1, 3] += 0.5
    oth[3, 4] += 1.5
    oth[3, 0] -= 2.0
    say("moe_route_compare: hand-worked examples")
    _check(oth, ref, np.array([[1, 0], [1, 3], [0, 1], [4, 1]]), np.array([[0, 1], [1, 2], [0, 1], [0, 1]]))
    _check(ref, ref, np.array([[0, 1]] * 4), np.array([[1, 0]] * 4))  # identical: sigma 0, no disagreement
    ref1 = np.array([[1.0, 0.9, 0.8, 0.0, 0.1]], np.float32)
    oth1 = ref1.copy()
    oth1[0, 3] -= 0.5
    _check(oth1, ref1, np.array([[0, 1]]), np.array([[0, 3]]), bias=np.array([0, 0, 0, 1.0, 0], np.float32))
    # sigma 0 with a positive margin (ids given, not recomputed): gap +inf
    _check(ref1, ref1, np.array([[0, 1]]), np.array([[0, 3]]), bias=np.array([0, 0, 0, 1.0, 0], np.float32))


def _torch_router(x_bf16, w_router, k, bias=None, chunk=None):
    """A batch-shape-dependent fp32 router: torch matmul over the batch or in
    chunks, ids by a stable sort (lowest index first among equal scores)."""
    xf = x_bf16.float()
    W = w_router.t()
    logits = xf @ W if chunk is None else torch.cat([xf[i:i + chunk] @ W for i in range(0, xf.shape[0], chunk)])
    s = logits if bias is None else logits + bias
    ids = torch.sort(-s, dim=1, stable=True).indices[:, :k].to(torch.int32)
    return logits.contiguous(), ids.contiguous()


@pytest.mark.parametrize("case,chunk", [("prefill_t2048", None), ("prefill_t2048", 64), ("skew_t8192", None)])
def test_compare_library_routing_against_torch_router(case, chunk):
    inp = synth.make_inputs(case)
    s = inp["shape"]
    dev = gpu_inputs(inp)
    shape = moe.shape_of(s)
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    moe.route(shape, dev, dev["x"], r, ws)
    bias = dev.get("sel_bias")
    tl, ti = _torch_router(dev["x"], dev["w_router"], s.k, bias, chunk)
    torch.cuda.synchronize()
    say(f"{case}: library free routing vs torch fp32 router (chunk {chunk})")
    np_bias = None if bias is None else bias.cpu().numpy()
    c = _check(r.logits.cpu().numpy(), tl.cpu().numpy(), r.topk_idx.cpu().numpy(), ti.cpu().numpy(), np_bias)
    # the same call again: the same bits
    c2 = moe.route_compare(r.logits, tl, r.topk_idx, ti, bias)
    torch.cuda.synchronize()
    assert c2.sigma.item() == c.sigma.item() and c2.n_disagree.item() == c.n_disagree.item()


def test_compare_single_token_and_k1():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal((1, 384)).astype(np.float32)
    oth = (ref + 1e-3 * rng.standard_normal((1, 384))).astype(np.float32)
    say("moe_route_compare: T=1, k=1")
    _check(oth, ref, np.array([[int(np.argmax(oth))]]), np.array([[int(np.argmax(ref))]]))
    _check(oth, ref, np.array([[7]]), np.array([[int(np.argmax(ref))]]))
