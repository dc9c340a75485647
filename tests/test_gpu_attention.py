"""The attention ops next to the layer on the GPU (moe_rope, moe_attention),
through the C ABI, against the attention oracle on the same seeded inputs.

Layout from "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said
No." (section "The gate"): 513-token sliding-window layers with rotary position
encoding, whole-context layers without.  Shapes not on the pages: 16 query
heads, 4 key/value heads, head_dim 128, theta 10000.

Bars (written here):
  * RoPE: the oracle rotates in double, the kernel reduces the angle in double
    and takes cos, sin and the rotation in fp32, whose absolute error is below
    2^-21 (|x_j| + |x_{j+D/2}|) (one rounding each for sin or cos, the two
    products and the sum); both round once to bf16.  Bar per element:
    |x - x_ref| <= one bf16 ulp of x_ref + 2^-20 (|x_j| + |x_{j+D/2}|); and as a
    guard against a systematic drift, at most a share 2^-12 of the n elements
    differ at all (near-tie differences run at about 1e-4 of them), with a
    floor of 4 elements for samples of fewer than 2^14 elements, where the
    share allows none;
  * attention, elementwise: |o - o_ref| <= 2^-8 |o_ref| + 2^-12 RMS(o_ref).
    The first term is the bf16 rounding of the output (half an ulp, 2^-8
    relative); the second covers the fp32 scores, exponentials and sums and the
    probabilities' two-part bf16 form (about 2^-16 relative each);
  * the window boundary, on uniform attention: a marker at p - 512 counts 1/513
    (to bf16), markers at p - 513 and p + 1 count exactly nothing.
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import attn, synth
from oracle import attn_oracle as A

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W = 513
THETA = 10000.0


def say(*a):
    print(*a, flush=True)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rand(rng, shape, scale=1.0):
    return synth.bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("T,H,D,pos0", [(64, 20, 128, 1000), (33, 4, 64, 0), (8, 16, 128, 100000),
                                        (5, 3, 256, 1 << 20),
                                        (7, 3, 36, 17)])  # D/2 not a multiple of 4: one pair per step
def test_rope_matches_oracle(T, H, D, pos0):
    rng = np.random.default_rng(T + D)
    x = _rand(rng, (T, H, D))
    say(f"moe_rope T={T} H={H} D={D} pos0={pos0}")
    g = _bits(attn.rope_(_dev_bf16(x), pos0, THETA))
    torch.cuda.synchronize()
    ref = A.rope(x, pos0, THETA)
    gf, rf, xf = (synth.bf16_bits_to_f32(a).astype(np.float64) for a in (g, ref, x))
    half = D // 2
    pair = np.abs(xf[..., :half]) + np.abs(xf[..., half:])
    pair = np.concatenate([pair, pair], axis=-1)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rf), 1e-38))) - 7)
    bound = ulp + 2.0 ** -20 * pair
    diff = np.abs(gf - rf)
    say(f"  elements differing: {(diff != 0).sum()} of {diff.size}; worst diff / bound {np.max(diff / bound):.3f}")
    assert np.all(diff <= bound) and (diff != 0).sum() <= max(4, diff.size * 2.0 ** -12)


def _check_attention(Hq, Hkv, window, Tq, Tk, q_pos0, rows=None, seed=0):
    rng = np.random.default_rng(seed)
    q = _rand(rng, (Tq, Hq, 128))
    k = _rand(rng, (Tk, Hkv, 128))
    v = _rand(rng, (Tk, Hkv, 128))
    shape = attn.AttnShape(Hq, Hkv, 128, window)
    say(f"moe_attention Hq={Hq} Hkv={Hkv} window={window} Tq={Tq} Tk={Tk} q_pos0={q_pos0} "
        f"(workspace {attn.workspace_bytes(shape, Tq, Tk, q_pos0)} B)")
    o = attn.attention(shape, _dev_bf16(q), _dev_bf16(k), _dev_bf16(v), q_pos0)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    sel = np.arange(Tq) if rows is None else rows
    ref = np.concatenate([A.attention(q[i:i + 1], k, v, q_pos0 + i, window) for i in sel]) if rows is not None \
        else A.attention(q, k, v, q_pos0, window)
    d = np.abs(og[sel] - ref)
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * rms
    say(f"  max |err| {d.max():.3g} = {d.max() / rms:.3g} x RMS; worst err / bound {np.max(d / bound):.3f} "
        f"over {len(sel)} queries")
    assert np.all(d <= bound)


@pytest.mark.parametrize("Hq,Hkv,window,Tq,Tk,q_pos0", [
    (16, 4, W, 256, 1024, 768),     # sliding-window prefill chunk, full windows
    (16, 4, W, 37, 37, 0),          # start of a sequence: ragged block, windows clipped at 0
    (16, 4, 0, 128, 640, 512),      # whole context, prefill chunk
    (16, 4, 0, 1, 4096, 4095),      # whole-context decode: keys split over blocks
    (16, 4, 0, 1, 4196, 4195),      # 66 splits, not a multiple of the merge's eight split groups
    (16, 1, 0, 1, 32768, 32767),    # one key/value head: 512 splits, two per merge thread
    (16, 4, W, 3, 2000, 1997),      # sliding-window decode of three tokens
    (8, 8, W, 100, 700, 600),       # one query head per key/value head (64 queries a block)
    (32, 2, 0, 20, 300, 280),       # groups of 16 heads (4 queries a block)
    (16, 4, W, 600, 1200, 600),     # a long batch: 8-wave blocks of 128 rows, ragged last block
    (8, 8, 0, 520, 900, 380),       # long batch, one query head per group (128 queries a block)
    (16, 1, W, 40, 45, 5),          # one key/value head for all query heads; a cache of 45 keys
    (64, 1, 0, 2, 3, 1),            # a group of 64 heads (one query a block), three keys
    (16, 4, 1, 37, 37, 0),          # a window of one key: each query sees only itself
    (16, 4, 65, 200, 300, 100),     # a window just over one key tile
    (16, 4, 65, 600, 900, 300),     # the same in 8-wave blocks
])
def test_attention_matches_oracle(Hq, Hkv, window, Tq, Tk, q_pos0):
    _check_attention(Hq, Hkv, window, Tq, Tk, q_pos0)


@pytest.mark.parametrize("window,Tq,Tk,q_pos0", [(W, 2048, 4096, 2048), (0, 2048, 4096, 2048),
                                                 (0, 1, 32768, 32767)])
def test_attention_full_size_sampled(window, Tq, Tk, q_pos0):
    """The benchmark's shapes, on sampled queries (first, last, a stride)."""
    rows = np.unique(np.concatenate([np.arange(0, Tq, 97), [Tq - 1]]))
    _check_attention(16, 4, window, Tq, Tk, q_pos0, rows=rows, seed=1)


@pytest.mark.parametrize("Hq,Hkv,Tq,Tk,q_pos0", [(32, 32, 1024, 1100, 76), (32, 32, 1000, 1500, 500),
                                                 (16, 4, 512, 8704, 8192)])
def test_attention_two_key_groups(Hq, Hkv, Tq, Tk, q_pos0):
    """Whole-context batches whose blocks span 16 or more key tiles: each block
    runs two key groups and merges their states.  32 query and 32 key/value
    heads: 256 blocks of 128 rows, no key split (a ragged last block in the
    second case); 512 queries after 8192 cached keys: 8 key splits of 17 tiles,
    the merged states written as split partials.  Sampled queries (every 7th
    and the last)."""
    rows = np.unique(np.concatenate([np.arange(0, Tq, 7), [Tq - 1]]))
    _check_attention(Hq, Hkv, 0, Tq, Tk, q_pos0, rows=rows, seed=2)


def test_window_boundary_exact():
    """Uniform attention (q = 0) of a query at position 600 over a 513-key
    window: it sees keys 88..600, so a marker at key 88 averages to 1/513 and
    markers at keys 87 and 601 add nothing."""
    Tk, p = 602, 600
    v = np.zeros((Tk, 4, 128), np.float32)
    v[:, :, 0] = 1.0
    v[p - W + 1, :, 1] = 1.0
    v[p - W, :, 2] = 1.0
    v[p + 1, :, 3] = 1.0
    rng = np.random.default_rng(3)
    k = _rand(rng, (Tk, 4, 128))
    q = np.zeros((1, 16, 128), np.float32)
    o = attn.attention(attn.AttnShape(16, 4, 128, W), _dev_bf16(synth.bf16_bits(q)), _dev_bf16(k),
                       _dev_bf16(synth.bf16_bits(v)), p)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[0]
    say(f"window boundary: o[0] {o[0, 0]}, o[1] {o[0, 1]} (1/513 = {1 / W:.6g}), o[2] {o[0, 2]}, o[3] {o[0, 3]}")
    assert np.all(o[:, 0] == 1.0)
    assert np.all(np.abs(o[:, 1] - 1.0 / W) <= 2.0 ** -8 / W)
    assert np.all(o[:, 2] == 0.0) and np.all(o[:, 3] == 0.0)
