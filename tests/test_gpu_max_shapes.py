"""The layer at the edges of the supported shape range, on the GPU through the
C ABI, against the oracle with the parity bars of the main workloads.

  * the widest layer (d_model 4608, d_ffn and d_ffn_shared 4096: one 16-row
    tile's activation and h rows fill the LDS of a workgroup) with FP8 weights,
    with the same weights and bf16 activations (W8A16), and with 4-bit group
    weights; as many experts as top_k (every token routes to every expert, so
    the experts hold T rows each) and a ragged T; with FP8 weights also with
    ten 16-row tiles per expert;
  * the most experts and the largest top_k (512 experts, top 8: eight candidates
    per lane in the selection), with the one-block dispatch (800 pairs) and the
    chunked one (2,400 pairs), free and forced;
  * the widest fp32 layer (d_model and d_ffn 2560), short and long batches;
  * the longest batch timed by the bench: the decode layer at T = 32768 with
    free routing (128-token router blocks, 32-row tiles, about 16 per expert),
    the dispatch checked whole and the outputs on sampled tokens.
Layers: weights N(0, 0.02) quantised to E4M3 with 128x128 block scales, router
weights N(0, 0.05), activations N(0, 1) in bf16 (the recipe of the main
workloads at other sizes).
"""
import numpy as np
import pytest

from mixture_experts_moe_amd import moe, synth
from oracle import moe_oracle as O

from test_gpu_parity import (DEV, W_ABS, check_dispatch, check_dispatch_properties, check_logits, check_y,
                             route_agreement, run_gpu, say, selection_scores)

pytestmark = pytest.mark.gpu


def _fp8_layer(T, d, E, k, F, Fs, seed, w="fp8"):
    """A layer with FP8 block-scaled weights ("fp8", or "fp8a16": the same
    weights with bf16 activations) or 4-bit group weights ("u4")."""
    rng = np.random.default_rng(seed)
    inp = dict(shape=synth.LayerShape(T=T, d=d, E=E, k=k, F=F, Fs=Fs, act="bf16", w=w),
               x=synth.bf16_bits(rng.standard_normal((T, d), dtype=np.float32)),
               w_router=rng.standard_normal((E, d), dtype=np.float32) * np.float32(0.05), sel_bias=None)
    quant = synth.u4_groups if w == "u4" else synth.fp8_blocks
    parts = ("w_", "s_", "b_") if w == "u4" else ("w_", "s_")
    for pre, n, Fg in (("", E, F), ("sh", 0, Fs)):
        for name, (r, c) in (("gate", (Fg, d)), ("up", (Fg, d)), ("down", (d, Fg))):
            mats = [quant(rng.standard_normal((r, c), dtype=np.float32) * np.float32(0.02)) for _ in range(max(n, 1))]
            for j, part in enumerate(parts):
                key = (pre + part if not pre else {"w_": "sh_", "s_": "ss_", "b_": "sb_"}[part]) + name
                inp[key] = np.stack([m[j] for m in mats]) if n else mats[0][j]
    return inp


def _dev(inp):
    keys = [k for k, v in inp.items() if isinstance(v, np.ndarray) and k not in ("x", "w_router")]
    w = synth.to_device({k: inp[k] for k in keys}, DEV)
    if inp["shape"].w == "u4":  # 4-bit weights exist only in the tiled layout
        w = moe.pack_layer_weights(w)
    w.update(synth.to_device({k: inp[k] for k in ("x", "w_router")}, DEV))
    return w


def _check(inp, g, forced=None, n_sample=None):
    s = inp["shape"]
    assert g["status"][0] == 0
    L = O.Layer(inp)
    if forced is None:
        _, lg, idx, w = O.route(L)
        check_logits(g["logits"], lg)
        bad, ex = route_agreement(g["topk_idx"], idx, selection_scores(inp, lg), s.k)
        say(f"  ids: {bad} mismatches, {ex} tokens exempt by the gap rule")
        assert bad == 0
        same = (g["topk_idx"] == idx).all(axis=1)
        tok = np.nonzero(same)[0]
    else:
        assert np.array_equal(g["topk_idx"], forced)
        check_dispatch(g, forced, s.E)
        tok = np.arange(s.T)
    if n_sample is not None:
        tok = tok[np.unique(np.linspace(0, len(tok) - 1, n_sample).astype(int))]
    ids = g["topk_idx"][tok]
    _, _, idf, wf = O.route_forced(L, np.ascontiguousarray(g["topk_idx"]), tok)
    assert np.array_equal(idf, ids)
    assert np.max(np.abs(g["topk_w"][tok] - wf)) <= W_ABS
    _, acc_ref = O.forward(L, idf, wf, tok)
    return check_y(g["y"][tok], acc_ref)


def _f32_layer(T, d, E, k, F, Fs, seed):
    """An all-fp32 layer: activations N(0, 1), router N(0, 0.05), expert and
    shared weights N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    inp = dict(shape=synth.LayerShape(T=T, d=d, E=E, k=k, F=F, Fs=Fs, act="f32", w="f32"),
               x=rng.standard_normal((T, d), dtype=np.float32),
               w_router=rng.standard_normal((E, d), dtype=np.float32) * np.float32(0.05), sel_bias=None)
    for key, shp in (("w_gate", (E, F, d)), ("w_up", (E, F, d)), ("w_down", (E, d, F)),
                     ("sh_gate", (Fs, d)), ("sh_up", (Fs, d)), ("sh_down", (d, Fs))):
        inp[key] = rng.standard_normal(shp, dtype=np.float32) * np.float32(0.02)
    return inp


@pytest.mark.parametrize("T", [40, 600])
def test_widest_f32_layer(T):
    """The widest fp32 layer (d_model and d_ffn 2560, the fp32 limit): 40 tokens
    (the short-batch router, ragged 16-row tiles) and 600 tokens (the long-batch
    router tiles and chunked top-k; sampled outputs).  All-fp32 arithmetic, so
    the outputs sit within 1e-4 of the oracle's RMS (only summation order
    differs)."""
    d, E, k, F = 2560, 4, 2, 2560
    inp = _f32_layer(T, d, E, k, F, F, seed=17)
    say(f"widest f32 layer T={T} d={d} E={E} k={k} F=Fs={F}")
    g = run_gpu(inp, dev=_dev(inp))
    assert _check(inp, g, n_sample=None if T <= 40 else 8) < 1e-4


@pytest.mark.parametrize("w", ["fp8", "fp8a16", "u4"])
def test_widest_layer(w):
    """The widest layer each weight type supports: d_model 4608, d_ffn 4096."""
    T, d, E, k, F = 40, 4608, 4, 4, 4096
    inp = _fp8_layer(T, d, E, k, F, F, seed=11, w=w)
    say(f"widest {w} layer T={T} d={d} E={E} k={k} F=Fs={F}")
    g = run_gpu(inp, dev=_dev(inp))
    _check(inp, g, n_sample=5)


def test_widest_layer_many_tiles():
    """The widest FP8 layer with 150 rows per expert: past the row count that
    picks 32-row tiles, which do not fit the LDS at this width (32 rows of h
    4096 wide), so the kernels stay at 16-row tiles, ten per expert with a
    ragged last one, and the down projection streams K in stages."""
    T, d, E, k, F = 150, 4608, 4, 4, 4096
    inp = _fp8_layer(T, d, E, k, F, F, seed=13)
    say(f"widest fp8 layer, many 16-row tiles per expert: T={T} d={d} E={E} k={k} F=Fs={F}")
    g = run_gpu(inp, dev=_dev(inp))
    _check(inp, g, n_sample=6)


@pytest.mark.parametrize("T,kind", [(100, "free"), (100, "forced"), (300, "free"), (300, "forced")])
def test_most_experts_top8(T, kind):
    d, E, k, F, Fs = 256, 512, 8, 128, 128
    inp = _fp8_layer(T, d, E, k, F, Fs, seed=12)
    forced = None
    if kind == "forced":
        forced = np.random.default_rng(T).integers(0, E, size=(T, k)).astype(np.int32)
        forced[0, :] = forced[0, 0]  # one token with every slot on one expert
    say(f"E={E} k={k} T={T} ({T * k} pairs) {kind}")
    g = run_gpu(inp, forced=forced, dev=_dev(inp))
    _check(inp, g, forced=forced)


def test_long_prefill_t32768_sampled():
    """T = 32768 on the decode layer, free routing, as the bench times it: the
    dispatch is the stable sort of the GPU's own ids (whole batch); logits, ids,
    weights and y against the oracle on every 64th token, the last token, and
    the last 32 rows (the ragged tail tile) of the three most loaded experts."""
    inp = synth.make_inputs("prefill_t32768")
    s = inp["shape"]
    say(f"prefill_t32768: T={s.T} free routing")
    g = run_gpu(inp)
    check_dispatch_properties(g, s.E)
    counts = g["counts"]
    say(f"  expert load: max {counts.max()} mean {counts.mean():.1f} min {counts.min()}")
    L = O.Layer(inp)
    heavy = np.argsort(-counts, kind="stable")[:3]
    tail = np.concatenate([g["perm"][max(g["offsets"][e], g["offsets"][e + 1] - 32):g["offsets"][e + 1]] // s.k
                           for e in heavy])
    tok = np.unique(np.concatenate([np.arange(0, s.T, 64), tail, [s.T - 1]]))
    _, lg, idx, w = O.route_threads(L, tok)
    check_logits(g["logits"][tok], lg)
    bad, ex = route_agreement(g["topk_idx"][tok], idx, selection_scores(inp, lg), s.k)
    say(f"  ids on {len(tok)} sampled tokens: {bad} mismatches, {ex} exempt")
    assert bad == 0
    same = (g["topk_idx"][tok] == idx).all(axis=1)
    assert np.max(np.abs(g["topk_w"][tok][same] - w[same])) <= W_ABS
    ts = tok[same]
    _, acc_ref = O.forward_threads(L, idx[same], w[same], ts)
    check_y(g["y"][ts], acc_ref)
