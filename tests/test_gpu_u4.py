"""4-bit group-quantised weights (MOE_U4_G64) on the GPU, through the C ABI.

The weights are scale * q + bias per row and group of 64 columns (bf16 scale
and bias), the reading of the 4-bit build that "We Stopped the Kolibri
Benchmark Before Scoring One Answer" runs (section "The gate, forced");
activations and h enter the projections in bf16.  The kernels take the codes
and group parameters in the library's tiled layout (moe_pack_weights_u4).

  * the packed layout, bit for bit, against a numpy restatement of the layout
    the header documents;
  * the layer against the oracle's 4-bit mode, with the parity bars of the
    other modes: the decode layer (fused expert launch), a 300-token batch, and
    small layers that take the other kernel paths (the down projection in
    stages for F > 640, a d_model that is not a multiple of 256, a shared
    expert narrower than the routed ones);
  * the stages called one at a time (two separate expert launches) give the
    fused launch's bits.
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import moe, synth
from oracle import moe_oracle as O

from test_gpu_parity import (DEV, W_ABS, check_dispatch_properties, check_logits, check_y, gpu_inputs,
                             route_agreement, run_gpu, say, selection_scores)

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _layout_reference(codes, scales, biases):
    """The documented tiled layout, restated with numpy: codes [n, rows, cols/2]
    uint8, scales/biases [n, rows, cols/64] bf16 bits -> (codes_out bytes,
    params_out bytes)."""
    n, rows, half = codes.shape
    cols = 2 * half
    nkb = cols // 128
    q = np.empty((n, rows, cols), np.uint32)
    q[:, :, 0::2] = codes & 0x0F
    q[:, :, 1::2] = codes >> 4
    words = np.empty((n, rows // 16, nkb, 64, 4), np.uint32)  # [mat, rt, kb, slot l, word m]
    for l in range(64):
        for m in range(4):
            c0 = 32 * m + 8 * (l // 16)
            rsel = np.arange(l % 16, rows, 16)
            w = np.zeros((n, rows // 16, nkb), np.uint32)
            for j in range(4):
                col_even = np.arange(nkb) * 128 + c0 + 2 * j
                w |= q[:, rsel][:, :, col_even] << (4 * j)
                w |= q[:, rsel][:, :, col_even + 1] << (16 + 4 * j)
            words[:, :, :, l, m] = w
    codes_out = words.astype("<u4").tobytes()
    ent = np.empty((n, rows // 16, nkb, 16, 4), np.uint16)  # [mat, rt, kb, row r, (s0, b0, s1, b1)]
    for r in range(16):
        rsel = np.arange(r, rows, 16)
        ent[:, :, :, r, 0] = scales[:, rsel][:, :, 0::2]
        ent[:, :, :, r, 1] = biases[:, rsel][:, :, 0::2]
        ent[:, :, :, r, 2] = scales[:, rsel][:, :, 1::2]
        ent[:, :, :, r, 3] = biases[:, rsel][:, :, 1::2]
    return codes_out, ent.astype("<u2").tobytes()


def test_pack_u4_layout_matches_header():
    rng = np.random.default_rng(5)
    n, rows, cols = 3, 48, 384
    codes = rng.integers(0, 256, (n, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, (n, rows, cols // 64), dtype=np.uint16)
    biases = rng.integers(0, 1 << 16, (n, rows, cols // 64), dtype=np.uint16)
    say(f"moe_pack_weights_u4 n={n} rows={rows} cols={cols} against the documented layout")
    c_out, p_out = moe.pack_weights_u4(torch.from_numpy(codes).to(DEV), _bf16_tensor(scales), _bf16_tensor(biases))
    torch.cuda.synchronize()
    ref_c, ref_p = _layout_reference(codes, scales, biases)
    assert c_out.cpu().numpy().tobytes() == ref_c
    assert p_out.cpu().numpy().tobytes() == ref_p


def _check_layer(inp, g, tok):
    s = inp["shape"]
    L = O.Layer(inp)
    _, lg, idx, w = O.route(L, tok)
    check_logits(g["logits"][tok], lg)
    bad, ex = route_agreement(g["topk_idx"][tok], idx, selection_scores(inp, lg), s.k)
    say(f"  ids on {len(tok)} tokens: {bad} mismatches, {ex} exempt")
    assert bad == 0
    same = (g["topk_idx"][tok] == idx).all(axis=1)
    assert np.max(np.abs(g["topk_w"][tok][same] - w[same])) <= W_ABS
    _, acc_ref = O.forward(L, idx[same], w[same], tok[same])
    check_y(g["y"][tok[same]], acc_ref)


@pytest.mark.parametrize("T", [32, 300])
def test_u4_free(T):
    """The decode layer with 4-bit weights against the oracle's 4-bit mode: the
    decode batch in full, a 300-token batch on sampled tokens."""
    inp = synth.make_inputs("decode_t32_u4", T=T)
    s = inp["shape"]
    say(f"decode_t32_u4 T={s.T}: 4-bit weights against the oracle")
    g = run_gpu(inp)
    assert g["status"][0] == 0
    check_dispatch_properties(g, s.E)
    tok = np.arange(s.T) if s.T <= 32 else np.unique(np.concatenate([np.arange(0, s.T, 11), [s.T - 1]]))
    _check_layer(inp, g, tok)


def _small_u4_inputs(d, F, Fs, T, E=8, k=2, seed=3):
    """A small random layer with 4-bit weights (quantised from N(0, 0.02) draws)."""
    rng = np.random.default_rng(seed)
    inp = dict(shape=synth.LayerShape(T=T, d=d, E=E, k=k, F=F, Fs=Fs, act="bf16", w="u4"),
               x=synth.bf16_bits(rng.standard_normal((T, d), dtype=np.float32)),
               w_router=(rng.standard_normal((E, d), dtype=np.float32) * 0.05).astype(np.float32), sel_bias=None)
    for pre, sp, bp, n, (Fg) in (("w_", "s_", "b_", E, F), ("sh_", "ss_", "sb_", None, Fs)):
        for name, (r, c) in (("gate", (Fg, d)), ("up", (Fg, d)), ("down", (d, Fg))):
            mats = [synth.u4_groups(rng.standard_normal((r, c), dtype=np.float32) * np.float32(0.02))
                    for _ in range(n or 1)]
            for key, j in ((pre, 0), (sp, 1), (bp, 2)):
                inp[key + name] = np.stack([m[j] for m in mats]) if n else mats[0][j]
    return inp


@pytest.mark.parametrize("d,F,Fs,T", [(256, 768, 128, 40),   # down in stages (F > 640), split launches
                                      (384, 256, 128, 33),   # d not a multiple of 256: split launches
                                      (512, 384, 640, 17)])  # fused launch, shared expert wider than routed
def test_u4_small_layers(d, F, Fs, T):
    inp = _small_u4_inputs(d, F, Fs, T)
    say(f"4-bit layer d={d} F={F} Fs={Fs} T={T} against the oracle on every token")
    g = run_gpu(inp, dev=gpu_inputs_u4(inp))
    assert g["status"][0] == 0
    _check_layer(inp, g, np.arange(T))


def gpu_inputs_u4(inp):
    """Device inputs of a small 4-bit layer (packed; not cached across layers)."""
    keys = [k for k, v in inp.items() if isinstance(v, np.ndarray) and k not in ("x", "w_router")]
    w = moe.pack_layer_weights(synth.to_device({k: inp[k] for k in keys}, DEV))
    w.update(synth.to_device({k: inp[k] for k in ("x", "w_router")}, DEV))
    return w


def test_u4_stages_match_fused():
    """Gate/up, down and combine called one at a time (two separate expert
    launches) give bitwise the output of one forward call (the fused launch)."""
    inp = synth.make_inputs("decode_t32_u4")
    s = inp["shape"]
    dev = gpu_inputs(inp)
    shape = moe.shape_of(s)
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    say(f"decode_t32_u4 T={s.T}: stages one at a time vs one forward call")
    moe.route(shape, dev, dev["x"], r, ws)
    y1 = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    moe.forward(shape, dev, dev["x"], r, y1, ws)
    for st in (moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        moe.forward_stages(shape, dev, dev["x"], r, y2, ws, st)
    torch.cuda.synchronize()
    assert r.status.item() == 0
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("T", [1, 64])
def test_u4_forced(T):
    """4-bit weights with forced routing (random ids, some repeated within a
    token), one token and a 64-token batch, against the oracle."""
    inp = synth.make_inputs("decode_t32_u4", T=T)
    s = inp["shape"]
    rng = np.random.default_rng(T)
    forced = rng.integers(0, s.E, size=(T, s.k)).astype(np.int32)
    forced[0, 1] = forced[0, 0]  # a duplicate id: computed twice, literally
    say(f"decode_t32_u4 T={T}: forced routing against the oracle")
    g = run_gpu(inp, forced=forced)
    assert g["status"][0] == 0 and np.array_equal(g["topk_idx"], forced)
    L = O.Layer(inp)
    _, _, idf, wf = O.route_forced(L, forced)
    assert np.max(np.abs(g["topk_w"] - wf)) <= W_ABS
    _, acc_ref = O.forward(L, idf, wf)
    check_y(g["y"], acc_ref)
