"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every pin compares the oracle with an independent source: torch's own number
format conversions, numpy float64 BLAS products and stable sorts, exact
integer arithmetic, closed forms, brute force, or the layer's dense
restatement.  Each pin also has a planted-mutant control: a deliberate bug
switched on inside the oracle (on the CPU) must make that pin fail, after the
planted-bug controls of "We Stopped the Kolibri Benchmark Before Scoring One
Answer" (section "The gate, forced") and the planted bugs of "We Ported Aleph
Alpha's Kolibri to a MacBook. Our Own Gate Said No." (section "The gate").
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import synth
from oracle import moe_oracle as O

F32_ULP = 2.0 ** -23


def _layer(case, T=None, **override):
    inp = dict(synth.make_inputs(case, T=T))
    for k, v in override.items():
        if k == "shape":
            inp["shape"] = v
        else:
            inp[k] = v
    return inp, O.Layer(inp)


def _x_f32(inp):
    x = inp["x"]
    return x if x.dtype == np.float32 else synth.bf16_bits_to_f32(x)


def _torch_e4m3_to_f32(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def _torch_f32_to_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _dequant_weight(codes, scales):
    """Ŵ = decode(code) * block scale, decoded by torch (independent of the oracle)."""
    w = _torch_e4m3_to_f32(codes)
    R, C = w.shape
    s = np.repeat(np.repeat(scales, 128, axis=0), 128, axis=1)
    return (w * s).astype(np.float32)


def _swiglu64(wg, wu, wd, x):
    g = wg.astype(np.float64) @ x.astype(np.float64)
    u = wu.astype(np.float64) @ x.astype(np.float64)
    h = g / (1.0 + np.exp(-g)) * u
    return wd.astype(np.float64) @ h


# ---------------------------------------------------------------- number formats

def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_decode(codes)
    ref = _torch_e4m3_to_f32(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.isnan(mine[nan]).all()
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # bit-exact, signed zeros too
    # OCP E4M3 landmarks: largest finite, smallest normal, smallest subnormal
    assert mine[0x7E] == 448.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0xFE] == -448.0


def test_e4m3_encode_vs_torch():
    vals = _torch_e4m3_to_f32(np.arange(0x7F, dtype=np.uint8))  # all non-negative finite values, ascending
    mids = (vals[:-1].astype(np.float64) + vals[1:]) / 2.0
    mids = mids.astype(np.float32)  # every midpoint of this grid is exactly representable in fp32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)), vals])
    grid16 = synth.bf16_bits_to_f32(np.arange(1 << 16, dtype=np.uint16).astype(np.uint16))
    rng = np.random.default_rng(7)
    rand_bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rand_small = (rng.standard_normal(1 << 21) * 30).astype(np.float32)
    v = np.concatenate([near, -near, grid16, rand_bits, rand_small]).astype(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 448.0)]
    mine = O.e4m3_encode(v)
    ref = _torch_f32_to_e4m3(v)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, (v[bad[:5]], mine[bad[:5]], ref[bad[:5]])
    # ties go to the even code: the midpoint of 1.0 (0x38) and 1.125 (0x39) -> 0x38,
    # of 1.125 and 1.25 (0x3A) -> 0x3A
    assert O.e4m3_encode([1.0625, 1.1875]).tolist() == [0x38, 0x3A]
    # saturation and NaN (reading: saturating conversion)
    assert O.e4m3_encode([448.0, 460.0, 1e9, np.inf, -1e9, -np.inf]).tolist() == [0x7E] * 4 + [0xFE] * 2
    assert O.e4m3_encode([np.nan]).tolist() == [0x7F]


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    v = np.concatenate([bits, ties, ties + 1, ties - 1]).view(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45], np.float32)])
    mine = O.f32_to_bf16(v)
    ref = synth.bf16_bits(v)
    nan = np.isnan(v)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.isnan(synth.bf16_bits_to_f32(mine[nan])).all()


def test_quant_groups_definition():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(128 * 64) * np.exp(rng.standard_normal(128 * 64))).astype(np.float32)
    v[:128] = 0.0  # an all-zero group takes scale 1 and zero codes
    codes, scales = O.quant_groups(v)
    g = v.reshape(-1, 128)
    amax = np.abs(g).max(axis=1)
    s_ref = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(scales, s_ref)
    ref = _torch_f32_to_e4m3((g / s_ref[:, None]).astype(np.float32)).ravel()
    assert np.array_equal(codes, ref)
    # the group maximum always lands on +-448
    mx = np.abs(_torch_e4m3_to_f32(codes).reshape(-1, 128)).max(axis=1)
    assert (mx[1:] == 448.0).all() and mx[0] == 0.0
    # a power-of-two rescale of a group changes only its scale
    c2, s2 = O.quant_groups(v * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2[1:], scales[1:] * 8)
    assert np.array_equal(codes, _quant_ref(v)[0])


def _quant_ref(v):
    """Per-128-group codes and scales from the quantiser's definition, computed
    without the oracle: s = amax/448 by numpy's correctly rounded float32
    division (1 for an all-zero group), codes = torch's float8_e4m3fn
    conversion (round to nearest even) of the float32 quotient v/s."""
    g = np.asarray(v, np.float32).reshape(-1, 128)
    amax = np.abs(g).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return _torch_f32_to_e4m3((g / s[:, None]).astype(np.float32)).ravel(), s


def _midpoint_rows(n_rows=2, d=2048):
    """bf16 activation rows whose every group quantises on exact E4M3 rounding
    midpoints.  Group g has amax = 784 * 2^j (j = g - 8), so s = amax/448 =
    1.75 * 2^j exactly, and its other values are +-m * s for midpoints
    m = (1 + (2i+1)/16) * 2^e of the normal E4M3 range (i = 0..7, e = -6..7):
    v/s = m exactly (m has 5 significant bits and 1.75 three, so m * s is a bf16
    value).  Round-to-nearest-even takes the even mantissa of each tie; a
    quantiser that rounds ties away from zero moves every midpoint with even i,
    and one that multiplies by fl(448/amax) = fl(4/7) * 2^-j (0.75 of half an
    ulp above 4/7) lifts the midpoints with i >= 3 over the tie, which moves
    i = 4 and i = 6."""
    mids = np.array([(1 + (2 * i + 1) / 16) * 2.0 ** e for e in range(-6, 8) for i in range(8)])
    rows = np.empty((n_rows, d), np.float32)
    for r in range(n_rows):
        for g in range(d // 128):
            s = 1.75 * 2.0 ** (g - 8)
            vals = np.concatenate([mids, mids[-15:]])[:127] * s
            sign = np.where((np.arange(127) + g + r) % 2 == 0, 1.0, -1.0)
            rows[r, g * 128] = 448.0 * s
            rows[r, g * 128 + 1:(g + 1) * 128] = np.roll(vals * sign, 3 * r + g)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.bf16_bits(rows)), rows)  # exact bf16 values
    return rows


def test_forward_quantiser_exact_on_midpoints():
    """The forward's own activation quantisation (the codes oracle_forward
    multiplies with, read back through oracle_expert_ffn_trace) equals the
    definition bit for bit on groups built so that every value is an exact
    rounding tie; each planted quantiser mistake (the reciprocal scale, ties
    away from zero) changes codes there, and only through this one quantiser."""
    inp, _ = _layer("decode_t32", T=4)
    rows = _midpoint_rows()
    x = inp["x"].copy()
    x[:2] = synth.bf16_bits(rows)
    L = O.Layer(dict(inp, x=x))
    for t in (0, 1):
        tr = O.expert_ffn_trace(L, 0, t)
        ref_c, ref_s = _quant_ref(rows[t])
        assert np.array_equal(tr["x_scales"].view(np.uint32), ref_s.view(np.uint32))
        assert np.all(ref_s == (1.75 * 2.0 ** (np.arange(16) - 8)).astype(np.float32))
        assert np.array_equal(tr["x_codes"], ref_c)
        # the row the products see is decode(code) * s, here the tie's even neighbour exactly
        assert np.array_equal(tr["x_used"], (_torch_e4m3_to_f32(ref_c) * np.repeat(ref_s, 128)).astype(np.float32))
    moved = {}
    for m in ("quant_reciprocal", "quant_ties_away"):
        with O.mutant(m):
            tr = O.expert_ffn_trace(L, 0, 0)
            codes_exported, _ = O.quant_groups(rows[0])
        moved[m] = int(np.sum(tr["x_codes"] != _quant_ref(rows[0])[0]))
        assert moved[m] > 0, m
        assert np.array_equal(codes_exported, tr["x_codes"]), m  # one quantiser: the same codes
    assert moved["quant_ties_away"] > moved["quant_reciprocal"]  # even i at every exponent vs i = 4, 6


def test_forward_quantiser_exact_on_layer_rows():
    """On the decode layer's rows: the x codes and scales the forward uses, and
    the h codes and scales it forms from its own h before the down projection,
    equal the definition bit for bit (torch E4M3, numpy float32 division); the
    products see decode(code) * s."""
    inp, L = _layer("decode_t32", T=6)
    xf = _x_f32(inp)
    n_h = 0
    for e, t in ((-1, 0), (0, 1), (200, 2), (383, 5)):
        tr = O.expert_ffn_trace(L, e, t)
        ref_c, ref_s = _quant_ref(xf[t])
        assert np.array_equal(tr["x_codes"], ref_c) and np.array_equal(tr["x_scales"], ref_s)
        assert np.array_equal(tr["x_used"], (_torch_e4m3_to_f32(ref_c) * np.repeat(ref_s, 128)).astype(np.float32))
        h_c, h_s = _quant_ref(tr["h"])
        assert np.array_equal(tr["h_codes"], h_c) and np.array_equal(tr["h_scales"], h_s)
        n_h += tr["h"].size
        _, y = O.expert_ffn(L, e, t)
        assert np.array_equal(y, tr["y"])  # the traced call is the forward's FFN
    assert n_h == 4 * 640


# ---------------------------------------------------------------- router

def _router_defect(case, tokens):
    inp, L = _layer(case)
    rc, logits, _, _ = O.route(L, tokens)
    assert rc == O.OK
    x = _x_f32(inp)[tokens].astype(np.float64)
    ref = (x @ inp["w_router"].astype(np.float64).T).astype(np.float32)
    ulps = np.abs(logits.astype(np.float64) - ref) / np.maximum(np.abs(ref), 1e-30) / F32_ULP
    return float(np.max(np.where(ref == logits, 0.0, ulps)))


def test_router_vs_float64_blas():
    tokens = np.arange(0, 32, 3)
    assert _router_defect("decode_t32", tokens) <= 1.0
    assert _router_defect("tiny_f32", np.arange(64)) <= 1.0
    for m in ("router_bf16", "logits_bf16"):
        with O.mutant(m):
            assert _router_defect("decode_t32", tokens) > 100.0, m


def test_router_exact_on_integer_grid():
    """Integer activations and a 1/64 grid make every logit an exact multiple of
    1/64; the oracle must return it exactly (closed form in int64)."""
    inp, L = _layer("ties_t256")
    tokens = np.arange(0, 256, 5)
    rc, logits, _, _ = O.route(L, tokens)
    xi = _x_f32(inp)[tokens].astype(np.int64)
    wi = np.rint(inp["w_router"].astype(np.float64) * 64).astype(np.int64)
    assert np.array_equal(wi.astype(np.float64) / 64, inp["w_router"].astype(np.float64))
    exact = (xi @ wi.T).astype(np.float64) / 64.0
    assert np.array_equal(logits.astype(np.float64), exact)


# ---------------------------------------------------------------- top-k and weights

def _brute_topk(score, k):
    E = score.shape[1]
    out = np.empty((score.shape[0], k), np.int32)
    for t in range(score.shape[0]):
        order = np.lexsort((np.arange(E), -score[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def _topk_defect(case, tokens):
    inp, L = _layer(case)
    _, logits, idx, _ = O.route(L, tokens)
    s = logits if inp["sel_bias"] is None else (logits + inp["sel_bias"][None, :]).astype(np.float32)
    return int(np.sum(idx != _brute_topk(s, inp["shape"].k)))


def test_topk_vs_full_stable_sort():
    assert _topk_defect("tiny_f32", np.arange(64)) == 0
    assert _topk_defect("ties_t256", np.arange(0, 256, 2)) == 0
    assert _topk_defect("skew_t8192", np.arange(0, 8192, 97)) == 0
    with O.mutant("tie_highest"):
        assert _topk_defect("ties_t256", np.arange(0, 256, 2)) > 0
    with O.mutant("select_unbiased"):
        assert _topk_defect("skew_t8192", np.arange(0, 8192, 97)) > 0


def test_ties_workload_has_exact_ties():
    inp, L = _layer("ties_t256")
    _, logits, idx, _ = O.route(L, np.arange(256))
    srt = -np.sort(-logits, axis=1)
    assert np.sum(srt[:, 5] == srt[:, 6]) >= 10  # exact 6th/7th ties exercise the tie-break


def _weight_defect(case, tokens):
    inp, L = _layer(case)
    _, logits, idx, w = O.route(L, tokens)
    sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    ref = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref /= ref.sum(axis=1, keepdims=True)
    return float(np.max(np.abs(w - ref)))


def test_weights_softmax_over_selected():
    assert _weight_defect("tiny_f32", np.arange(64)) <= 1e-6
    assert _weight_defect("skew_t8192", np.arange(0, 8192, 97)) <= 1e-6
    with O.mutant("softmax_all"):
        assert _weight_defect("tiny_f32", np.arange(64)) > 1e-3
    with O.mutant("weights_biased"):
        assert _weight_defect("skew_t8192", np.arange(0, 8192, 97)) > 1e-3


def test_weights_special_cases():
    inp, L = _layer("tiny_f32", w_router=np.zeros((16, 256), np.float32))
    _, logits, idx, w = O.route(L)
    assert (logits == 0).all()
    assert (idx == np.arange(2)[None, :]).all()  # all tied: lowest indices, in order
    assert (w == np.float32(1.0) / np.float32(2.0)).all()
    inp, L = _layer("tiny_f32")
    s1 = dataclass_replace(inp["shape"], k=1)
    inp1, L1 = _layer("tiny_f32", shape=s1)
    _, _, idx1, w1 = O.route(L1)
    assert (w1 == 1.0).all()
    _, _, _, wk = O.route(L)
    assert np.max(np.abs(wk.sum(axis=1) - 1.0)) <= 2 * F32_ULP


def dataclass_replace(s, **kw):
    import dataclasses
    return dataclasses.replace(s, **kw)


def test_forced_replays_free_and_validates():
    inp, L = _layer("tiny_f32")
    _, lf, idf, wf = O.route(L)
    rc, l2, id2, w2 = O.route_forced(L, idf)
    assert rc == O.OK and np.array_equal(lf, l2) and np.array_equal(idf, id2) and np.array_equal(wf, w2)
    bad = idf.copy()
    bad[3, 1] = 16
    bad[5, 0] = -1
    rc, _, id3, w3 = O.route_forced(L, bad)
    assert rc == O.ERR_FORCED_INDEX
    assert id3[3, 1] == -1 and w3[3, 1] == 0 and w3[3, 0] == 1.0
    assert id3[5, 0] == -1 and w3[5, 0] == 0 and w3[5, 1] == 1.0
    # forced order is the caller's: reversing the slots reverses idx and w
    rc, _, id4, w4 = O.route_forced(L, idf[:, ::-1])
    assert np.array_equal(id4, idf[:, ::-1]) and np.allclose(w4, wf[:, ::-1], rtol=0, atol=1e-7)


# ---------------------------------------------------------------- dispatch

def _dispatch_defect(idx, E):
    counts, offsets, perm, inv = O.dispatch(idx, E)
    flat = idx.ravel()
    ref_perm = np.argsort(flat, kind="stable").astype(np.int32)
    bad = int(np.sum(perm != ref_perm))
    ok = counts.sum() == flat.size and np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    ok &= np.array_equal(counts, np.bincount(flat, minlength=E))
    ok &= np.array_equal(perm[inv], np.arange(flat.size)) and np.array_equal(inv[perm], np.arange(flat.size))
    return bad + (0 if ok else 1)


def test_dispatch_vs_stable_argsort():
    rng = np.random.default_rng(5)
    for T, k, E in ((64, 2, 16), (513, 6, 384), (1, 6, 384), (300, 6, 7)):
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
        assert _dispatch_defect(idx, E) == 0
    idx = np.zeros((40, 6), np.int32)  # one expert takes every pair
    assert _dispatch_defect(idx, 384) == 0
    with O.mutant("reversed_order"):
        assert _dispatch_defect(rng.integers(0, 16, size=(64, 2)).astype(np.int32), 16) > 0


def test_dispatch_drops_invalid_pairs():
    idx = np.array([[0, -1], [2, 0], [0, 2]], np.int32)
    counts, offsets, perm, inv = O.dispatch(idx, 3)
    assert counts.tolist() == [3, 0, 2]
    assert perm.tolist() == [0, 3, 4, 2, 5, -1]
    assert inv.tolist() == [0, -1, 3, 1, 2, 4]


# ---------------------------------------------------------------- expert FFN

def _ffn_defect_f32(expert, t=5):
    inp, L = _layer("tiny_f32")
    xu, y = O.expert_ffn(L, expert, t)
    x = inp["x"][t]
    assert np.array_equal(xu, x)
    if expert < 0:
        wg, wu, wd = inp["sh_gate"], inp["sh_up"], inp["sh_down"]
    else:
        wg, wu, wd = inp["w_gate"][expert], inp["w_up"][expert], inp["w_down"][expert]
    ref = _swiglu64(wg, wu, wd, x)
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def test_ffn_f32_vs_textbook_swiglu():
    for e in (-1, 0, 7, 15):
        assert _ffn_defect_f32(e) <= 1e-5
    for m in ("silu_sign", "gate_up_swap"):
        with O.mutant(m):
            assert _ffn_defect_f32(3) > 1e-2, m


def test_ffn_bf16_weights_vs_textbook_swiglu():
    inp, L = _layer("ties_t256_bf16w", T=8)
    for e in (-1, 0, 383):
        xu, y = O.expert_ffn(L, e, 2)
        assert np.array_equal(xu, _x_f32(inp)[2])
        pre = ("sh_" if e < 0 else "w_")
        get = (lambda n: inp[pre + n]) if e < 0 else (lambda n: inp[pre + n][e])
        ref = _swiglu64(*(synth.bf16_bits_to_f32(get(n)) for n in ("gate", "up", "down")), xu)
        assert np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)) <= 1e-5


def _fp8_expert_weights(inp, e):
    if e < 0:
        return [_dequant_weight(inp["sh_" + n], inp["ss_" + n]) for n in ("gate", "up", "down")]
    return [_dequant_weight(inp["w_" + n][e], inp["s_" + n][e]) for n in ("gate", "up", "down")]


def _fp8_linear_defect(inp, L, e, t):
    """Oracle FFN with h left unquantised vs the float64 textbook SwiGLU on
    torch-decoded block-scaled weights and the oracle's quantised x."""
    with O.mutant("no_h_quant"):
        xu, y = O.expert_ffn(L, e, t)
    ref = _swiglu64(*_fp8_expert_weights(inp, e), xu)
    return float(np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)))


def test_ffn_fp8_block_scaled_vs_textbook():
    inp, L = _layer("decode_t32", T=4)
    for e in (-1, 0, 200):
        assert _fp8_linear_defect(inp, L, e, 1) <= 1e-5
    # quantised x: decode(code) * s reproduces the activation within E4M3's half-ulp
    xu, _ = O.expert_ffn(L, 0, 1)
    x = _x_f32(inp)[1]
    g = np.abs(x.reshape(-1, 128)).max(axis=1, keepdims=True)
    assert np.all(np.abs(xu - x).reshape(-1, 128) <= g / 448 * 16 + 1e-12)
    with O.mutant("scale_transposed"):
        xu2, y2 = O.expert_ffn(L, 0, 1)
    ref = _swiglu64(*_fp8_expert_weights(inp, 0), xu)
    assert np.max(np.abs(y2 - ref)) / np.sqrt(np.mean(ref ** 2)) > 1e-2


def test_ffn_fp8_h_quant_effect():
    inp, L = _layer("decode_t32", T=4)
    xu, y = O.expert_ffn(L, 11, 2)
    with O.mutant("no_h_quant"):
        _, y_nq = O.expert_ffn(L, 11, 2)
    d = np.abs(y - y_nq)
    assert d.max() > 0  # the h quantisation step is really there
    wg, wu, wd = _fp8_expert_weights(inp, 11)
    g = wg.astype(np.float64) @ xu
    h = g / (1 + np.exp(-g)) * (wu.astype(np.float64) @ xu)
    # per group, |h - decode(Q(h))| <= half an E4M3 step at the group's scale
    bound = np.abs(wd.astype(np.float64)) @ np.repeat(np.abs(h).reshape(-1, 128).max(axis=1) / 448 * 16, 128)
    assert np.all(d <= bound * 1.001 + 1e-7)


def test_ffn_fp8_exact_arithmetic_case():
    """Codes from {0, +-0.5, +-1, +-2}, power-of-two scales and activations whose
    group maximum is 7*2^j: quantising x is exact, and the projections are
    exact sums, so g and u equal the integer-grid closed form."""
    inp, _ = _layer("decode_t32", T=4)
    rng = np.random.default_rng(2)
    small = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], np.uint8)  # 0, +-0.5, +-1, +-2
    E = 8
    exact = dict(inp, shape=dataclass_replace(inp["shape"], E=E), w_router=inp["w_router"][:E])
    for n in ("gate", "up", "down"):
        exact["w_" + n] = small[rng.integers(0, small.size, size=(E,) + inp["w_" + n].shape[1:])]
        exact["s_" + n] = (2.0 ** rng.integers(-8, -4, size=(E,) + inp["s_" + n].shape[1:])).astype(np.float32)
        exact["sh_" + n] = small[rng.integers(0, small.size, size=inp["sh_" + n].shape)]
        exact["ss_" + n] = (2.0 ** rng.integers(-8, -4, size=inp["ss_" + n].shape)).astype(np.float32)
    xv = rng.choice(np.array([0, 0.5, -0.5, 1, -1, 2, -2], np.float32), size=(4, 2048))
    xv[:, ::128] = 7.0 * 2.0 ** rng.integers(1, 3, size=(4, 16))  # 14 or 28: the group maximum
    exact["x"] = synth.bf16_bits(xv)
    Le = O.Layer(exact)
    with O.mutant("no_h_quant"):
        xu, y = O.expert_ffn(Le, 5, 0)
    assert np.array_equal(xu, xv[0])
    wg, wu, wd = _fp8_expert_weights(exact, 5)
    assert np.array_equal(wg @ xu.astype(np.float64), (wg.astype(np.float64) @ xu.astype(np.float64)))
    ref = _swiglu64(wg, wu, wd, xu)
    assert np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)) <= 1e-5


def test_block_scale_locality():
    """Doubling one block scale of W_down changes only the 128 outputs of that
    block, by exactly that block's contribution."""
    inp, L = _layer("decode_t32", T=4)
    e, nb, kb, t = 17, 3, 2, 1
    xu, y0 = O.expert_ffn(L, e, t)
    s2 = inp["s_down"].copy()
    s2[e, nb, kb] *= 2
    inp2 = dict(inp, s_down=s2)
    _, y1 = O.expert_ffn(O.Layer(inp2), e, t)
    diff = (y1.astype(np.float64) - y0).reshape(16, 128)
    mask = np.zeros(16, bool)
    mask[nb] = True
    assert (diff[~mask] == 0).all()
    wg, wu, wd = _fp8_expert_weights(inp, e)
    g = wg.astype(np.float64) @ xu
    h = (g / (1 + np.exp(-g)) * (wu.astype(np.float64) @ xu)).astype(np.float32)
    hq_c, hq_s = O.quant_groups(h)
    hq = _torch_e4m3_to_f32(hq_c) * np.repeat(hq_s, 128)
    contrib = wd[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].astype(np.float64) @ hq[kb * 128:(kb + 1) * 128]
    assert np.max(np.abs(diff[nb] - contrib)) <= 1e-5 * np.sqrt(np.mean(y0.astype(np.float64) ** 2))
    with O.mutant("scale_transposed"):
        _, z0 = O.expert_ffn(L, e, t)
        _, z1 = O.expert_ffn(O.Layer(inp2), e, t)
    dz = (z1.astype(np.float64) - z0).reshape(16, 128)
    assert not (dz[~mask] == 0).all() or np.max(np.abs(dz[nb] - contrib)) > 1e-3


# ---------------------------------------------------------------- whole layer

def _dense_defect(case, T=None):
    inp, L = _layer(case, T=T)
    _, _, idx, w = O.route(L)
    _, acc = O.forward(L, idx, w)
    dense = O.forward_dense_masked(L, idx, w)
    return float(np.max(np.abs(acc - dense)) / np.sqrt(np.mean(dense.astype(np.float64) ** 2)))


def test_forward_vs_dense_masked():
    assert _dense_defect("tiny_f32") <= 1e-5
    for m in ("no_shared", "combine_no_weight"):
        with O.mutant(m):
            assert _dense_defect("tiny_f32") > 1e-2, m


def test_shared_expert_alone():
    inp, L = _layer("tiny_f32")
    zero = dict(inp, w_down=np.zeros_like(inp["w_down"]))
    Lz = O.Layer(zero)
    _, _, idx, w = O.route(Lz)
    _, acc = O.forward(Lz, idx, w)
    for t in (0, 17, 63):
        _, ys = O.expert_ffn(Lz, -1, t)
        assert np.array_equal(acc[t], ys)
    with O.mutant("no_shared"):
        _, acc2 = O.forward(Lz, idx, w)
    assert (acc2 == 0).all()


def test_bf16_output_is_rounded_acc():
    inp, L = _layer("decode_t32", T=3)
    _, _, idx, w = O.route(L)
    y, acc = O.forward(L, idx, w)
    assert np.array_equal(y, synth.bf16_bits(acc))


def test_token_permutation_equivariance():
    inp, L = _layer("decode_t32", T=6)
    _, _, idx, w = O.route(L)
    y, _ = O.forward(L, idx, w)
    perm = np.array([4, 0, 5, 2, 1, 3])
    L2 = O.Layer(dict(inp, x=inp["x"][perm]))
    _, _, idx2, w2 = O.route(L2)
    y2, _ = O.forward(L2, idx2, w2)
    assert np.array_equal(idx2, idx[perm]) and np.array_equal(w2, w[perm]) and np.array_equal(y2, y[perm])


def test_token_subset_matches_full():
    inp, L = _layer("decode_t32", T=8)
    _, lg, idx, w = O.route(L)
    tok = np.array([6, 1, 3])
    _, lg2, idx2, w2 = O.route(L, tok)
    assert np.array_equal(lg2, lg[tok]) and np.array_equal(idx2, idx[tok]) and np.array_equal(w2, w[tok])
    y, _ = O.forward(L, idx, w)
    y2, _ = O.forward(L, idx[tok], w[tok], tok)
    assert np.array_equal(y2, y[tok])


def test_threaded_oracle_bitwise_equals_single_thread():
    """The all-cores drivers run the same per-token code on contiguous token
    ranges: logits, ids, weights and outputs are bitwise those of the
    single-threaded calls, for any thread count (more threads than tokens too)."""
    inp, L = _layer("decode_t32", T=13)
    _, lg, idx, w = O.route(L)
    y, acc = O.forward(L, idx, w)
    for n in (1, 3, 8, 20):
        _, lg2, idx2, w2 = O.route_threads(L, n_threads=n)
        assert np.array_equal(lg2.view(np.uint32), lg.view(np.uint32))
        assert np.array_equal(idx2, idx) and np.array_equal(w2.view(np.uint32), w.view(np.uint32))
        y2, acc2 = O.forward_threads(L, idx, w, n_threads=n)
        assert np.array_equal(y2, y) and np.array_equal(acc2.view(np.uint32), acc.view(np.uint32))
    tok = np.array([12, 0, 7, 3, 9])
    y3, _ = O.forward_threads(L, idx[tok], w[tok], tok, n_threads=2)
    assert np.array_equal(y3, y[tok])


def test_skew_workload_is_skewed():
    inp, L = _layer("skew_t8192")
    tok = np.arange(0, 8192, 8)
    _, _, idx, _ = O.route(L, tok)
    counts = np.bincount(idx.ravel(), minlength=384)
    assert counts.max() > 10 * counts.mean()


# ---------------------------------------------------------------- W8A16 (FP8 weights, bf16 activations)

def _small_fp8_layer(w_mode, T=16, seed=7):
    """A small layer with block-scaled E4M3 weights (d=256, E=8, k=2, F=Fs=128),
    as the given weight mode: "fp8" / "fp8a16" (codes and scales) or "f32"
    (the same weights decoded by torch: decode(code) * scale in fp32)."""
    rng = np.random.default_rng(seed)
    d, E, k, F, Fs = 256, 8, 2, 128, 128
    x = synth.bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    inp = dict(shape=synth.LayerShape(T=T, d=d, E=E, k=k, F=F, Fs=Fs, act="bf16", w=w_mode),
               x=x, w_router=(rng.standard_normal((E, d), dtype=np.float32) * 0.05).astype(np.float32),
               sel_bias=None)
    for pre, sp, dims, n in (("w_", "s_", (F, d, d, F), E), ("sh_", "ss_", (Fs, d, d, Fs), None)):
        for name, (r, c) in (("gate", dims[:2]), ("up", dims[:2]), ("down", dims[2:])):
            ws = [rng.standard_normal((r, c), dtype=np.float32) * np.float32(0.02) for _ in range(n or 1)]
            blocks = [synth.fp8_blocks(w) for w in ws]
            if w_mode == "f32":
                vals = [_dequant_weight(cq, sq) for cq, sq in blocks]
                inp[pre + name] = np.stack(vals) if n else vals[0]
            else:
                inp[pre + name] = np.stack([b[0] for b in blocks]) if n else blocks[0][0]
                inp[sp + name] = np.stack([b[1] for b in blocks]) if n else blocks[0][1]
    return inp, O.Layer(inp)


def test_w8a16_equals_f32_mode_on_decoded_weights():
    """W8A16 is the FP8 weights' exact values, unquantised activations and h:
    bitwise the oracle's fp32-weight mode run on the same weights decoded by
    torch (each element decode(code) * scale, one fp32 multiply)."""
    a16, La = _small_fp8_layer("fp8a16")
    f32, Lf = _small_fp8_layer("f32")
    _, la, ia, wa = O.route(La)
    _, lf, i_f, wf = O.route(Lf)
    assert np.array_equal(la.view(np.uint32), lf.view(np.uint32))
    assert np.array_equal(ia, i_f) and np.array_equal(wa.view(np.uint32), wf.view(np.uint32))
    ya, acc_a = O.forward(La, ia, wa)
    yf, acc_f = O.forward(Lf, i_f, wf)
    assert np.array_equal(acc_a.view(np.uint32), acc_f.view(np.uint32))
    assert np.array_equal(ya, yf)
    # and it is not the FP8 mode, whose activations and h are quantised
    q, Lq = _small_fp8_layer("fp8")
    _, acc_q = O.forward(Lq, ia, wa)
    assert np.max(np.abs(acc_q - acc_a)) > 1e-4 * np.sqrt(np.mean(acc_a.astype(np.float64) ** 2))


def test_w8a16_expert_ffn_vs_textbook():
    """One expert in W8A16: the activation row enters as the bf16 values
    themselves, and the FFN is the float64 textbook SwiGLU on torch-decoded
    block-scaled weights."""
    inp, L = _small_fp8_layer("fp8a16")
    for e, t in ((-1, 3), (0, 5), (6, 11)):
        xu, y = O.expert_ffn(L, e, t)
        assert np.array_equal(xu.view(np.uint32), _x_f32(inp)[t].view(np.uint32))
        ref = _swiglu64(*_fp8_expert_weights(inp, e), xu)
        assert np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)) <= 1e-6


# ---------------------------------------------------------------- 4-bit weights

def _u4_dequant(codes, scales, biases):
    """scale * q + bias per (row, group of 64 columns), unpacked with numpy bit
    operations (the even column in the low nibble) and computed in float64;
    asserted exact in fp32 so that the fp32-weight mode sees the same values."""
    codes = np.asarray(codes, np.uint8)
    R, half = codes.shape
    q = np.empty((R, 2 * half), np.float64)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    s = np.repeat(synth.bf16_bits_to_f32(scales).astype(np.float64), 64, axis=1)
    b = np.repeat(synth.bf16_bits_to_f32(biases).astype(np.float64), 64, axis=1)
    w = s * q + b
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    return w.astype(np.float32)


def _small_u4_layer(w_mode, T=16, seed=11, unit=False):
    """A small layer with 4-bit group-quantised weights (d=256, E=8, k=2,
    F=Fs=128) as "u4" (codes, scales, biases) or "f32" (the same weights
    dequantised by _u4_dequant).  unit: every scale 1 and bias 0, so the weights
    are the integer codes themselves."""
    rng = np.random.default_rng(seed)
    d, E, k, F, Fs = 256, 8, 2, 128, 128
    x = synth.bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    inp = dict(shape=synth.LayerShape(T=T, d=d, E=E, k=k, F=F, Fs=Fs, act="bf16", w=w_mode),
               x=x, w_router=(rng.standard_normal((E, d), dtype=np.float32) * 0.05).astype(np.float32),
               sel_bias=None)
    for pre, sp, bp, dims, n in (("w_", "s_", "b_", (F, d, d, F), E), ("sh_", "ss_", "sb_", (Fs, d, d, Fs), None)):
        for name, (r, c) in (("gate", dims[:2]), ("up", dims[:2]), ("down", dims[2:])):
            mats = []
            for _ in range(n or 1):
                codes, sc, bi = synth.u4_groups(rng.standard_normal((r, c), dtype=np.float32) * np.float32(0.02))
                if unit:
                    sc = np.full_like(sc, 0x3F80)  # bf16 1.0
                    bi = np.zeros_like(bi)
                mats.append((codes, sc, bi))
            if w_mode == "f32":
                vals = [_u4_dequant(*m) for m in mats]
                inp[pre + name] = np.stack(vals) if n else vals[0]
            else:
                for key, j in ((pre, 0), (sp, 1), (bp, 2)):
                    inp[key + name] = np.stack([m[j] for m in mats]) if n else mats[0][j]
    return inp, O.Layer(inp)


@pytest.mark.parametrize("unit", [False, True])
def test_u4_equals_f32_mode_on_dequantised_weights(unit):
    """The 4-bit mode is the layer on the weights scale * q + bias: bitwise the
    oracle's fp32-weight mode on the same weights dequantised independently
    (numpy bit operations, float64, exact in fp32).  With unit scales and zero
    biases the weights are the integer codes.  Each planted 4-bit mistake (the
    nibbles swapped, the bias dropped, groups of 128) breaks the equality."""
    u4, Lu = _small_u4_layer("u4", unit=unit)
    f32, Lf = _small_u4_layer("f32", unit=unit)
    _, lu, iu, wu = O.route(Lu)
    _, lf, i_f, wf = O.route(Lf)
    assert np.array_equal(lu.view(np.uint32), lf.view(np.uint32)) and np.array_equal(iu, i_f)
    yu, acc_u = O.forward(Lu, iu, wu)
    yf, acc_f = O.forward(Lf, i_f, wf)
    assert np.array_equal(acc_u.view(np.uint32), acc_f.view(np.uint32))
    assert np.array_equal(yu, yf)
    rms = np.sqrt(np.mean(acc_f.astype(np.float64) ** 2))
    for m in ("u4_nibble_swap",) + (() if unit else ("u4_group128", "u4_no_bias")):  # unit: all groups alike
        with O.mutant(m):
            _, acc_m = O.forward(Lu, iu, wu)
        assert np.max(np.abs(acc_m - acc_f)) > 1e-3 * rms, m


def test_u4_expert_ffn_vs_textbook():
    """One expert with 4-bit weights: the activation row enters as its bf16
    values, and the FFN is the float64 textbook SwiGLU on the dequantised
    weights."""
    inp, L = _small_u4_layer("u4")
    for e, t in ((-1, 2), (0, 7), (5, 13)):
        xu, y = O.expert_ffn(L, e, t)
        assert np.array_equal(xu.view(np.uint32), _x_f32(inp)[t].view(np.uint32))
        if e < 0:
            ws = [_u4_dequant(inp["sh_" + n], inp["ss_" + n], inp["sb_" + n]) for n in ("gate", "up", "down")]
        else:
            ws = [_u4_dequant(inp["w_" + n][e], inp["s_" + n][e], inp["b_" + n][e]) for n in ("gate", "up", "down")]
        ref = _swiglu64(*ws, xu)
        assert np.max(np.abs(y - ref)) / np.sqrt(np.mean(ref ** 2)) <= 1e-6


# ---------------------------------------------------------------- routing as a distribution

def _cmp_case_basic():
    """Four tokens, E=6, k=2, no selection bias.  The other side's logits are the
    reference's plus +0.5 at (1, 3), +1.5 at (3, 4) and -2.0 at (3, 0), so
    sigma^2 = (0.25 + 2.25 + 4) / 24.  Token 0 has the same set in another slot
    order; token 1 swaps expert 2 (ref score 2.5) for 3 (2.25): margin 0.25;
    token 2 is an all-equal row resolved the same way; token 3 swaps 0 (5.0)
    for 4 (3.0): margin 2.0."""
    ref = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -2.0],
                    [0.0, 3.0, 2.5, 2.25, 1.0, 0.0],
                    [1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                    [5.0, 4.0, 0.0, -1.0, 3.0, 2.0]], np.float32)
    oth = ref.copy()
    oth[1, 3] += 0.5
    oth[3, 4] += 1.5
    oth[3, 0] -= 2.0
    ref_idx = np.array([[0, 1], [1, 2], [0, 1], [0, 1]], np.int32)
    idx = np.array([[1, 0], [1, 3], [0, 1], [4, 1]], np.int32)
    return oth, ref, idx, ref_idx


def test_route_compare_worked_example():
    oth, ref, idx, ref_idx = _cmp_case_basic()
    gap, sigma, nd, mg = O.route_compare(oth, ref, idx, ref_idx)
    sig = np.sqrt(6.5 / 24.0)  # 0.52041650...
    assert abs(sigma - sig) <= 1e-12
    assert nd == 2
    assert gap[0] == -1.0 and gap[2] == -1.0
    assert abs(gap[1] - 0.25 / sig) <= 1e-6 and abs(gap[3] - 2.0 / sig) <= 1e-6  # 0.48038, 3.84308
    assert abs(mg - 2.0 / sig) <= 1e-6


def test_route_compare_bias_and_worst_pair():
    """The margin uses the reference's selection score (logit + bias), and a
    token with several swapped experts takes its largest margin; each planted
    change (margins from the bare logits, the closest pair) moves the result."""
    # bias: ref scores [1.0, 0.9, 0.8, 1.0, 0.1] choose {0, 3}; the other side
    # (logit 3 lowered by 0.5) chooses {0, 1}; margin 1.0 - 0.9 = 0.1 (biased),
    # -0.9 from the bare logits
    ref = np.array([[1.0, 0.9, 0.8, 0.0, 0.1]], np.float32)
    oth = ref.copy()
    oth[0, 3] -= 0.5
    bias = np.array([0, 0, 0, 1.0, 0], np.float32)
    args = (oth, ref, np.array([[0, 1]], np.int32), np.array([[0, 3]], np.int32), bias)
    sig = np.sqrt(0.25 / 5)
    gap, sigma, nd, mg = O.route_compare(*args)
    assert nd == 1 and abs(sigma - sig) <= 1e-12 and abs(gap[0] - 0.1 / sig) <= 1e-6
    with O.mutant("compare_unbiased"):
        assert O.route_compare(*args)[0][0] < 0
    # worst pair: ref {0, 1, 2} from [3, 2, 1, 0, -1, -2]; the other side (+2.5
    # at 3, +3.5 at 4) chooses {0, 3, 4}: pairs (1,3) 2, (1,4) 3, (2,3) 1, (2,4) 2
    ref = np.array([[3, 2, 1, 0, -1, -2]], np.float32)
    oth = ref + np.array([[0, 0, 0, 2.5, 3.5, 0]], np.float32)
    args = (oth, ref, np.array([[0, 3, 4]], np.int32), np.array([[0, 1, 2]], np.int32))
    sig = np.sqrt((2.5 ** 2 + 3.5 ** 2) / 6)
    gap, sigma, nd, mg = O.route_compare(*args)
    assert abs(gap[0] - 3.0 / sig) <= 1e-6 and mg == gap[0]
    with O.mutant("compare_min_pair"):
        assert abs(O.route_compare(*args)[0][0] - 1.0 / sig) <= 1e-6


def test_route_compare_invariants():
    """Identical sides: sigma 0, no disagreement.  Slot order inside a token does
    not matter.  Scaling the logit difference by c scales sigma by c and every
    gap by 1/c (the ids are inputs, not recomputed)."""
    oth, ref, idx, ref_idx = _cmp_case_basic()
    gap, sigma, nd, mg = O.route_compare(ref, ref, ref_idx, ref_idx)
    assert sigma == 0.0 and nd == 0 and mg == -1.0 and np.all(gap == -1.0)
    g0, s0, n0, m0 = O.route_compare(oth, ref, idx, ref_idx)
    g1, s1, n1, m1 = O.route_compare(oth, ref, idx[:, ::-1], ref_idx[:, ::-1])
    assert np.array_equal(g0, g1) and s0 == s1 and n0 == n1
    oth4 = ref + 4.0 * (oth - ref)  # exact: the differences are small binary fractions
    g4, s4, n4, m4 = O.route_compare(oth4, ref, idx, ref_idx)
    assert abs(s4 - 4 * s0) <= 1e-12 and n4 == n0
    d = g0 >= 0
    assert np.allclose(g4[d], g0[d] / 4, rtol=1e-6) and np.array_equal(g4[~d], g0[~d])
