"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
the same seeded inputs.

Bars (written here, derived in the design notes):
  * router logits: |dl| <= 1e-4 * max(|l|, rms of the token's logits);
  * free-routing ids: the ordered row must match wherever every adjacent gap
    among the top k+1 selection scores exceeds 1e-3; the set must match where
    the k / k+1 gap exceeds 1e-3; other tokens are exempt and counted (on the
    integer-grid workload, where logits are exact, every token must match);
  * forced ids and the dispatch (counts, offsets, perm, inv_perm): bit-exact;
  * routing weights: |dw| <= 1e-5;
  * layer output: max |dy| <= 2e-2 * RMS(y_oracle) over the compared tokens.
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import moe, synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

LOGIT_REL = 1e-4
GAP = 1e-3
W_ABS = 1e-5
Y_REL = 2e-2

_weights_dev: dict = {}
_WKEYS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
          "ss_gate", "ss_up", "ss_down", "b_gate", "b_up", "b_down", "sb_gate", "sb_up", "sb_down")


def say(*a):
    print(*a, flush=True)


def gpu_inputs(inp):
    """Device tensors of one workload; the (large) expert weights are uploaded
    once per process and shared by every workload of the same layer."""
    key = id(inp["w_gate"])
    if key not in _weights_dev:
        w = synth.to_device({k: inp[k] for k in _WKEYS if inp.get(k) is not None}, DEV)
        if inp["shape"].w == "u4":  # 4-bit weights exist only in the tiled layout
            w = moe.pack_layer_weights(w)
        _weights_dev[key] = (inp["w_gate"], w)  # the host array is held, so its id is never reused
    d = dict(_weights_dev[key][1])
    d.update(synth.to_device({k: inp[k] for k in ("x", "w_router", "sel_bias") if inp.get(k) is not None}, DEV))
    return d


def run_gpu(inp, forced=None, dev=None, routing=None, expect_status=moe.MOE_OK):
    """One route + forward through the C ABI; asserts the device status word
    (and the sticky forward status, when the routing carries one)."""
    s = inp["shape"]
    shape = moe.shape_of(s)
    dev = dev or gpu_inputs(inp)
    r = routing or moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    y = torch.empty((s.T, s.d), dtype=torch.float32 if s.act == "f32" else torch.bfloat16, device=DEV)
    if forced is None:
        moe.route(shape, dev, dev["x"], r, ws)
    else:
        moe.route_forced(shape, dev, dev["x"], torch.from_numpy(np.ascontiguousarray(forced, np.int32)).to(DEV),
                         r, ws)
    moe.forward(shape, dev, dev["x"], r, y, ws)
    torch.cuda.synchronize()
    out = {n: getattr(r, n).cpu().numpy() for n in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm",
                                                      "status")}
    out["logits"] = r.logits.cpu().numpy() if r.logits is not None else None
    out["y"] = y.float().cpu().numpy()
    assert out["status"][0] == expect_status, moe.status_string(int(out["status"][0]))
    if r.forward_status is not None:
        assert r.forward_status.item() == moe.MOE_OK, moe.status_string(r.forward_status.item())
    return out


def selection_scores(inp, logits):
    b = inp.get("sel_bias")
    return logits if b is None else (logits + b[None, :]).astype(np.float32)


def check_logits(gpu, ref):
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2, axis=1, keepdims=True))
    bound = LOGIT_REL * np.maximum(np.abs(ref), rms)
    bad = np.abs(gpu.astype(np.float64) - ref) > bound
    assert not bad.any(), f"{bad.sum()} logits outside 1e-4 relative"


def route_agreement(gpu_idx, ref_idx, ref_scores, k):
    """Returns (mismatches on non-exempt tokens, exempt tokens)."""
    srt = -np.sort(-ref_scores.astype(np.float64), axis=1)[:, :k + 1]
    if srt.shape[1] == k:  # k == E: every expert is chosen, the k / k+1 gap is unbounded
        srt = np.concatenate([srt, np.full((srt.shape[0], 1), -np.inf)], axis=1)
    gaps = srt[:, :-1] - srt[:, 1:]
    bad = exempt = 0
    for t in range(gpu_idx.shape[0]):
        if (gaps[t] > GAP).all():
            bad += int(not np.array_equal(gpu_idx[t], ref_idx[t]))
        elif gaps[t, k - 1] > GAP:
            bad += int(set(gpu_idx[t].tolist()) != set(ref_idx[t].tolist()))
        else:
            exempt += 1
    return bad, exempt


def check_y(y_gpu, acc_ref):
    """Layer output against the oracle's fp32 result before its final rounding.
    (Two independently bf16-rounded outputs may differ by a whole bf16 ulp on a
    rounding straddle; the GPU's own rounding adds at most half an ulp here.)"""
    ref = acc_ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - ref)))
    say(f"  max|dy| = {err:.3e}  rms(y) = {rms:.3e}  ratio = {err / rms:.3e}")
    assert err <= Y_REL * rms, f"layer output error {err / rms:.3e} x rms exceeds {Y_REL}"
    return err / rms


def check_dispatch(gpu, ref_idx, E):
    c, o, p, inv = O.dispatch(ref_idx, E)
    assert np.array_equal(gpu["counts"], c)
    assert np.array_equal(gpu["offsets"], o)
    assert np.array_equal(gpu["perm"], p)
    assert np.array_equal(gpu["inv_perm"], inv)


def check_dispatch_properties(gpu, E):
    """Holds at any size: the dispatch is the stable sort of the GPU's own ids."""
    idx = gpu["topk_idx"].ravel()
    valid = (idx >= 0) & (idx < E)
    counts = np.bincount(idx[valid], minlength=E)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    n = int(valid.sum())
    perm = gpu["perm"]
    assert np.array_equal(perm[:n], np.nonzero(valid)[0][np.argsort(idx[valid], kind="stable")])
    assert (perm[n:] == -1).all()
    inv = gpu["inv_perm"]
    assert np.array_equal(inv[perm[:n]], np.arange(n))
    assert (inv[~valid] == -1).all()


# ------------------------------------------------------------------ activation quantisation

def test_quantize_rows_bitexact():
    rng = np.random.default_rng(1)
    xf = (rng.standard_normal((512, 2048)) * np.exp(rng.standard_normal((512, 1)))).astype(np.float32)
    xf[3, :128] = 0.0
    xf[4, 128:256] = 1e-30
    for act in ("bf16", "f32"):
        say(f"quantize_rows {act} [512, 2048]")
        x_np = synth.bf16_bits(xf) if act == "bf16" else xf
        xv = synth.bf16_bits_to_f32(x_np) if act == "bf16" else xf
        xt = synth.to_device({"x": x_np}, DEV)["x"]
        codes = torch.empty((512, 2048), dtype=torch.uint8, device=DEV)
        scales = torch.empty((512, 16), dtype=torch.float32, device=DEV)
        moe.quantize_rows(xt, codes, scales)
        torch.cuda.synchronize()
        c_ref, s_ref = O.quant_groups(xv)
        assert np.array_equal(scales.cpu().numpy().ravel(), s_ref)
        assert np.array_equal(codes.cpu().numpy().ravel(), c_ref)


# ------------------------------------------------------------------ tiny fp32 layer

def test_tiny_free_and_forced():
    inp = synth.make_inputs("tiny_f32")
    s = inp["shape"]
    say(f"tiny_f32 T={s.T} d={s.d} E={s.E} k={s.k} free")
    L = O.Layer(inp)
    _, lg, idx, w = O.route(L)
    g = run_gpu(inp)
    assert g["status"][0] == 0
    check_logits(g["logits"], lg)
    bad, ex = route_agreement(g["topk_idx"], idx, selection_scores(inp, lg), s.k)
    assert bad == 0 and ex <= 2
    same = (g["topk_idx"] == idx).all(axis=1)
    if same.all():
        check_dispatch(g, idx, s.E)
    else:
        check_dispatch_properties(g, s.E)
    assert np.max(np.abs(g["topk_w"][same] - w[same])) <= W_ABS
    _, acc_ref = O.forward(L, idx, w)
    check_y(g["y"][same], acc_ref[same])
    say("tiny_f32 forced from the oracle's recorded ids")
    gf = run_gpu(inp, forced=idx)
    assert np.array_equal(gf["topk_idx"], idx)
    check_dispatch(gf, idx, s.E)
    assert np.max(np.abs(gf["topk_w"] - w)) <= W_ABS
    _, acc_ref = O.forward(L, idx, w)
    r = check_y(gf["y"], acc_ref)
    assert r < 1e-4  # all-fp32 path: only summation order differs


def test_tiny_f32_long_batch():
    """The fp32 layer at T=700: 1,400 pairs take the long-batch router tiles and
    the chunked top-k and dispatch, and the expert tiles end in ragged tails.
    Free and forced routing against the oracle; the first 64 tokens' logits,
    ids and outputs equal the 64-token batch's bit for bit (every fp32 logit
    and output is one chain in a fixed order, whatever the batch)."""
    big = synth.make_inputs("tiny_f32", T=700)
    s = big["shape"]
    say(f"tiny_f32 T={s.T} d={s.d} E={s.E} k={s.k} free")
    L = O.Layer(big)
    _, lg, idx, w = O.route(L)
    g = run_gpu(big)
    check_logits(g["logits"], lg)
    bad, ex = route_agreement(g["topk_idx"], idx, selection_scores(big, lg), s.k)
    assert bad == 0 and ex <= 8
    same = (g["topk_idx"] == idx).all(axis=1)
    _, acc_ref = O.forward(L, idx, w)
    check_y(g["y"][same], acc_ref[same])
    say("tiny_f32 T=700 forced from the oracle's recorded ids")
    gf = run_gpu(big, forced=idx)
    assert np.array_equal(gf["topk_idx"], idx)
    check_dispatch(gf, idx, s.E)
    assert check_y(gf["y"], acc_ref) < 1e-4
    say("tiny_f32: the first 64 tokens alone")
    small = synth.make_inputs("tiny_f32")
    assert small["shape"].T == 64 and np.array_equal(small["x"], big["x"][:64])
    gs = run_gpu(small)
    assert np.array_equal(gs["logits"].view(np.uint32), g["logits"][:64].view(np.uint32))
    assert np.array_equal(gs["topk_idx"], g["topk_idx"][:64])
    assert np.array_equal(gs["y"].view(np.uint32), g["y"][:64].view(np.uint32))


# ------------------------------------------------------------------ decode shape, FP8 experts

def test_decode_free():
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    say(f"decode_t32 T={s.T} d={s.d} E={s.E} k={s.k} F={s.F} free")
    L = O.Layer(inp)
    _, lg, idx, w = O.route(L)
    g = run_gpu(inp)
    check_logits(g["logits"], lg)
    bad, ex = route_agreement(g["topk_idx"], idx, selection_scores(inp, lg), s.k)
    say(f"  ids: {bad} mismatches, {ex} exempt")
    assert bad == 0
    check_dispatch_properties(g, s.E)
    same = (g["topk_idx"] == idx).all(axis=1)
    assert np.max(np.abs(g["topk_w"][same] - w[same])) <= W_ABS
    if same.all():
        check_dispatch(g, idx, s.E)
    # output against the oracle's own routing, on the tokens whose ids agree
    _, acc_ref = O.forward(L, idx, w)
    check_y(g["y"][same], acc_ref[same])


def test_decode_forced_and_free_equivalence():
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    L = O.Layer(inp)
    _, _, idx, w = O.route(L)
    say("decode_t32 forced from the oracle's recorded ids")
    g = run_gpu(inp, forced=idx)
    assert g["status"][0] == 0
    assert np.array_equal(g["topk_idx"], idx)
    check_dispatch(g, idx, s.E)
    assert np.max(np.abs(g["topk_w"] - w)) <= W_ABS
    _, acc_ref = O.forward(L, idx, w)
    check_y(g["y"], acc_ref)
    say("decode_t32: forced(free ids) is bitwise the free result")
    gfree = run_gpu(inp)
    gforce = run_gpu(inp, forced=gfree["topk_idx"])
    for n in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "logits", "y"):
        assert np.array_equal(gfree[n], gforce[n]), n


def test_decode_deterministic():
    inp = synth.make_inputs("decode_t32")
    say("decode_t32 run twice: bitwise identical")
    a, b = run_gpu(inp), run_gpu(inp)
    for n in ("logits", "topk_idx", "topk_w", "perm", "inv_perm", "y"):
        assert np.array_equal(a[n], b[n]), n


# ------------------------------------------------------------------ near-ties workload

@pytest.mark.parametrize("case", ["ties_t256", "ties_t256_bf16w"])
def test_ties_exact_routing(case):
    inp = synth.make_inputs(case)
    s = inp["shape"]
    say(f"{case} T={s.T} w={s.w}: exact logits, every token's ids must match")
    L = O.Layer(inp)
    _, lg, idx, w = O.route(L)
    srt = -np.sort(-lg, axis=1)
    say(f"  exact 6th/7th ties in the oracle: {int(np.sum(srt[:, 5] == srt[:, 6]))} tokens")
    g = run_gpu(inp)
    assert np.array_equal(g["logits"], lg)
    assert np.array_equal(g["topk_idx"], idx)
    check_dispatch(g, idx, s.E)
    assert np.max(np.abs(g["topk_w"] - w)) <= W_ABS
    _, acc_ref = O.forward_threads(L, idx, w)  # every token
    check_y(g["y"], acc_ref)


# ------------------------------------------------------------------ prefill, forced routing

def test_prefill_forced_full_size():
    inp = synth.make_inputs("prefill_t2048")
    s = inp["shape"]
    L = O.Layer(inp)
    say(f"prefill_t2048: oracle free pass over T={s.T} records the ids ({O.host_threads()} threads)")
    _, lg, idx, w = O.route_threads(L)
    g = run_gpu(inp, forced=idx)
    say("  GPU forced pass")
    check_logits(g["logits"], lg)
    assert np.array_equal(g["topk_idx"], idx)
    check_dispatch(g, idx, s.E)
    assert np.max(np.abs(g["topk_w"] - w)) <= W_ABS
    say("  oracle forward over every token")
    _, acc_ref = O.forward_threads(L, idx, w)
    check_y(g["y"], acc_ref)


# ------------------------------------------------------------------ W8A16 weight mode

@pytest.mark.parametrize("T", [32, 300])
def test_w8a16_free(T):
    """The FP8 weights used as W8A16 (bf16 activations into both projections,
    unquantised; h in bf16) against the oracle's W8A16 mode: the decode batch
    in full, and a 300-token batch (long routing path, 16-row tiles) on sampled
    tokens."""
    inp = synth.make_inputs("decode_t32_w8a16", T=T)
    s = inp["shape"]
    say(f"decode_t32_w8a16 T={s.T}: W8A16 against the oracle")
    g = run_gpu(inp)
    assert g["status"][0] == 0
    check_dispatch_properties(g, s.E)
    L = O.Layer(inp)
    tok = np.arange(s.T) if s.T <= 32 else np.unique(np.concatenate([np.arange(0, s.T, 11), [s.T - 1]]))
    _, lg, idx, w = O.route(L, tok)
    check_logits(g["logits"][tok], lg)
    bad, ex = route_agreement(g["topk_idx"][tok], idx, selection_scores(inp, lg), s.k)
    say(f"  ids on {len(tok)} tokens: {bad} mismatches, {ex} exempt")
    assert bad == 0
    same = (g["topk_idx"][tok] == idx).all(axis=1)
    assert np.max(np.abs(g["topk_w"][tok][same] - w[same])) <= W_ABS
    _, acc_ref = O.forward(L, idx[same], w[same], tok[same])
    check_y(g["y"][tok[same]], acc_ref)
    # and it is a different computation from the FP8 mode on the same layer, x and experts
    q_inp = dict(synth.make_inputs("decode_t32", T=T))
    q_inp["x"] = inp["x"]
    q = run_gpu(q_inp, forced=g["topk_idx"])
    assert not np.array_equal(q["y"].view(np.uint32), g["y"].view(np.uint32))


# ------------------------------------------------------------------ skewed load, free routing

def test_skew_free_full_size():
    inp = synth.make_inputs("skew_t8192")
    s = inp["shape"]
    say(f"skew_t8192 T={s.T} free routing with the Zipf selection bias")
    g = run_gpu(inp)
    counts = g["counts"]
    say(f"  expert load: max {counts.max()} mean {counts.mean():.1f} zeros {(counts == 0).sum()}")
    assert counts.max() > 10 * counts.mean()
    check_dispatch_properties(g, s.E)
    L = O.Layer(inp)
    # every token (the oracle on all host cores), so every row of the heavy
    # experts' ragged tail tiles is compared too
    tok = np.arange(s.T)
    say(f"  oracle route + forward over all {s.T} tokens on {O.host_threads()} threads")
    _, lg, idx, w = O.route_threads(L, tok)
    check_logits(g["logits"][tok], lg)
    bad, ex = route_agreement(g["topk_idx"][tok], idx, selection_scores(inp, lg), s.k)
    say(f"  ids on {len(tok)} tokens: {bad} mismatches, {ex} exempt")
    assert bad == 0
    same = (g["topk_idx"][tok] == idx).all(axis=1)
    assert np.max(np.abs(g["topk_w"][tok][same] - w[same])) <= W_ABS
    ts = tok[same]
    _, acc_ref = O.forward_threads(L, idx[same], w[same], ts)
    check_y(g["y"][ts], acc_ref)


# ------------------------------------------------------------------ edge shapes

def _forced_random(T, k, E, seed, n_experts_used=None):
    rng = np.random.default_rng(seed)
    pool = np.arange(E) if n_experts_used is None else rng.choice(E, n_experts_used, replace=False)
    return pool[rng.integers(0, len(pool), size=(T, k))].astype(np.int32)


@pytest.mark.parametrize("T,kind", [(1, "free"), (37, "free"), (64, "one_expert"), (100, "free"), (170, "forced"),
                                    (300, "few_experts"), (5462, "forced"), (8792, "forced"),
                                    (8192, "few_experts")])
def test_edge_shapes(T, kind):
    """T=1; a ragged tail; every pair on one expert (duplicate ids per token);
    batches of up to 170 tokens (1024 pairs) route through the one-block
    dispatch, longer ones per chunk; most experts empty; pair counts 32,772 and
    52,752 (just above 32,768 and not
    a multiple of 64; and 8 x 1,099 x 6, the expert-GEMM row counts of section 3
    of "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No.");
    the last with 49,152 pairs on three experts (over five hundred 32-row tiles
    of one expert)."""
    inp = synth.make_inputs("prefill_t2048", T=T)
    s = inp["shape"]
    say(f"edge T={T} ({T * s.k} pairs) {kind}")
    L = O.Layer(inp)
    if kind == "free":
        g = run_gpu(inp)
        _, lg, idx, w = O.route(L)
        bad, ex = route_agreement(g["topk_idx"], idx, selection_scores(inp, lg), s.k)
        assert bad == 0
        assert np.array_equal(g["topk_idx"], idx), "tokens exempt by the gap rule: compare on a subset"
        forced = idx
    else:
        forced = {"one_expert": lambda: np.full((T, s.k), 7, np.int32),
                  "few_experts": lambda: _forced_random(T, s.k, s.E, 5, n_experts_used=3),
                  "forced": lambda: _forced_random(T, s.k, s.E, T)}[kind]()
        g = run_gpu(inp, forced=forced)
        assert np.array_equal(g["topk_idx"], forced)
    check_dispatch(g, forced, s.E)
    tok = np.unique(np.linspace(0, T - 1, min(T, 24)).astype(int))
    _, _, idf, wf = O.route_forced(L, forced, tok)
    assert np.max(np.abs(g["topk_w"][tok] - wf)) <= W_ABS
    _, acc_ref = O.forward(L, idf, wf, tok)
    check_y(g["y"][tok], acc_ref)


def test_invalid_forced_ids_flag_status_and_stay_in_bounds():
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    L = O.Layer(inp)
    _, _, idx, _ = O.route(L)
    bad = idx.copy()
    bad[2, 0], bad[5, 3], bad[31, 5], bad[7, 1] = -3, s.E, 100000, -1
    say("decode_t32 forced with 4 invalid ids")
    shape = moe.shape_of(s)
    P, E, T, k = s.T * s.k, s.E, s.T, s.k
    guard = 64
    SENT = -123456

    def padded(n, dtype):
        t = torch.full((n + guard,), SENT, dtype=dtype, device=DEV)
        return t, t[:n]

    bufs = {n: padded(sz, dt) for n, sz, dt in (("topk_idx", T * k, torch.int32), ("topk_w", T * k, torch.float32),
                                                  ("counts", E, torch.int32), ("offsets", E + 1, torch.int32),
                                                  ("perm", P, torch.int32), ("inv_perm", P, torch.int32),
                                                  ("status", 1, torch.int32), ("logits", T * E, torch.float32))}
    r = moe.Routing(logits=bufs["logits"][1].view(T, E), topk_idx=bufs["topk_idx"][1].view(T, k),
                    topk_w=bufs["topk_w"][1].view(T, k), counts=bufs["counts"][1], offsets=bufs["offsets"][1],
                    perm=bufs["perm"][1], inv_perm=bufs["inv_perm"][1], status=bufs["status"][1],
                    plan=torch.empty(moe.plan_bytes(shape), dtype=torch.uint8, device=DEV))
    g = run_gpu(inp, forced=bad, routing=r, expect_status=moe.MOE_ERR_FORCED_INDEX)
    for n, (full, _) in bufs.items():
        tail = full[-guard:].cpu().numpy()
        assert (tail.view(np.int32) == SENT).all() if full.dtype == torch.int32 else \
            (tail == np.float32(SENT)).all(), f"{n}: write past the end"
    assert g["status"][0] == moe.MOE_ERR_FORCED_INDEX
    rc, _, idf, wf = O.route_forced(L, bad)
    assert rc == O.ERR_FORCED_INDEX
    assert np.array_equal(g["topk_idx"], idf)
    assert np.max(np.abs(g["topk_w"] - wf)) <= W_ABS
    check_dispatch(g, idf, s.E)
    _, acc_ref = O.forward(L, idf, wf)
    check_y(g["y"], acc_ref)


def test_zero_tokens_is_a_no_op():
    inp = synth.make_inputs("decode_t32", T=1)
    s = inp["shape"]
    shape = moe.make_shape(0, s.d, s.E, s.k, s.F, s.Fs)
    dev = gpu_inputs(inp)
    r = moe.alloc_routing(moe.make_shape(1, s.d, s.E, s.k, s.F, s.Fs), DEV)
    r.status.fill_(77)
    y = torch.full((1, s.d), 3.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    moe.route(shape, dev, dev["x"], r, ws)
    moe.forward(shape, dev, dev["x"], r, y, ws)
    torch.cuda.synchronize()
    assert r.status.item() == 77 and (y.float() == 3.0).all()


def test_forward_stages_match_forward():
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    say("decode_t32: stages called one at a time == moe_forward, bitwise")
    shape = moe.shape_of(s)
    dev = gpu_inputs(inp)
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    y1 = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    moe.route(shape, dev, dev["x"], r, ws)
    moe.forward(shape, dev, dev["x"], r, y1, ws)
    b = moe.Bound(shape, dev, dev["x"], r, y2, ws)
    for st in (moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE):
        b.forward(st)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    with pytest.raises(moe.MoeError):
        b.forward(8)


def test_forward_repeats_on_one_plan():
    """With FP8 weights in 16-row tiles the two projections run as one launch
    that synchronises on per-tile counters in the plan and leaves them at zero:
    one routing call serves repeated forward calls and any split of the stages,
    bitwise, and the status word stays MOE_OK."""
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    say("decode_t32: five forward calls on one plan (whole, whole, and three stage splits)")
    shape = moe.shape_of(s)
    dev = gpu_inputs(inp)
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    moe.route(shape, dev, dev["x"], r, ws)
    G, D, C = moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE
    ys = []
    for seq in ([G | D | C], [G | D | C], [G | D, C], [G, D | C], [G | D | C]):
        y = torch.full((s.T, s.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        b = moe.Bound(shape, dev, dev["x"], r, y, ws)
        for st in seq:
            b.forward(st)
        ys.append(y)
    torch.cuda.synchronize()
    assert r.status.item() == 0
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))


def test_routing_calls_share_a_plan():
    """One plan buffer, sized for the largest shape, serves routing and forward
    calls of any length and routing path in any order (short batches, the
    per-chunk path, 32-row tiles with XCD schedules): each result equals the one
    on a fresh plan, bit for bit."""
    cases = [("decode_t32", None), ("prefill_t2048", 100), ("decode_t32", None), ("prefill_t2048", 2048),
             ("prefill_t2048", 48), ("decode_t32", None), ("prefill_t2048", 1)]
    inps = [synth.make_inputs(c) if T is None else synth.make_inputs(c, T=T) for c, T in cases]
    plan = torch.empty(max(moe.plan_bytes(moe.shape_of(i["shape"])) for i in inps), dtype=torch.uint8, device=DEV)
    for inp in inps:
        s = inp["shape"]
        say(f"T={s.T}: fresh plan vs the shared one")
        fresh = run_gpu(inp)
        r = moe.alloc_routing(moe.shape_of(s), DEV)
        r.plan = plan
        shared = run_gpu(inp, routing=r)
        for n in ("topk_idx", "counts", "offsets", "perm", "inv_perm", "status"):
            assert np.array_equal(fresh[n], shared[n]), n
        for n in ("topk_w", "logits", "y"):
            assert np.array_equal(fresh[n].view(np.uint32), shared[n].view(np.uint32)), n


def test_forward_wait_timeout_is_reported_and_sticky():
    """The one-launch expert kernel's bounded wait, forced to run out from the
    host (MOE_FORWARD_TEST_WAIT_TIMEOUT: each down block waits for one gate/up
    block more than its tile has, 16 polls): the launch ends normally and sets
    MOE_ERR_DEVICE_SYNC in the status word and in the sticky forward status.
    A routing call then resets the status word and rebuilds the plan, the next
    forward is bitwise a clean run's, and the sticky word still holds the
    failure until the caller clears it."""
    inp = synth.make_inputs("decode_t32")
    s = inp["shape"]
    say("decode_t32: fused expert launch with its waits forced to run out (16 polls), then a clean call")
    shape = moe.shape_of(s)
    dev = gpu_inputs(inp)
    ref = run_gpu(inp, dev=dev)
    r = moe.alloc_routing(shape, DEV)
    ws = moe.alloc_workspace(shape, DEV)
    y = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=DEV)
    b = moe.Bound(shape, dev, dev["x"], r, y, ws)
    b.route()
    b.forward(moe.STAGE_ALL | moe.FORWARD_TEST_WAIT_TIMEOUT)
    torch.cuda.synchronize()
    assert r.status.item() == moe.MOE_ERR_DEVICE_SYNC
    assert r.forward_status.item() == moe.MOE_ERR_DEVICE_SYNC
    b.route()
    b.forward()
    torch.cuda.synchronize()
    assert r.status.item() == moe.MOE_OK
    assert r.forward_status.item() == moe.MOE_ERR_DEVICE_SYNC  # sticky until the caller clears it
    assert np.array_equal(y.float().cpu().numpy().view(np.uint32), ref["y"].view(np.uint32))
    r.forward_status.zero_()
    b.forward()
    torch.cuda.synchronize()
    assert r.status.item() == moe.MOE_OK and r.forward_status.item() == moe.MOE_OK


# ------------------------------------------------------------------ tiled weight layout

def test_pack_weights_layout():
    """moe_pack_weights against the documented tile layout, rebuilt on the host."""
    n, rows, rb = 3, 48, 384
    src = torch.randint(0, 256, (n, rows, rb), dtype=torch.uint8)
    say(f"pack {n} x {rows} x {rb} bytes")
    got = moe.pack_weights(src.to(DEV)).cpu().numpy().reshape(n, -1)
    a = src.numpy()
    want = np.empty_like(got)
    nkb = rb // 128
    for m in range(n):
        for rt in range(rows // 16):
            for kb in range(nkb):
                base = 2048 * (rt * nkb + kb)
                for h in range(2):
                    for l in range(64):
                        o = base + 1024 * h + 16 * l
                        c = 128 * kb + 16 * (l // 16) + 64 * h
                        want[m, o:o + 16] = a[m, 16 * rt + l % 16, c:c + 16]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case,T", [("decode_t32", None), ("prefill_t2048", 700), ("ties_t256_bf16w", None),
                                    ("decode_t32_w8a16", None), ("skew_t8192", 4000)])
def test_tiled_layout_matches_rowmajor(case, T):
    """The same layer with packed weights gives the same bits as with row-major ones."""
    inp = synth.make_inputs(case, T=T)
    s = inp["shape"]
    say(f"{case} T={s.T}: tiled weights == row-major weights, bitwise")
    dev = gpu_inputs(inp)
    packed = moe.pack_layer_weights(dev)
    ys = []
    for layout, w in (("rowmajor", dev), ("tiled", packed)):
        shape = moe.shape_of(s, layout=layout)
        r = moe.alloc_routing(shape, DEV)
        ws = moe.alloc_workspace(shape, DEV)
        y = torch.empty((s.T, s.d), dtype=torch.bfloat16, device=DEV)
        moe.route(shape, w, w["x"], r, ws)
        moe.forward(shape, w, w["x"], r, y, ws)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))


# ------------------------------------------------------------------ the two long-batch routers

def test_long_batch_routers_agree_bitwise():
    """From 4096 tokens the router runs in 128-token blocks of 64 x 32 products
    per wave, below that in 64-token blocks: the same tokens give the same
    logits, ids and weights, bit for bit, on every one of 4095 tokens."""
    big = synth.make_inputs("skew_t8192", T=4096)
    small = synth.make_inputs("skew_t8192", T=4095)
    say("skew layer: 4096 tokens (128-token router blocks) vs their first 4095 (64-token blocks)")
    g1, g2 = run_gpu(big), run_gpu(small)
    n = 4095
    assert np.array_equal(g1["logits"][:n].view(np.uint32), g2["logits"].view(np.uint32))
    assert np.array_equal(g1["topk_idx"][:n], g2["topk_idx"])
    assert np.array_equal(g1["topk_w"][:n].view(np.uint32), g2["topk_w"].view(np.uint32))


# ------------------------------------------------------------------ batch invariance

@pytest.mark.parametrize("T_big", [300, 2048, 8192])
def test_batch_invariance(T_big):
    """A token's logits, ids, weights and output do not depend on the batch it
    sits in: the 32 decode tokens alone (short-batch kernels, 16-row tiles) and
    as the first rows of a larger batch (long-batch router; at T=2048 32-row
    tiles and the XCD schedule, at T=8192 with many tiles per expert) give the
    same bits.  (The pages' port drifted
    when only the prefill chunk size changed: "We Ported Aleph Alpha's Kolibri
    to a MacBook. Our Own Gate Said No.", section "Taking it apart".)"""
    small = synth.make_inputs("decode_t32")
    big = synth.make_inputs("prefill_t2048", T=T_big)
    s = small["shape"]
    big = dict(big)
    xb = big["x"].copy()
    xb[: s.T] = small["x"]
    big["x"] = xb
    say(f"decode_t32 alone vs inside a T={T_big} batch")
    g1 = run_gpu(small)
    g2 = run_gpu(big)
    assert np.array_equal(g1["logits"].view(np.uint32), g2["logits"][: s.T].view(np.uint32))
    assert np.array_equal(g1["topk_idx"], g2["topk_idx"][: s.T])
    assert np.array_equal(g1["topk_w"].view(np.uint32), g2["topk_w"][: s.T].view(np.uint32))
    assert np.array_equal(g1["y"].view(np.uint32), g2["y"][: s.T].view(np.uint32))
