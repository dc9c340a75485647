#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step = the whole hot path on one batch: router + top-k + dispatch
(moe_route, or moe_route_forced when the workload replays recorded choices)
then the expert FFNs and the combine (moe_forward).  Inputs and weights are
resident in HBM before timing starts; the expert weights are packed once into
the library's tiled layout (moe_pack_weights, a load-time step outside the
timed region) and rotate over several device copies so every step streams
them from HBM rather than from the 256 MB last-level cache.

Prints one JSON line.  `value` is tokens/s of the whole step; `roofline` is
for the dominant kernel (at decode the fused expert kernel: grouped gate/up,
SwiGLU and down projections in one launch), from its average launch duration
(back-to-back launches between two HIP events on the stream it runs on);
`stage_us` attributes the step to its stages with events between them, which
add a few microseconds each (with the fused kernel, `gate_up` holds both
projections and `down` is empty); `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 matrix
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector
METRIC = "MoE-layer tokens/s (decode T=32, prefill T=2048); % HBM BW / % FP8 MFMA peak"

DESCRIPTION = {
    "decode_t32": "decode batch, T=32 tokens, d=2048, E=384 experts, top-6, SwiGLU F=640 + shared F=640, "
                  "FP8 E4M3 128x128-block-scaled expert weights, bf16 activations, fp32 router, free routing",
    "prefill_t2048": "prefill chunk, T=2048 tokens, same layer, routing forced from ids recorded by a free pass",
    "skew_t8192": "skewed prefill, T=8192 tokens, same layer, Zipf(1.1) selection bias, free routing",
    "ties_t256": "near-tie batch, T=256, integer activations, 1/64-grid router, free routing",
    "ties_t256_bf16w": "near-tie batch, T=256, bf16 expert weights, free routing",
    "decode_t32_w8a16": "decode batch, T=32, the same FP8 weights used as W8A16 (bf16 activations into both "
                        "projections, unquantised), free routing",
    "decode_t32_u4": "decode batch, T=32, the same layer with 4-bit affine group-quantised expert weights (bf16 "
                     "scale and bias per row and 64 columns), bf16 activations, free routing",
    "tiny_f32": "tiny fp32 layer, T=64, d=256, E=16, top-2, F=Fs=128, free routing (latency-bound; no roofline "
                "claim)",
    "prefill_t32768": "long prefill, T=32768 tokens, same layer as decode, free routing: the only batch size of "
                      "this layer whose matrix-core work (F_mm at the FP8 peak) outweighs its weight stream",
}
FORCED = {"prefill_t2048"}

# HBM bytes per launch of the fused expert kernel on the default workload, from two
# rocprofv3 --pmc passes over this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by what the counter reads for the 480 MiB weight copies
# the same run makes (fetch x2.0, write x1.0).  Valid only for the kernel sources
# they were taken on: any change to them makes `traffic` null until re-measured.
KERNEL_SOURCES = ("mixture_experts_moe_amd/csrc/experts.hip", "mixture_experts_moe_amd/csrc/moe_device.h",
                  "mixture_experts_moe_amd/csrc/moe_kernels.h", "mixture_experts_moe_amd/csrc/moe_api.hip")
TRAFFIC = {  # workload -> counters of the fused expert kernel, tiled layout
    "decode_t32": {"sources_sha256": "47fe357800ffc8e63657776bf2711fac2f33aead0cbc5d729f9fd36740dcff94",
                   "fetch_bytes": 607132445, "write_bytes": 2227088},
}


def sources_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    t = TRAFFIC.get(workload)
    if t is None or t["sources_sha256"] != sources_sha256():
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t32", choices=sorted(DESCRIPTION))
    ap.add_argument("--rotate", type=int, default=4, help="device copies of the expert weights")
    ap.add_argument("--layout", default="tiled", choices=("tiled", "rowmajor"), help="expert-weight layout")
    ap.add_argument("--attention", type=int, default=1, help="time the attention ops next to the layer (0: skip)")
    ap.add_argument("--compare", default="skew_t8192",
                    help="workload whose routing moe_route_compare is timed on ('' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget (0: skip)")
    ap.add_argument("--also", default="prefill_t2048,skew_t8192,ties_t256,ties_t256_bf16w,decode_t32_w8a16,"
                    "decode_t32_u4,tiny_f32,prefill_t32768", help="extra workloads timed after the main one (comma list)")
    return ap.parse_args()


def algorithmic(s, counts):
    """Algorithmic bytes and flops (what the method must move / compute)."""
    bw = {"fp8": 1, "fp8a16": 1, "bf16": 2, "f32": 4, "u4": 0.5}[s.w]
    ba = {"bf16": 2, "f32": 4}[s.act]
    U = int((counts > 0).sum())
    P = s.T * s.k
    fp8 = s.w == "fp8"                # activations and h quantised to E4M3
    scaled = s.w in ("fp8", "fp8a16")  # block-scaled FP8 weights

    def nb(r, c):  # scale bytes: fp32 per 128x128 block, or a bf16 scale and bias per row and 64 columns
        return (r // 128) * (c // 128) * 4 if scaled else (r * (c // 64) * 4 if s.w == "u4" else 0)
    gu_w = int(U * 2 * (s.F * s.d * bw + nb(s.F, s.d)) + 2 * (s.Fs * s.d * bw + nb(s.Fs, s.d)))
    dn_w = int(U * (s.d * s.F * bw + nb(s.d, s.F)) + (s.d * s.Fs * bw + nb(s.d, s.Fs)))
    act_in = s.T * s.d + s.T * (s.d // 128) * 4 if fp8 else s.T * s.d * ba
    h_rows = P + s.T
    h_bytes = h_rows * s.F * (1 if fp8 else 2) + (h_rows * (s.F // 128) * 4 if fp8 else 0)
    return {
        "U": U,
        "gateup_bytes": gu_w + act_in + h_bytes,
        "down_bytes": dn_w + h_bytes + h_rows * s.d * 4,
        "B_alg": gu_w + dn_w + 4 * s.E * s.d + 2 * s.T * s.d * ba,
        "F_mm": 2 * (P + s.T) * 3 * s.d * s.F,
        "F_router": 2 * s.T * s.d * s.E,
    }


def step_roofline(s, alg, t_step):
    """Step figures against the chip's peaks.  The products run on the bf16
    matrix cores (FP8 codes and 4-bit codes are decoded exactly to bf16 in
    registers), so the matrix-core fraction is against the dense bf16 peak;
    fp32 layers run on the vector ALUs.  `fp8_equiv_mfma_frac` is the same work
    against the dense FP8 peak, the figure a path on the FP8 instruction would
    be held to; it is labelled as such and not the bound of these kernels."""
    hbm = alg["B_alg"] / (HBM_PEAK_GBS * 1e9)
    mm_peak = FP32_PEAK_TFLOPS if s.w == "f32" else BF16_PEAK_TFLOPS
    mm = alg["F_mm"] / (mm_peak * 1e12)
    return {"B_alg_bytes": alg["B_alg"], "F_mm_flops": alg["F_mm"], "distinct_experts": alg["U"],
            "hbm_frac": hbm / t_step,
            "mfma_frac": mm / t_step, "mfma_peak_tflops": mm_peak,
            "mfma_unit": "fp32 vector ALU" if s.w == "f32" else "bf16 matrix cores (decoded weight codes)",
            "fp8_equiv_mfma_frac": alg["F_mm"] / t_step / (FP8_PEAK_TFLOPS * 1e12),
            "bound": "hbm" if hbm >= mm else "mfma",
            "roofline_frac": max(hbm, mm) / t_step}


def run_workload(name, steps, warmup, rotate, layout):
    import torch
    from mixture_experts_moe_amd import moe, synth

    print(f"bench: {name}: {steps} steps after {warmup} warm-up", file=sys.stderr, flush=True)
    inp = synth.make_inputs(name)
    s = inp["shape"]
    dev = synth.to_device(inp, "cuda:0")
    if s.w == "f32":
        layout = "rowmajor"  # fp32 weights have no tiled layout
    if layout == "tiled":
        dev = moe.pack_layer_weights(dev)
    shape = moe.shape_of(s, layout=layout)
    # every weight tensor rotates: routed and shared expert matrices, their block
    # scales or group parameters, the router and the selection bias
    wkeys = [k for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
                         "ss_gate", "ss_up", "ss_down", "w_router", "w_router_planes", "sel_bias")
             if dev.get(k) is not None]
    copies = [dev] + [dict(dev, **{k: dev[k].clone() for k in wkeys}) for _ in range(max(0, rotate - 1))]
    r = moe.alloc_routing(shape, "cuda:0")
    ws = moe.alloc_workspace(shape, "cuda:0")
    y = torch.empty((s.T, s.d), dtype=torch.bfloat16 if s.act == "bf16" else torch.float32, device="cuda:0")
    forced = None
    if name in FORCED:  # record the choices of a free routing pass, then replay them
        moe.route(shape, dev, dev["x"], r, ws)
        torch.cuda.synchronize()
        forced = r.topk_idx.clone()

    st = torch.cuda.current_stream()
    bound = [moe.Bound(shape, w, w["x"], r, y, ws, forced_idx=forced, stream=st) for w in copies]

    def step(i):
        b = bound[i % len(bound)]
        b.route()
        b.forward()

    def check_status(what):
        # the routing status word (reset by every routing call) and the sticky
        # forward status (set by any forward call whose bounded wait ran out)
        assert r.status.item() == moe.MOE_OK, f"{name} {what}: {moe.status_string(r.status.item())}"
        assert r.forward_status.item() == moe.MOE_OK, f"{name} {what}: {moe.status_string(r.forward_status.item())}"

    # timed pass: one routing call and one forward call per step
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    check_status("timed steps")

    # attribution pass (same kernels): events around the routing call, and events
    # the library records on the stream between the forward stages
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for i in range(steps):
        b = bound[i % len(bound)]
        ev[i][0].record(st)
        b.route()
        ev[i][1].record(st)
        b.forward(moe.STAGE_ALL, events=ev[i][2:])
    torch.cuda.synchronize()
    check_status("attribution steps")
    names = ("route", "gate_up", "down", "combine")
    pairs = ((0, 1), (2, 3), (3, 4), (4, 5))
    stage_us = {n: float(np.mean([ev[i][a].elapsed_time(ev[i][b]) for i in range(steps)])) * 1e3
                for n, (a, b) in zip(names, pairs)}
    per_step = np.array([ev[i][0].elapsed_time(ev[i][5]) for i in range(steps)]) * 1e3
    pct = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}

    # launch duration of the expert projections (gate/up + down: one fused
    # kernel for FP8 weights in 16-row tiles, e.g. decode; two kernels
    # otherwise): back-to-back launches on the routing above, rotating over the
    # weight copies, between two events on the same stream.  The stage events
    # above add a few microseconds to each stage; this is the figure rocprofv3
    # reports for the kernel.
    n_l = max(20, steps // 2)
    experts = moe.STAGE_GATE_UP | moe.STAGE_DOWN
    for i in range(3):
        bound[i % len(bound)].forward(experts)
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    l0.record(st)
    for i in range(n_l):
        bound[i % len(bound)].forward(experts)
    l1.record(st)
    torch.cuda.synchronize()
    stage_us["experts_launch"] = l0.elapsed_time(l1) * 1e3 / n_l
    counts = r.counts.cpu().numpy()
    check_status("expert launches")
    return s, wall, stage_us, algorithmic(s, counts), counts, pct


def run_route_compare(name, steps):
    """moe_route_compare of the library's free routing against a torch fp32
    matmul router on the same batch (the pages' routing-as-a-distribution check
    at this batch's size), timed back to back between two events."""
    import torch
    from mixture_experts_moe_amd import moe, synth

    inp = synth.make_inputs(name)
    s = inp["shape"]
    dev = synth.to_device(inp, "cuda:0")
    shape = moe.shape_of(s)
    r = moe.alloc_routing(shape, "cuda:0")
    ws = moe.alloc_workspace(shape, "cuda:0")
    moe.route(shape, dev, dev["x"], r, ws)
    bias = dev.get("sel_bias")
    ref = dev["x"].float() @ dev["w_router"].t()
    ref_ids = torch.sort(-(ref if bias is None else ref + bias), dim=1, stable=True).indices[:, :s.k]
    ref_ids = ref_ids.to(torch.int32).contiguous()
    cmp = moe.RouteCompare(s.T, "cuda:0")
    st = torch.cuda.current_stream()
    for _ in range(5):
        cmp(r.logits, ref, r.topk_idx, ref_ids, bias, st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        cmp(r.logits, ref, r.topk_idx, ref_ids, bias, st)
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # logits and reference logits, both id arrays, the bias, the gaps; the
    # per-token workspace (20 bytes) written and read back
    nbytes = 2 * s.T * s.E * 4 + 2 * s.T * s.k * 4 + s.E * 4 + s.T * 4 + 2 * 20 * s.T
    return {"T": s.T, "E": s.E, "k": s.k, "us_per_call": us, "launches": 3, "bytes": nbytes,
            "GBs": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "sigma": cmp.out.sigma.item(), "disagreement_rate": cmp.out.n_disagree.item() / s.T,
            "max_gap_sigma": cmp.out.max_gap.item(),
            "reference": "torch fp32 matmul router over the whole batch, ids by stable sort"}


# The attention ops next to the layer: 16 query heads, 4 key/value heads,
# head_dim 128, the 513-token window; a prefill chunk of 2048 tokens after 2048
# cached ones, and one decode token after a 32768-token context.
ATTN_CASES = {
    "attn_swa_prefill_t2048": dict(window=513, Tq=2048, Tk=4096, q_pos0=2048),
    "attn_nope_prefill_t2048": dict(window=0, Tq=2048, Tk=4096, q_pos0=2048),
    "attn_nope_decode_ctx32768": dict(window=0, Tq=1, Tk=32768, q_pos0=32767),
}


def run_attention(steps):
    """moe_attention on each case and moe_rope on the prefill chunk's queries
    and keys, back to back between two events, against their rooflines
    (prefill: the matrix cores at the bf16 peak on 4*Tq*keys*D*Hq flops; decode
    and RoPE: HBM on the bytes they must move)."""
    import torch
    from mixture_experts_moe_amd import attn

    Hq, Hkv, D = 16, 4, 128
    g = torch.Generator(device="cuda:0").manual_seed(0)
    out = {}
    st = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    for name, c in ATTN_CASES.items():
        Tq, Tk, q0, Wn = c["Tq"], c["Tk"], c["q_pos0"], c["window"]
        q = torch.randn((Tq, Hq, D), generator=g, device="cuda:0").to(torch.bfloat16)
        k = torch.randn((Tk, Hkv, D), generator=g, device="cuda:0").to(torch.bfloat16)
        v = torch.randn((Tk, Hkv, D), generator=g, device="cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        call = attn.Attention(attn.AttnShape(Hq, Hkv, D, Wn), Tq, Tk, q0)
        us = timed(lambda: call(q, k, v, o, st), max(20, steps))
        pos = q0 + np.arange(Tq)
        lo = np.maximum(0, pos - Wn + 1) if Wn else np.zeros(Tq, np.int64)
        n_keys = float(np.sum(pos - lo + 1))               # attended (query, key) pairs per head
        flops = 4.0 * n_keys * D * Hq
        span = int(pos[-1] + 1 - lo[0])                     # keys any query reads
        nbytes = 2 * Tq * Hq * D * 2 + 2 * span * Hkv * D * 2  # q in, o out, k and v once
        bound = "mfma" if flops / (BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
        r = {"us_per_call": us, "flops": flops, "bytes": nbytes, "bound": bound,
             "TFLOPs": flops / (us * 1e-6) / 1e12, "GBs": nbytes / (us * 1e-6) / 1e9,
             "workspace_bytes": int(call.ws.numel()) if attn.workspace_bytes(call.shape, Tq, Tk, q0) else 0}
        r["frac"] = r["TFLOPs"] / BF16_PEAK_TFLOPS if bound == "mfma" else r["GBs"] / HBM_PEAK_GBS
        out[name] = r
    x = torch.randn((2048, Hq + Hkv, D), generator=g, device="cuda:0").to(torch.bfloat16)
    us = timed(lambda: attn.rope_(x, 2048, 10000.0, st), max(20, steps))
    nbytes = 2 * x.numel() * 2
    out["rope_t2048_20heads"] = {"us_per_call": us, "bytes": nbytes, "bound": "hbm", "GBs": nbytes / (us * 1e-6) / 1e9,
                                 "frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    return out


def host_cpu():
    """The host's logical core count and CPU model (from /proc/cpuinfo)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count() or 1, model


def cpu_baseline(name, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the workload: first
    single-threaded, then its all-cores driver (the same per-token code on
    contiguous token ranges, one std::thread each) on the host's cores, capped at
    16 (a GPU machine's CPU share), whose results must be bitwise the
    single-threaded ones.  `value` is the all-cores rate."""
    from mixture_experts_moe_amd import synth
    from oracle import moe_oracle as O

    inp = synth.make_inputs(name)
    s = inp["shape"]
    L = O.Layer(inp)
    n_cpu, model = host_cpu()
    threads = O.host_threads()

    def run(n_tok, budget, n_threads):
        tok = np.linspace(0, s.T - 1, n_tok).astype(np.int32)
        done, t0, res = 0, time.perf_counter(), None
        while True:
            if n_threads == 1:
                _, lg, idx, w = O.route(L, tok)
                y, acc = O.forward(L, idx, w, tok)
            else:
                _, lg, idx, w = O.route_threads(L, tok, n_threads)
                y, acc = O.forward_threads(L, idx, w, tok, n_threads)
            res = res or (lg, idx, w, y)
            done += n_tok
            el = time.perf_counter() - t0
            if el >= budget:
                return done / el, done // n_tok, el, res

    one, p1, el1, r1 = run(min(s.T, 32), budget_s / 2, 1)
    n_all = min(s.T, 32 * threads)
    many, p2, el2, r2 = run(n_all, budget_s / 2, threads)
    # the first 32 sampled tokens of both runs are the same tokens only when both
    # samples cover the whole batch; compare the all-cores run with a
    # single-threaded pass over its own sample instead
    tok = np.linspace(0, s.T - 1, n_all).astype(np.int32)
    _, lg, idx, w = O.route(L, tok)
    y, _ = O.forward(L, idx, w, tok)
    bitwise = (np.array_equal(lg.view(np.uint32), r2[0].view(np.uint32)) and np.array_equal(idx, r2[1])
               and np.array_equal(w.view(np.uint32), r2[2].view(np.uint32)) and np.array_equal(y, r2[3]))
    assert bitwise, "all-cores oracle differs from the single-threaded oracle"
    return {"value": many, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_logical_cpus": n_cpu, "host_cpu_model": model,
            "single_thread": {"value": one, "unit": "tokens/s", "cores": 1,
                              "sample": f"{p1} passes of route + forward over 32 of the workload's {s.T} tokens "
                                        f"({el1:.1f} s)"},
            "all_cores_bitwise_equal_single_thread": bitwise,
            "sample": f"{p2} passes of route + forward over {n_all} of the workload's {s.T} tokens ({el2:.1f} s) on "
                      f"{threads} threads, contiguous token ranges, C++ oracle with double-accumulated dot "
                      f"products"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the layer on one GPU; --gpus must be 1 (the layer is not sharded across GPUs)", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    s, wall, st_us, alg, counts, pct = run_workload(a.workload, a.steps, a.warmup, a.rotate, a.layout)
    t_step = wall
    ex_bytes = alg["gateup_bytes"] + alg["down_bytes"]
    achieved = ex_bytes / (st_us["experts_launch"] * 1e-6) / 1e9
    out = {
        "metric": METRIC, "value": s.T / t_step, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3" if s.w == "fp8" else s.w, "data": "synthetic",
        "config": {"workload": f"{a.workload}: {DESCRIPTION[a.workload]}", "T": s.T, "d_model": s.d,
                   "n_experts": s.E, "top_k": s.k, "d_ffn": s.F, "d_ffn_shared": s.Fs,
                   "weight_copies_rotated": a.rotate, "weight_layout": a.layout},
        "roofline": {"bound": "hbm",
                     "kernel": "experts_fused_kernel (grouped gate/up + SwiGLU + h quantisation + down x routing "
                               "weight, one launch)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(a.workload) if a.layout == "tiled" else None,
                     "bytes_per_launch": ex_bytes, "avg_launch_us": st_us["experts_launch"]},
        "stage_us": st_us,
        "step_us_event_percentiles": pct,
        "step_roofline": step_roofline(s, alg, t_step),
    }
    extra = {}
    for name in [w for w in a.also.split(",") if w and w != a.workload]:
        s2, wall2, st2, alg2, counts2, pct2 = run_workload(name, max(10, a.steps // 4), max(3, a.warmup // 4),
                                                           a.rotate, a.layout)
        extra[name] = {"tokens_per_s": s2.T / wall2, "ms_per_step": wall2 * 1e3, "stage_us": st2,
                       "step_us_event_percentiles": pct2,
                       "experts_GBs": (alg2["gateup_bytes"] + alg2["down_bytes"]) / (st2["experts_launch"] * 1e-6)
                       / 1e9,
                       **step_roofline(s2, alg2, wall2),
                       "max_over_mean_expert_load": float(counts2.max() / max(1e-9, counts2.mean()))}
    if a.compare:
        print(f"bench: route_compare on {a.compare}", file=sys.stderr, flush=True)
        extra["route_compare_" + a.compare] = run_route_compare(a.compare, max(20, a.steps // 2))
    if a.attention:
        print("bench: attention ops", file=sys.stderr, flush=True)
        extra.update(run_attention(max(20, a.steps // 2)))
    if extra:
        out["also"] = extra
    if a.cpu_seconds > 0:
        print("bench: CPU baseline (the oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(a.workload, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
