"""Seeded synthetic inputs for one mixture-of-experts layer.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It only *draws* inputs; it holds none of the layer's arithmetic
(no routing, no top-k, no quantisation of activations, no expert FFN).
The one transformation it applies, turning the normal base draws of the
expert weights into FP8 E4M3 codes with one fp32 scale per 128x128 block,
produces the layer's *inputs* (the weights arrive quantised) and uses
torch's own float8_e4m3fn conversion.

Workloads (all seeded, all synthetic; the pages publish neither weights nor
per-layer inputs):

* ``tiny_f32``      T=64, d=256, E=16, k=2, F=Fs=128, everything fp32.
* ``decode_t32``    T=32 on the large layer: d=2048, E=384, k=6, F=Fs=640,
                    FP8 E4M3 weights with fp32 128x128 block scales, bf16
                    activations, fp32 router.
* ``prefill_t2048`` T=2048 on the same layer; the caller forces routing from
                    the choices a free routing pass recorded.
* ``skew_t8192``    T=8192 on the same layer, plus a per-expert selection
                    bias -1.1*ln(rank) (the log-pmf of Zipf(1.1) over a
                    seeded ranking of the experts), so a few experts draw
                    far more than the mean number of tokens.
* ``ties_t256``     T=256 on the same layer with integer activations in
                    [-3, 3] and router weights on a 1/64 grid, so every logit
                    is an exact multiple of 1/64 and top-k ties are common.
* ``ties_t256_bf16w`` the same, with bf16 expert weights rounded from the
                    same base draws instead of FP8 codes.
* ``decode_t32_w8a16`` the decode batch with the same FP8 weights used as
                    W8A16: activations enter both projections in bf16,
                    unquantised.
* ``decode_t32_u4`` the decode batch with 4-bit weights: the same base draws
                    quantised per row and group of 64 columns as
                    round((w - min) / scale) with scale = (max - min) / 15 and
                    bias = min (both bf16), two codes to a byte, the even column
                    in the low nibble; activations enter in bf16.

Per-layer shapes are the large Kolibri-style layer of "We Ported Aleph
Alpha's Kolibri to a MacBook. Our Own Gate Said No." (section "The gate":
384 experts scored per token, top 6, one shared expert); d_model, the FFN
width and the SwiGLU shape are this project's synthetic choices.
"""
from __future__ import annotations

import dataclasses
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = ["LayerShape", "CASES", "make_inputs", "bf16_bits", "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    T: int
    d: int
    E: int
    k: int
    F: int
    Fs: int
    act: str  # "f32" | "bf16"
    w: str  # "f32" | "bf16" | "fp8" | "fp8a16" (the same FP8 weights, activations not quantised) | "u4"

    @property
    def P(self) -> int:
        return self.T * self.k


_TINY = dict(d=256, E=16, k=2, F=128, Fs=128)
_BIG = dict(d=2048, E=384, k=6, F=640, Fs=640)

# name -> (layer id, default T, activation dtype, weight dtype, x recipe, router recipe, bias)
CASES = {
    "tiny_f32": ("tiny", 64, "f32", "f32", "normal", "normal", False),
    "decode_t32": ("big", 32, "bf16", "fp8", "normal", "normal", False),
    "prefill_t2048": ("big", 2048, "bf16", "fp8", "normal", "normal", False),
    "skew_t8192": ("big", 8192, "bf16", "fp8", "normal", "normal", True),
    "ties_t256": ("big", 256, "bf16", "fp8", "int3", "grid64", False),
    "decode_t32_w8a16": ("big", 32, "bf16", "fp8a16", "normal", "normal", False),
    "decode_t32_u4": ("big", 32, "bf16", "u4", "normal", "normal", False),
    "ties_t256_bf16w": ("big", 256, "bf16", "bf16", "int3", "grid64", False),
    # the one batch size of this layer where the matrix-core work outweighs the weight stream
    "prefill_t32768": ("big", 32768, "bf16", "fp8", "normal", "normal", False),
}

# Sub-stream identifiers: every tensor (and every expert of a tensor) draws from
# its own seeded stream, so huge tensors are produced expert by expert and the
# result does not depend on thread scheduling.
_CASE_CODE = {name: i + 1 for i, name in enumerate(CASES)}
_T_X, _T_ROUTER, _T_BIAS, _T_GATE, _T_UP, _T_DOWN = 1, 2, 3, 10, 11, 12
_SHARED = 1 << 20  # expert slot used for the shared expert's streams
_LAYER_CODE = {"tiny": 1, "big": 2}

_WEIGHT_STD = 0.02
_ROUTER_STD = 0.05


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def fp8_blocks(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise a [R, C] fp32 weight (R, C multiples of 128) to E4M3 codes plus
    one fp32 scale per 128x128 block, scale = amax(block) / 448, so that
    weight ~= decode(code) * scale."""
    R, C = w.shape
    blk = w.reshape(R // 128, 128, C // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = blk / scale[:, None, :, None]
    q = np.clip(q, -448.0, 448.0).astype(np.float32).reshape(R, C)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def u4_groups(w: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantise a [R, C] fp32 weight (C a multiple of 64) to 4-bit affine groups:
    per row and group of 64 columns, scale = bf16((max - min) / 15) and bias =
    bf16(min); q = clip(round((w - bias) / scale), 0, 15), two codes to a byte
    with the even column in the low nibble.  Returns (codes [R, C/2] uint8,
    scales and biases [R, C/64] as bf16 bits); weight ~= scale * q + bias."""
    R, C = w.shape
    g = w.reshape(R, C // 64, 64)
    lo, hi = g.min(axis=2), g.max(axis=2)
    scale_b = bf16_bits(np.maximum((hi - lo) / np.float32(15.0), np.float32(1e-8)))
    bias_b = bf16_bits(lo)
    sc, bi = bf16_bits_to_f32(scale_b), bf16_bits_to_f32(bias_b)
    q = np.clip(np.rint((g - bi[:, :, None]) / sc[:, :, None]), 0, 15).astype(np.uint8).reshape(R, C)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, scale_b, bias_b


_layer_cache: dict = {}
_layer_lock = threading.Lock()


def _expert_weights(layer: str, seed: int, w_dtype: str) -> dict:
    """Expert and shared-expert weights of one layer, cached per process."""
    key = (layer, seed, w_dtype)
    with _layer_lock:
        if key in _layer_cache:
            return _layer_cache[key]
    dims = _TINY if layer == "tiny" else _BIG
    d, E, F, Fs = dims["d"], dims["E"], dims["F"], dims["Fs"]
    lc = _LAYER_CODE[layer]
    std = np.float32(_WEIGHT_STD)

    def draw(tensor: int, e: int, shape) -> np.ndarray:
        return _rng(seed, lc, tensor, e).standard_normal(shape, dtype=np.float32) * std

    out: dict = {}
    if w_dtype == "f32":
        wdt, sh = np.float32, None
    elif w_dtype == "bf16":
        wdt, sh = np.uint16, None
    elif w_dtype in ("fp8", "u4"):
        wdt = np.uint8
    else:
        raise ValueError(w_dtype)
    cdiv = 2 if w_dtype == "u4" else 1  # 4-bit codes: two to a byte
    out["w_gate"] = np.empty((E, F, d // cdiv), wdt)
    out["w_up"] = np.empty((E, F, d // cdiv), wdt)
    out["w_down"] = np.empty((E, d, F // cdiv), wdt)
    if w_dtype == "fp8":
        out["s_gate"] = np.empty((E, F // 128, d // 128), np.float32)
        out["s_up"] = np.empty((E, F // 128, d // 128), np.float32)
        out["s_down"] = np.empty((E, d // 128, F // 128), np.float32)
    if w_dtype == "u4":
        for p in ("s_", "b_"):
            out[p + "gate"] = np.empty((E, F, d // 64), np.uint16)
            out[p + "up"] = np.empty((E, F, d // 64), np.uint16)
            out[p + "down"] = np.empty((E, d, F // 64), np.uint16)

    def convert(w: np.ndarray):
        if w_dtype == "f32":
            return w, None, None
        if w_dtype == "bf16":
            return bf16_bits(w), None, None
        if w_dtype == "u4":
            return u4_groups(w)
        return (*fp8_blocks(w), None)

    def one(e: int):
        for name, tensor, shape in (("gate", _T_GATE, (F, d)), ("up", _T_UP, (F, d)), ("down", _T_DOWN, (d, F))):
            c, s, b = convert(draw(tensor, e, shape))
            out["w_" + name][e] = c
            if s is not None:
                out["s_" + name][e] = s
            if b is not None:
                out["b_" + name][e] = b

    with ThreadPoolExecutor(max_workers=min(16, max(1, torch.get_num_threads()))) as ex:
        list(ex.map(one, range(E)))

    for name, tensor, shape in (("gate", _T_GATE, (Fs, d)), ("up", _T_UP, (Fs, d)), ("down", _T_DOWN, (d, Fs))):
        c, s, b = convert(draw(tensor, _SHARED, shape))
        out["sh_" + name] = c
        out["ss_" + name] = s
        if b is not None:
            out["sb_" + name] = b
    with _layer_lock:
        _layer_cache[key] = out
    return out


def make_inputs(case: str, T: int | None = None, seed: int = 0) -> dict:
    """All inputs of one workload as numpy arrays.

    Keys: ``shape`` (LayerShape), ``x`` ([T,d] float32, or uint16 bf16 bits),
    ``w_router`` ([E,d] float32), ``sel_bias`` ([E] float32 or None),
    ``w_gate``/``w_up`` ([E,F,d]), ``w_down`` ([E,d,F]) as float32, uint16 bf16
    bits or uint8 E4M3 codes, ``s_gate``/``s_up`` ([E,F/128,d/128]) and
    ``s_down`` ([E,d/128,F/128]) fp32 block scales (FP8 only, else absent);
    4-bit weights: ``w_*`` codes [E,F,d/2] / [E,d,F/2] uint8 and bf16-bit
    group scales ``s_*`` and biases ``b_*`` ([E,F,d/64] / [E,d,F/64]),
    ``sh_gate``/``sh_up`` ([Fs,d]), ``sh_down`` ([d,Fs]) and their scales
    ``ss_*`` (and 4-bit biases ``sb_*``) for the shared expert.  Rows of ``x`` for a smaller ``T`` are a
    prefix of those for a larger one.
    """
    layer, T0, act, w_dtype, x_recipe, r_recipe, with_bias = CASES[case]
    T = T0 if T is None else int(T)
    dims = _TINY if layer == "tiny" else _BIG
    shape = LayerShape(T=T, act=act, w=w_dtype, **dims)
    cc = _CASE_CODE[case]
    d, E = shape.d, shape.E

    rx = _rng(seed, cc, _T_X)
    if x_recipe == "normal":
        x = rx.standard_normal((T, d), dtype=np.float32)
    else:  # integers in [-3, 3]: exact in bf16, exact products with a 1/64 grid
        x = np.clip(np.rint(rx.standard_normal((T, d), dtype=np.float32)), -3, 3).astype(np.float32)
    x = x if act == "f32" else bf16_bits(x)

    rr = _rng(seed, _LAYER_CODE[layer], _T_ROUTER, 0 if r_recipe == "normal" else 1)
    if r_recipe == "normal":
        w_router = rr.standard_normal((E, d), dtype=np.float32) * np.float32(_ROUTER_STD)
    else:
        w_router = (np.rint(64.0 * 0.01 * rr.standard_normal((E, d))) / 64.0).astype(np.float32)

    sel_bias = None
    if with_bias:
        ranks = _rng(seed, cc, _T_BIAS).permutation(E) + 1
        sel_bias = (-1.1 * np.log(ranks.astype(np.float64))).astype(np.float32)

    out = dict(shape=shape, x=x, w_router=np.ascontiguousarray(w_router), sel_bias=sel_bias)
    out.update(_expert_weights(layer, seed, "fp8" if w_dtype == "fp8a16" else w_dtype))
    return out


def to_device(inp: dict, device="cuda") -> dict:
    """The workload's arrays as torch tensors on `device`, keyed like the C ABI's
    moe_weights fields plus ``x``: bf16 bit patterns become torch.bfloat16,
    E4M3 codes stay uint8."""
    out = {}
    for k, v in inp.items():
        if not isinstance(v, np.ndarray):
            continue
        if v.dtype == np.uint16:
            t = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(v)
        out[k] = t.to(device)
    return out
