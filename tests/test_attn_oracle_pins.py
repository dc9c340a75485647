"""Pins of the attention oracle (rotary position encoding, sliding-window and
whole-context causal attention) against facts that do not come from it:
closed forms, torch's own attention routine in float64, invariants of the
definitions, and planted mutants that each pin must catch -- among them the
"window one token short" bug that "We Ported Aleph Alpha's Kolibri to a
MacBook. Our Own Gate Said No." (section "The gate") planted in its reference.
"""
import numpy as np
import pytest
import torch

from mixture_experts_moe_amd import synth
from oracle import attn_oracle as A

W = 513  # the pages' window ("The gate": a sliding window of 513 tokens)


def _bits(a):
    return synth.bf16_bits(np.asarray(a, np.float32))


def _f(bits):
    return synth.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def test_window_boundary_exact():
    """Uniform attention (q = 0): the output is the mean of v over the attended
    keys.  A query at position 600 sees keys 88..600 (513 of them): a marker at
    key 88 contributes 1/513, one at key 87 and one at key 601 (the future)
    nothing.  A window one token short loses key 88."""
    Tk, D, p = 602, 8, 600
    v = np.zeros((Tk, 1, D), np.float32)
    v[:, 0, 0] = 1.0
    v[p - W + 1, 0, 1] = 1.0
    v[p - W, 0, 2] = 1.0
    v[p + 1, 0, 3] = 1.0
    q = np.zeros((1, 1, D), np.float32)
    k = np.random.default_rng(0).standard_normal((Tk, 1, D)).astype(np.float32)
    o = A.attention(_bits(q), _bits(k), _bits(v), p, W)[0, 0]
    assert abs(o[0] - 1.0) < 1e-7 and abs(o[1] - 1.0 / W) < 1e-9 and o[2] == 0.0 and o[3] == 0.0
    with A.mutant("window_short"):
        assert A.attention(_bits(q), _bits(k), _bits(v), p, W)[0, 0, 1] == 0.0
    # whole context (window 0): every key up to the query, none after it
    o = A.attention(_bits(q), _bits(k), _bits(v), p, 0)[0, 0]
    assert abs(o[1] - 1.0 / (p + 1)) < 1e-9 and abs(o[2] - 1.0 / (p + 1)) < 1e-9 and o[3] == 0.0


@pytest.mark.parametrize("window", [0, 5, W])
def test_attention_vs_torch_sdpa(window):
    """Against torch's scaled_dot_product_attention in float64 with the causal
    (and window) mask written as a boolean matrix, grouped heads expanded."""
    rng = np.random.default_rng(1)
    Tq, Tk, Hq, Hkv, D, q0 = 9, 40, 4, 2, 16, 31
    q, k, v = (_bits(rng.standard_normal(s)) for s in ((Tq, Hq, D), (Tk, Hkv, D), (Tk, Hkv, D)))
    o = A.attention(q, k, v, q0, window)
    pos_q = q0 + np.arange(Tq)[:, None]
    pos_k = np.arange(Tk)[None, :]
    mask = pos_k <= pos_q
    if window:
        mask &= pos_q - pos_k < window
    G = Hq // Hkv
    kt = torch.from_numpy(np.repeat(_f(k), G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(_f(v), G, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(_f(q)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    ref = ref.permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-6 * np.max(np.abs(ref))
    with A.mutant("no_scale"):
        assert np.max(np.abs(A.attention(q, k, v, q0, window) - ref)) > 1e-3


def test_grouped_heads_and_key_order():
    """Head h reads key/value head h // (Hq/Hkv): with constant values per
    key/value head, each query head returns its group's constant.  Without
    positional encoding, a query that sees the whole context is unchanged when
    the keys before it are permuted together with their values."""
    rng = np.random.default_rng(2)
    Tk, Hq, Hkv, D = 20, 6, 3, 8
    v = np.zeros((Tk, Hkv, D), np.float32)
    for g in range(Hkv):
        v[:, g, :] = g + 1
    q = _bits(rng.standard_normal((1, Hq, D)))
    k = _bits(rng.standard_normal((Tk, Hkv, D)))
    o = A.attention(q, k, _bits(v), Tk - 1, 0)[0]
    for h in range(Hq):
        assert np.all(np.abs(o[h] - (h // 2 + 1)) < 1e-6)
    v = _bits(rng.standard_normal((Tk, Hkv, D)))
    perm = np.concatenate([rng.permutation(Tk - 1), [Tk - 1]])
    o1 = A.attention(q, k, v, Tk - 1, 0)
    o2 = A.attention(q, k[perm], v[perm], Tk - 1, 0)
    assert np.max(np.abs(o1 - o2)) <= 1e-6 * np.max(np.abs(o1))


def test_rope_closed_form_and_pairing():
    """D = 2: the pair (x, y) is rotated by the position itself (frequency
    theta^0 = 1).  D = 8: a vector with only dims 0 and 4 set stays in those
    two dims (pairs (j, j + D/2)); the interleaved-pairs and wrong-sign mutants
    change it."""
    theta = 10000.0
    for pos in (0, 1, 7, 1000):
        x = _bits(np.array([[[0.75, -0.5]]]))
        r = _f(A.rope(x, pos, theta))[0, 0]
        c, s = np.cos(pos), np.sin(pos)
        ref = np.array([0.75 * c + 0.5 * s, 0.75 * s - 0.5 * c])
        assert np.all(np.abs(r - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    x = np.zeros((1, 1, 8), np.float32)
    x[0, 0, 0], x[0, 0, 4] = 1.0, 0.5
    r = _f(A.rope(_bits(x), 3, theta))[0, 0]
    assert np.all(r[[1, 2, 3, 5, 6, 7]] == 0) and abs(r[0] - (np.cos(3) - 0.5 * np.sin(3))) < 4e-3
    with A.mutant("rope_interleaved"):
        assert _f(A.rope(_bits(x), 3, theta))[0, 0, 1] != 0
    with A.mutant("rope_sign"):
        assert abs(_f(A.rope(_bits(x), 3, theta))[0, 0, 0] - r[0]) > 0.1


def test_rope_relative_position_and_norm():
    """Rotation keeps each pair's length, and q(m).k(n) depends only on m - n
    (up to the bf16 rounding of the rotated values)."""
    rng = np.random.default_rng(4)
    D, theta = 64, 10000.0
    q = _bits(rng.standard_normal((1, 1, D)))
    k = _bits(rng.standard_normal((1, 1, D)))
    qf, kf = _f(q)[0, 0], _f(k)[0, 0]
    dots = []
    for shift in (0, 5, 1234):
        rq = _f(A.rope(q, 40 + shift, theta))[0, 0]
        rk = _f(A.rope(k, 17 + shift, theta))[0, 0]
        n0 = qf[:32] ** 2 + qf[32:] ** 2
        n1 = rq[:32] ** 2 + rq[32:] ** 2
        assert np.all(np.abs(n1 - n0) <= 2.0 ** -6 * n0 + 1e-12)
        dots.append(rq @ rk)
    scale = np.linalg.norm(qf) * np.linalg.norm(kf)
    assert max(dots) - min(dots) <= 2.0 ** -6 * scale
