"""Pins of the oracle's one-row-per-position full-layer cache ("vrow").

Gemma-4-12B-CoreAI card, "The per-tier cost": the full layers' K/V pair is the
KV term that grows with the context, and cutting it is an open lever.
gemma4-12b card, architecture notes: on a full layer V is the scale-free
RMSNorm of the raw k projection and K the k_norm-weighted RMSNorm of the same
row, rotated, so K = RoPE(w * V) and the V row alone determines both.  The
reading: the key is formed from the stored fp16 row at full precision.

Pins: an exact reduction to the K/V-pair oracle where the formed key is an
fp16 value (no rotation, power-of-two weights), a brute-force fp64 evaluation
with explicit 2x2 rotations on tiny inputs, and the step: a vrow model against
a pair model whose K rows hold the same keys rounded to fp16.
"""
import copy

import numpy as np
import pytest

from int4_q4_gemv_amd import synth
from test_oracle_model import build_oracle_model


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def from16(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_reduces_to_pair_layout_when_the_key_is_exact(orc):
    rng = np.random.default_rng(0)
    n, Hq, D, cap, pos0 = 3, 4, 64, 90, 70
    q = f16(rng.normal(0, 1, (n, Hq, D)))
    v = f16(rng.normal(0, 1, (cap, D)))
    kw = (2.0 ** rng.integers(-2, 3, D)).astype(np.float32)     # kw * v stays an fp16 value
    k = f16(from16(v) * kw.astype(np.float64))
    assert np.array_equal(from16(k), from16(v) * kw)
    got = orc.flash_full_vrow(q, v, kw, 1e6, 0, pos0, 1.0)
    ref = orc.flash_full(q, k, v, pos0, 1.0)
    assert np.array_equal(got, ref)
    # the same rows with a rotation differ: rot_pairs is honoured
    assert not np.allclose(orc.flash_full_vrow(q, v, kw, 1e6, 8, pos0, 1.0), ref)


def brute_force(q16, v16, kw, theta, rot, pos0, scale):
    q, v = from16(q16), from16(v16)
    n, Hq, D = q.shape
    half = D // 2
    out = np.zeros((n, Hq, D))
    for i in range(n):
        P = pos0 + i
        keys = np.empty((P + 1, D))
        for t in range(P + 1):
            x = v[t] * kw.astype(np.float64)
            for p in range(rot):
                a = t * theta ** (-2.0 * p / D)
                R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
                x[p], x[p + half] = R @ np.array([x[p], x[p + half]])
            keys[t] = x
        s = scale * (q[i] @ keys.T)                       # [Hq, P+1]
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[i] = (e @ v[:P + 1]) / e.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("D,rot,theta,pos0,n", [(64, 8, 1e4, 40, 2), (128, 16, 1e6, 77, 4), (32, 16, 1e4, 0, 3)])
def test_matches_brute_force_rotation(orc, D, rot, theta, pos0, n):
    rng = np.random.default_rng(D + rot)
    Hq, cap = 3, pos0 + n + 5
    q = f16(rng.normal(0, 1, (n, Hq, D)))
    v = f16(rng.normal(0, 1, (cap, D)))
    kw = rng.normal(1.0, 0.1, D).astype(np.float32)
    got = orc.flash_full_vrow(q, v, kw, theta, rot, pos0, 0.3)
    ref = brute_force(q, v, kw, theta, rot, pos0, 0.3)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_row_rule_ignores_rows_past_the_position(orc):
    rng = np.random.default_rng(5)
    n, Hq, D, cap, pos0 = 2, 2, 64, 64, 20
    q = f16(rng.normal(0, 1, (n, Hq, D)))
    v = f16(rng.normal(0, 1, (cap, D)))
    kw = np.ones(D, np.float32)
    a = orc.flash_full_vrow(q, v, kw, 1e4, 32, pos0, 1.0)
    v2 = v.copy()
    v2[pos0 + n:] = f16(np.full((cap - pos0 - n, D), 6e4))     # poison past the last row
    assert np.array_equal(orc.flash_full_vrow(q, v2, kw, 1e4, 32, pos0, 1.0), a)
    v2[pos0] = f16(rng.normal(0, 1, D))                          # row 0 of the block sees pos0
    b = orc.flash_full_vrow(q, v2, kw, 1e4, 32, pos0, 1.0)
    assert not np.allclose(b[0], a[0])


def pair_from_vrow(orc, cfg, m, ctx):
    """The pair-layout model whose full-layer K rows are fp16(RoPE_t(w * v_t))
    of the same V rows: the keys the vrow model forms, rounded to fp16."""
    p = copy.copy(m)
    p.kv_format = 0
    p.layers = [copy.copy(L) for L in m.layers]
    for L in p.layers:
        L.v_cache = L.v_cache.copy()
        if L.is_full:
            D = cfg.full_head_dim
            k = np.zeros_like(L.v_cache)
            for t in range(ctx):
                x = from16(L.v_cache[t]) * L.k_norm.astype(np.float64)
                k[t] = orc.f64_to_f16(orc.rope(x, t, cfg.full_theta, cfg.full_rot_pairs))
            L.k_cache = k
        else:
            L.k_cache = L.k_cache.copy()
    return p


def vrow_model(orc, cfg, seed, ctx):
    m = build_oracle_model(orc, cfg, seed, ctx)
    m.kv_format = 1
    for L in m.layers:
        if L.is_full:
            L.k_cache = None
    return m


def test_step_matches_pair_layout_up_to_key_rounding(orc):
    cfg, ctx = synth.TOY, 180
    m = vrow_model(orc, cfg, 11, ctx)
    p = pair_from_vrow(orc, cfg, m, ctx)
    toks = synth.tokens(cfg, 4, 11)
    lv, av = m.decode_step(toks, ctx)
    lp, ap = p.decode_step(toks, ctx)
    # the caches agree: the vrow model wrote only V rows, the same ones
    for Lv, Lp in zip(m.layers, p.layers):
        assert np.array_equal(Lv.v_cache, Lp.v_cache)
    err = np.abs(lv - lp).max()
    assert err < 5e-3 * np.abs(lp).max(), err
    assert err > 0                                        # the keys really differ by rounding
    # a model that forgets the weights (w = 1) is far off
    w1 = copy.copy(m)
    w1.layers = [copy.copy(L) for L in m.layers]
    for L in w1.layers:
        L.v_cache = L.v_cache.copy()
    w1.layers[1].k_norm = np.ones_like(w1.layers[1].k_norm)
    lw, _ = w1.decode_step(toks, ctx)
    assert np.abs(lw - lp).max() > 10 * err


def test_vrow_needs_v_norm_on_full_layers(orc):
    cfg = synth.TOY
    m = vrow_model(orc, cfg, 12, 100)
    m.layers[1].v_norm = False
    with pytest.raises(ValueError):
        m.decode_step(synth.tokens(cfg, 1, 12), 100)
