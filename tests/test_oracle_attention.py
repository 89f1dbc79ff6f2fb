"""Pins of the oracle's attention and of the sliding-ring admission rule.

Ring rule: Gemma-4-12B-CoreAI card, section "v5/ -- ring extent R = 2W" (a
slot's implied position p = q - ((q - j) mod R) is admitted iff q - p < W) and
gemma-4-E4B-CoreAI card, section "ring/" (written, causal, in-window slots).
Full attention: gemma4-12b card, "The fix" (one global KV head, a decode query
attends every written key, scale 1.0).
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def f16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------------ ring rule ----
def simulate_ring(R, writes):
    """Linear history: each write of position p lands in slot p mod R and
    replaces what was there.  Returns held[j] (or -1) and the number of
    writes that landed on an already-used slot."""
    held = [-1] * R
    on_used = 0
    for p in writes:
        if held[p % R] >= 0:
            on_used += 1
        held[p % R] = p
    return held, on_used


def test_page_count_of_writes_on_used_slots():
    g = GOLD["ring_overwrites"]
    _, on_used = simulate_ring(g["ring_slots"], range(g["tokens"]))
    assert on_used == g["writes_on_used_slot"]


def test_page_wrap_count():
    g = GOLD["ring_wraps"]
    assert g["chunks"] * g["chunk"] == g["prompt_tokens"]
    assert g["prompt_tokens"] + g["decode_steps"] - 1 == g["final_position"]
    assert g["window"] + g["chunk"] == g["ring_slots"]
    wraps = (g["final_position"] + 1) / g["ring_slots"]
    assert round(wraps) == g["wraps_about"]


@pytest.mark.parametrize("W", range(1, 9))
def test_ring_rule_matches_linear_history(orc, W):
    for R in range(W, 21):
        for q in range(0, 3 * R):
            held, _ = simulate_ring(R, range(q + 1))
            truth = np.array([h >= 0 and q - h < W for h in held])
            assert np.array_equal(orc.ring_admit(q, R, W), truth), (W, R, q)


def test_rejected_rows_never_admitted_iff_R_ge_W_plus_n_minus_1(orc):
    """Rows q+1..q+n-1 of a verify block were written then rejected; a query
    at q must admit exactly the slots holding positions in (q-W, q]."""
    for W in range(1, 7):
        for n in range(1, 5):
            for R in range(W, W + 8):
                ok_all = True
                for q in range(0, 3 * R):
                    held, _ = simulate_ring(R, list(range(q + 1)) + list(range(q + 1, q + n)))
                    truth = np.array([0 <= h <= q and q - h < W for h in held])
                    ok_all &= bool(np.array_equal(orc.ring_admit(q, R, W), truth))
                assert ok_all == (R >= W + n - 1), (W, n, R)


def test_ring_of_one_window_admits_a_rejected_row(orc):
    # R = W: a rejected row at q+1 sits at implied position q+1-R, inside the window
    R = W = 16
    q = 40
    adm = orc.ring_admit(q, R, W)
    assert adm[(q + 1) % R]


def test_poisoned_workload_admitted_slots(orc):
    # query 100000, W 1024, R 2048: admitted positions 98977..100000 -> slots 673..1696
    adm = orc.ring_admit(100000, 2048, 1024)
    assert np.array_equal(np.nonzero(adm)[0], np.arange(673, 1697))
    assert not adm[1697:1701].any()


# ------------------------------------------------------------ attention ----
def sdpa_ref(q, k, v, admit, scale):
    """torch's scaled_dot_product_attention in fp64 (library routine)."""
    Hq, D = q.shape
    Hkv = k.shape[0]
    qt = torch.tensor(q, dtype=torch.float64)[:, None, :]            # [Hq, 1, D]
    kt = torch.tensor(k, dtype=torch.float64).repeat_interleave(Hq // Hkv, dim=0)
    vt = torch.tensor(v, dtype=torch.float64).repeat_interleave(Hq // Hkv, dim=0)
    mask = torch.tensor(admit, dtype=torch.bool)[None, None, :].expand(Hq, 1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,D,S,scale", [(4, 2, 8, 5, 1.0), (16, 1, 16, 9, 0.25), (6, 3, 4, 7, 2.0)])
def test_attend_matches_library_sdpa(orc, Hq, Hkv, D, S, scale):
    rng = np.random.default_rng(Hq * 100 + S)
    q = rng.normal(0, 1, (Hq, D)).astype(np.float16)
    k = rng.normal(0, 1, (Hkv, S, D)).astype(np.float16)
    v = rng.normal(0, 1, (Hkv, S, D)).astype(np.float16)
    admit = rng.random(S) < 0.7
    admit[0] = True
    got = orc.attend(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), admit, scale)
    ref = sdpa_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), admit, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_uniform_keys_give_mean_of_admitted_values(orc):
    # V[g][slot] = slot id + 100 g, exact in fp16; keys zero -> equal weights
    Hq, Hkv, D, R, W = 4, 2, 8, 64, 20
    q = np.random.default_rng(1).normal(0, 1, (1, Hq, D)).astype(np.float16)
    k = np.zeros((Hkv, R, D), np.float16)
    v = np.zeros((Hkv, R, D), np.float16)
    for g in range(Hkv):
        v[g] = (np.arange(R)[:, None] + 100 * g).astype(np.float16)
    for P in (0, 5, 19, 20, 63, 64, 100, 127, 130):
        out = orc.flash_ring(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), W, P, 1.0)
        slots = [p % R for p in range(max(0, P - W + 1), P + 1)]
        for h in range(Hq):
            assert np.all(out[0, h] == np.mean(slots) + 100 * (h // (Hq // Hkv)))


def test_single_key_and_scale_zero(orc):
    rng = np.random.default_rng(2)
    Hq, D, cap = 16, 32, 10
    q = rng.normal(0, 1, (2, Hq, D)).astype(np.float16)
    k = rng.normal(0, 1, (cap, D)).astype(np.float16)
    v = rng.normal(0, 1, (cap, D)).astype(np.float16)
    out = orc.flash_full(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), 0, 1.0)
    assert np.array_equal(out[0], np.broadcast_to(v[0].astype(np.float64), (Hq, D)))
    out0 = orc.flash_full(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), 3, 0.0)
    assert np.allclose(out0[0], v[:4].astype(np.float64).mean(0), rtol=0, atol=1e-15)
    assert np.allclose(out0[1], v[:5].astype(np.float64).mean(0), rtol=0, atol=1e-15)


def test_dominant_score_selects_its_value(orc):
    Hq, D, cap = 16, 64, 40
    rng = np.random.default_rng(3)
    q = np.zeros((1, Hq, D), np.float16); q[0, :, 0] = 10.0
    k = rng.normal(0, 0.01, (cap, D)).astype(np.float16)
    k[17, 0] = 10.0          # score gap ~100
    v = rng.normal(0, 1, (cap, D)).astype(np.float16)
    out = orc.flash_full(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), 30, 1.0)
    assert np.allclose(out[0], v[17].astype(np.float64), atol=1e-30 + 1e-40)


def test_capacity_does_not_change_results(orc):
    rng = np.random.default_rng(4)
    Hq, D = 16, 64
    q = rng.normal(0, 1, (3, Hq, D)).astype(np.float16)
    k = rng.normal(0, 1, (50, D)).astype(np.float16)
    v = rng.normal(0, 1, (50, D)).astype(np.float16)
    small = orc.flash_full(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), 40, 1.0)
    kb = np.concatenate([k, rng.normal(0, 1, (200, D)).astype(np.float16)])
    vb = np.concatenate([v, rng.normal(0, 1, (200, D)).astype(np.float16)])
    big = orc.flash_full(q.view(np.uint16), kb.view(np.uint16), vb.view(np.uint16), 40, 1.0)
    assert np.array_equal(small, big)


def test_verify_rows_are_causal(orc):
    rng = np.random.default_rng(5)
    Hq, D = 16, 32
    q = rng.normal(0, 1, (4, Hq, D)).astype(np.float16)
    k = rng.normal(0, 1, (20, D)).astype(np.float16)
    v = rng.normal(0, 1, (20, D)).astype(np.float16)
    blk = orc.flash_full(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), 10, 1.0)
    for i in range(4):
        one = orc.flash_full(q[i:i + 1].view(np.uint16), k.view(np.uint16), v.view(np.uint16), 10 + i, 1.0)
        assert np.array_equal(blk[i], one[0])


def test_ring_poison_never_reaches_output(orc):
    rng = np.random.default_rng(6)
    Hq, Hkv, D, R, W = 16, 8, 32, 64, 32
    P = 200
    q = rng.normal(0, 1, (1, Hq, D)).astype(np.float16)
    k = rng.normal(0, 1, (Hkv, R, D)).astype(np.float16)
    v = rng.normal(0, 1, (Hkv, R, D)).astype(np.float16)
    clean = orc.flash_ring(q.view(np.uint16), k.view(np.uint16), v.view(np.uint16), W, P, 1.0)
    kp, vp = k.copy(), v.copy()
    for i in range(1, 5):
        kp[:, (P + i) % R] = 6e4
        vp[:, (P + i) % R] = -6e4
    dirty = orc.flash_ring(q.view(np.uint16), kp.view(np.uint16), vp.view(np.uint16), W, P, 1.0)
    assert np.array_equal(clean, dirty)
