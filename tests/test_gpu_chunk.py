"""GPU parity of the prefill chunk: q4_gemm (the chunk's MFMA product) against
the oracle's q4 product, and prefill_chunk against the oracle's multi-row
step (gemma-4-E4B-CoreAI card, Provenance and ring/: a 64-row prefill entry
point beside the 1-row decode; Gemma-4-12B-CoreAI card, "v5/ -- ring extent
R = 2W": a block of rows is written before it is attended)."""
import dataclasses

import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import assert_close, assert_close_composed, check_argmax, f16bits
from test_gpu_decode import build_pair, sub_model, sub_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


# ------------------------------------------------------------- q4_gemm ----
def grid_weights(N, K, seed):
    """Weights on the q4 grid with scale 1: every block holds a -8, so
    absmax / 8 = 1 and the codes are the weights."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(N, K))
    for b in range(K // 32):
        q[np.arange(N), b * 32 + rng.integers(0, 32, N)] = -8
    return q


@pytest.mark.parametrize("n", [1, 5, 16, 64])
@pytest.mark.parametrize("N,K", [(16, 128), (100, 96), (130, 512), (33, 3840)])
def test_gemm_integer_probe_bit_exact(N, K, n):
    print(f"gemm integer N={N} K={K} n={n}", flush=True)
    q = grid_weights(N, K, N + K + n)
    packed = q4.q4_pack(torch.from_numpy(q.astype(np.float32)).to(DEV))
    x = np.random.default_rng(n).integers(-2, 3, size=(n, K))
    y = q4.q4_gemm(packed, N, K, torch.from_numpy(x.astype(np.float16)).to(DEV)).cpu().numpy()
    assert np.array_equal(y, (x @ q.T).astype(np.float32))


def test_gemm_one_hot_columns_bit_exact():
    N, K = 200, 1024
    w, _ = synth.gemv_inputs(N, K, 1, seed_w=7)
    packed = q4.q4_pack(w.to(DEV))
    ks = list(range(0, K, 97)) + [K - 1]
    x = torch.zeros(len(ks), K, dtype=torch.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = q4.q4_gemm(packed, N, K, x.to(DEV)).cpu()
    cols = q4.q4_gemv(packed, N, K, x.to(DEV)[:4]).cpu()          # the decode product, one hot
    assert torch.equal(y[:4], cols)
    canon = q4.q4_unpack(packed, N, K).cpu().numpy()
    d = canon[:, :, 0].astype(np.uint16) | (canon[:, :, 1].astype(np.uint16) << 8)
    d = d.view(np.float16).astype(np.float64)
    for i, k in enumerate(ks):
        byte = canon[:, k // 32, 2 + (k % 32) % 16]
        code = ((byte >> 4) if (k % 32) >= 16 else (byte & 15)).astype(np.int64) - 8
        assert np.array_equal(y[i].numpy().astype(np.float64), d[:, k // 32] * code), k


@pytest.mark.parametrize("N,K,n", [(64, 128, 1), (100, 96, 7), (333, 256, 64), (1000, 3840, 64),
                                   (77, 15360, 33), (3840, 4096, 64)])
def test_gemm_random_vs_oracle(orc, N, K, n):
    print(f"gemm random N={N} K={K} n={n}", flush=True)
    w, x = synth.gemv_inputs(N, K, n, seed_w=N + 3, seed_x=K + 5)
    packed = q4.q4_pack(w.to(DEV))
    y = q4.q4_gemm(packed, N, K, x.to(DEV))
    ref = orc.q4_gemv(orc.q4_pack(w.numpy()), N, K, f16bits(x))
    assert_close(y, ref, what=f"q4_gemm N={N} K={K} n={n}")


def test_gemm_12b_shape_sampled_rows(orc):
    N, K, n = 15360, 3840, 64
    w, x = synth.gemv_inputs(N, K, n, seed_w=1, seed_x=2)
    packed = q4.q4_pack(w.to(DEV))
    y = q4.q4_gemm(packed, N, K, x.to(DEV)).cpu()
    rows = np.sort(np.random.default_rng(3).choice(N, 128, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 15, 16, N - 1]]))
    ref = orc.q4_gemv(orc.q4_pack(w[rows].numpy()), len(rows), K, f16bits(x))
    assert_close(y[:, rows], ref, what="12B q4_gemm sampled rows")
    assert torch.equal(y, q4.q4_gemm(packed, N, K, x.to(DEV)).cpu())


# -------------------------------------------------------- prefill chunk ----
@pytest.fixture(scope="module")
def stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s


def check_cache_rows(cfg, gm, om, pos0, n, what):
    """The K/V rows the chunk wrote, against the oracle's.  Rows of later
    layers are computed from the residual stream, a composition with fp16
    rounding points inside (compared under the composed bar); 64 rows give
    many more elements than a decode step, so a rare flip of an fp16 rounding
    upstream does show there."""
    for l, L in enumerate(gm.layers):
        for nm in ("k_cache", "v_cache"):
            if L.get(nm) is None:
                continue
            g = L[nm].float().cpu().numpy()
            r = getattr(om.layers[l], nm).view(np.float16).astype(np.float32)
            if cfg.is_full(l):
                g, r = g[pos0:pos0 + n], r[pos0:pos0 + n]
            else:
                slots = [(pos0 + i) % cfg.ring for i in range(n)]
                g, r = g[:, slots], r[:, slots]
            if l == 0:      # straight from the embedding: the elementwise bar
                assert_close(g, r, atol=2e-3, rtol=2e-3, what=f"{what}: layer {l} {nm} rows")
            else:           # formed from an earlier layer's output: the composed bar
                assert_close_composed(g, r, what=f"{what}: layer {l} {nm} rows")


def check_layers_alone(gm, om, toks, pos0, what):
    """Every layer run alone as a one-layer chunk from the token embedding
    (same weights, caches and positions on both sides): the residual stream of
    every row under the composed-output bar.  (After two random layers the
    stream of some rows already sits several elementwise bars from the oracle
    for the decode path too -- an fp16 rounding flipped by fp32-vs-fp64 sums in
    scale-1 attention moves a score by its whole ulp; so depth is checked layer
    by layer, as for the 12B model.)"""
    for l in range(len(gm.layers)):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        _, _, h = g1.prefill(toks, pos0, want_hidden=True)
        torch.cuda.synchronize()
        ref_h = o1.run_layer(0, o1.embed_tokens(toks), pos0)
        assert_close_composed(h, ref_h, what=f"{what}: layer {l} alone, residual")


@pytest.mark.parametrize("n,pos0", [(64, 0), (64, 128), (17, 200), (1, 77), (64, 192), (40, 9)])
def test_toy_prefill_vs_oracle(orc, stream, n, pos0):
    print(f"toy prefill n={n} pos0={pos0}", flush=True)
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 20, pos0)
    toks = synth.tokens(cfg, n, 20 + n)
    logits, am, h = gm.prefill(toks, pos0, want_hidden=True)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, pos0)
    assert_close(logits, ref[-1], what=f"toy prefill logits n={n} pos0={pos0}")
    check_argmax(logits[None], am, ref[-1:], 4e-3)
    check_cache_rows(cfg, gm, om, pos0, n, f"toy prefill n={n}")
    # fresh caches for the one-layer runs
    gm, om = build_pair(orc, cfg, 20, pos0)
    check_layers_alone(gm, om, toks, pos0, f"toy prefill n={n} pos0={pos0}")


def test_toy_prefill_then_decode(orc, stream):
    """A 64-row chunk from an empty cache, then 6 greedy decode steps that
    attend the rows the chunk wrote, against the oracle's step stream."""
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 21, 0)
    toks = synth.tokens(cfg, 64, 21)
    logits, am, _ = gm.prefill(toks, 0)
    torch.cuda.synchronize()
    ref, ram = om.decode_step(toks, 0)
    assert_close(logits, ref[-1], what="chunk logits")
    tok = int(ram[-1])
    for p in range(64, 70):
        lg, _ = gm.step([tok], p)
        torch.cuda.synchronize()
        rl, rm = om.decode_step([tok], p)
        assert_close(lg, rl, what=f"decode after chunk, position {p}")
        tok = int(rm[0])


def test_toy_prefill_vrow(orc, stream):
    """The chunk over one-row full-layer caches (kv_format 1)."""
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 22, 100, kv="vrow")
    toks = synth.tokens(cfg, 64, 22)
    logits, am, h = gm.prefill(toks, 100, want_hidden=True)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 100)
    assert_close(logits, ref[-1], what="toy vrow prefill logits")
    check_cache_rows(cfg, gm, om, 100, 64, "toy vrow prefill")
    gm, om = build_pair(orc, cfg, 22, 100, kv="vrow")
    check_layers_alone(gm, om, toks, 100, "toy vrow prefill")


def test_prefill_argument_checks(stream):
    cfg = synth.TOY
    gm = q4.build_decode_model(cfg, 23, 10, device=DEV, gen_device="cpu")
    with pytest.raises(q4.Q4Error):            # more than 64 rows
        gm.prefill(list(range(65)), 10)
    with pytest.raises(q4.Q4Error):            # ring too short: R = 128 < W + 65 - 1 for ... n = 64 fits,
        m2 = dataclasses.replace(cfg, ring=96)  # but a 96-slot ring does not hold W + 63 = 127
        gx = q4.DecodeModel(m2, gm.layers, gm.embed, gm.final_norm)
        gx.prefill(list(range(64)), 10)
    with pytest.raises(q4.Q4Error):            # past the full-layer capacity
        gm.prefill(list(range(8)), cfg.full_cap - 4)


@pytest.mark.parametrize("n, pos0", [(64, 2048), (23, 2048), (64, 6000)])
def test_12b_prefill_layers_vs_oracle(orc, stream, n, pos0):
    """A 12B-shape sliding and full layer (layers 0 and 5 of a 6-layer model)
    each run as a one-layer chunk of n rows at positions pos0 .. (the ring
    wraps), against the oracle under the composed-output bar.  From 4096
    positions on, the full layer's 4-row kernel takes 32 splits instead of 16."""
    print(f"12B prefill layers n={n} pos0={pos0}", flush=True)
    cfg = dataclasses.replace(synth.FULL48, n_layers=6, full_cap=8192)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gm, om = build_pair(orc, cfg, 5, pos0, gen_device=DEV)
    torch.cuda.synchronize()
    toks = synth.tokens(cfg, n, 5)
    for l in (0, 5):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        logits, am, h = g1.prefill(toks, pos0, want_hidden=True)
        torch.cuda.synchronize()
        ref_h = o1.run_layer(0, o1.embed_tokens(toks), pos0)
        ref_logits, _ = o1.run_head(ref_h[-1:])
        assert_close_composed(h, ref_h, what=f"12B prefill layer {l}: residual (n={n}, pos0={pos0})")
        assert_close_composed(logits[None], ref_logits, what=f"12B prefill layer {l}: logits (n={n}, pos0={pos0})")
        check_argmax(logits[None], am, ref_logits, 1.6e-2)
        print(f"  layer {l} ok", flush=True)
    del gm
    torch.cuda.empty_cache()


def test_prefill_full_layer_rows4_d256(orc, stream):
    """A model whose full layer has 16 query heads of 256 dims (one KV head):
    the chunk's full-layer attention then takes the 4-rows-per-workgroup
    kernel at D = 256 (the 12B layers use D = 512); 64 and 29 rows."""
    cfg = dataclasses.replace(synth.TOY, n_heads=16, sl_kv_heads=8, full_head_dim=256)
    for n, pos0 in ((64, 100), (29, 3)):
        print(f"rows4 D=256 n={n} pos0={pos0}", flush=True)
        gm, om = build_pair(orc, cfg, 24, pos0)
        toks = synth.tokens(cfg, n, 24)
        logits, am, h = gm.prefill(toks, pos0, want_hidden=True)
        torch.cuda.synchronize()
        ref, _ = om.decode_step(toks, pos0)
        assert_close(logits, ref[-1], what=f"rows4 D=256 logits n={n}")
        check_cache_rows(cfg, gm, om, pos0, n, f"rows4 D=256 n={n}")
        gm, om = build_pair(orc, cfg, 24, pos0)
        check_layers_alone(gm, om, toks, pos0, f"rows4 D=256 n={n}")


def test_one_kv_head_wide_sliding_layers(orc, stream):
    """Sliding layers with one KV head of 256 dims under 16 query heads, and
    full layers of 128 dims (the sliding head wider than the full one, so the
    ring layers size the attention records): the chunk's ring attention takes
    one row per workgroup (16 query heads fill the MFMA columns) and the
    4-row kernel stays on the full layers.  The prefill chunk (64 and 29
    rows) and a width-4 verify block against the oracle."""
    cfg = dataclasses.replace(synth.TOY, n_heads=16, sl_kv_heads=1, sl_head_dim=256, full_head_dim=128)
    for n, pos0 in ((64, 100), (29, 3)):
        print(f"one KV head, wide sliding layers: chunk n={n} pos0={pos0}", flush=True)
        gm, om = build_pair(orc, cfg, 25, pos0)
        toks = synth.tokens(cfg, n, 25)
        logits, am, h = gm.prefill(toks, pos0, want_hidden=True)
        torch.cuda.synchronize()
        ref, _ = om.decode_step(toks, pos0)
        assert_close(logits, ref[-1], what=f"one KV head chunk logits n={n}")
        check_cache_rows(cfg, gm, om, pos0, n, f"one KV head chunk n={n}")
    print("one KV head, wide sliding layers: verify block", flush=True)
    gm, om = build_pair(orc, cfg, 25, 150)
    toks = synth.tokens(cfg, 4, 26)
    logits, am = gm.step(toks, 150)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 150)
    assert_close(logits, ref, what="one KV head verify logits")
    check_argmax(logits, am, ref, 4e-3)
