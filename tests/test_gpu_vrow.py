"""GPU parity of the full layers that cache one row per position ("vrow"):
flash_decode_full_vrow against the oracle at small ragged sizes and at the
32K / 131K workloads, its reduction to the K/V-pair kernel, and the decode
step with kv_format 1 (toy model and a 12B-shape full layer).

Gemma-4-12B-CoreAI card, "The per-tier cost" (the full-layer pair is the KV
term that grows with the context); gemma4-12b card, architecture notes (V is
the scale-free norm of the raw k projection, K its k_norm-weighted norm,
rotated, so K = RoPE(kw * V))."""
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


def kw_for(D, seed):
    return synth.normal((D,), 0.1, synth.gen(seed), mean=1.0)


@pytest.mark.parametrize("D,rot,theta", [(128, 16, 1e6), (128, 64, 1e4), (512, 64, 1e6), (512, 7, 1e4)])
@pytest.mark.parametrize("ctx,n_rows", [(1, 1), (31, 1), (200, 2), (333, 4), (4100, 1)])
def test_vrow_small_vs_oracle(orc, D, rot, theta, ctx, n_rows):
    print(f"vrow D={D} rot={rot} ctx={ctx} rows={n_rows}", flush=True)
    cap = ctx + 40
    q, _, v = synth.full_attn_inputs(ctx, cap, n_rows, Hq=16, D=D, seed=ctx + D + rot)
    kw = kw_for(D, ctx + rot)
    pos0 = ctx - n_rows
    out = q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), theta, rot, pos0, 1.0)
    ref = orc.flash_full_vrow(f16bits(q), f16bits(v), kw.numpy(), theta, rot, pos0, 1.0)
    assert_close(out[0], ref, what=f"vrow D={D} rot={rot} ctx={ctx}")


def test_vrow_scale_and_heads(orc):
    q, _, v = synth.full_attn_inputs(700, 800, 1, Hq=8, D=128, seed=15)
    kw = kw_for(128, 15)
    out = q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 32, 699, 0.0625)
    ref = orc.flash_full_vrow(f16bits(q), f16bits(v), kw.numpy(), 1e6, 32, 699, 0.0625)
    assert_close(out[0], ref, what="vrow scale 1/16, 8 heads")


def test_vrow_without_rotation_equals_pair_kernel():
    """rot_pairs = 0 and weights 1, 2, 4: kw * v is an fp16 value, so the
    pair kernel over K = kw * v runs the same products in the same order
    (the lo parts are zero) and gives the same bits."""
    for D in (128, 512):
        q, _, v = synth.full_attn_inputs(3000, 3010, 2, Hq=16, D=D, seed=21 + D)
        e = torch.randint(0, 3, (D,), generator=synth.gen(22))   # upscaling only: no subnormal
        kw = torch.pow(2.0, e.float())
        k = (v.float() * kw).half()
        assert torch.equal(k.float(), v.float() * kw)
        a = q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 0, 2998, 1.0)
        b = q4.flash_decode_full(q.to(DEV), k.to(DEV), v.to(DEV), 2998, 1.0)
        torch.cuda.synchronize()
        assert torch.equal(a, b), D


def test_vrow_capacity_independence():
    q, _, v = synth.full_attn_inputs(3000, 3000, 1, seed=26)
    kw = kw_for(512, 26)
    big = torch.cat([v, torch.full((5000, 512), float("nan"), dtype=torch.float16)])
    a = q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 64, 2999, 1.0)
    b = q4.flash_decode_full_vrow(q.to(DEV), big.to(DEV), kw.to(DEV), 1e6, 64, 2999, 1.0)
    assert torch.equal(a, b)


@pytest.mark.parametrize("ctx", [32768, 131072])
def test_vrow_config_sizes_vs_oracle(orc, ctx):
    """The full-attention workload at 32K and 131K context, every output."""
    print(f"vrow config ctx={ctx}", flush=True)
    q, _, v = synth.full_attn_inputs(ctx, ctx + 4, 1, seed=3)
    kw = kw_for(512, 3)
    out = q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 64, ctx - 1, 1.0)
    ref = orc.flash_full_vrow(f16bits(q), f16bits(v), kw.numpy(), 1e6, 64, ctx - 1, 1.0)
    assert_close(out[0], ref, what=f"vrow ctx={ctx}")


def test_vrow_multi_sequence(orc):
    n_seq, cap, D = 3, 600, 128
    qs, vs = [], []
    for s in range(n_seq):
        q, _, v = synth.full_attn_inputs(500 + 30 * s, cap, 2, Hq=16, D=D, seed=40 + s)
        qs.append(q); vs.append(v)
    kw = kw_for(D, 40)
    pos = [498, 528, 558]
    out = q4.flash_decode_full_vrow(torch.stack(qs).to(DEV), torch.stack(vs).to(DEV), kw.to(DEV), 1e4, 64,
                                    pos, 1.0)
    for s in range(n_seq):
        ref = orc.flash_full_vrow(f16bits(qs[s]), f16bits(vs[s]), kw.numpy(), 1e4, 64, pos[s], 1.0)
        assert_close(out[s], ref, what=f"vrow seq {s}")


def test_vrow_argument_checks():
    q, _, v = synth.full_attn_inputs(100, 120, 1, Hq=16, D=256, seed=2)
    kw = torch.ones(256)
    with pytest.raises(q4.Q4Error):      # D = 256 is not a one-row layout
        q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 16, 99, 1.0)
    q, _, v = synth.full_attn_inputs(100, 120, 1, Hq=16, D=512, seed=2)
    kw = torch.ones(512)
    with pytest.raises(q4.Q4Error):      # more rotated pairs than the kernel forms
        q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 65, 99, 1.0)
    with pytest.raises(q4.Q4Error):      # position past the capacity
        q4.flash_decode_full_vrow(q.to(DEV), v.to(DEV), kw.to(DEV), 1e6, 64, 120, 1.0)


# ------------------------------------------------------------ decode step ----
def build_vrow_pair(orc, cfg, seed, ctx, gen_device="cpu"):
    gm, om = build_pair(orc, cfg, seed, ctx, gen_device=gen_device, kv="vrow")
    assert gm.kv_format == 1 and om.kv_format == 1
    return gm, om


@pytest.fixture(scope="module")
def stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s


@pytest.mark.parametrize("n", [1, 4])
@pytest.mark.parametrize("graph", [False, True])
def test_toy_vrow_step_vs_oracle(orc, stream, n, graph):
    print(f"toy vrow step n={n} graph={graph}", flush=True)
    cfg = synth.TOY
    gm, om = build_vrow_pair(orc, cfg, 9, 200)
    toks = synth.tokens(cfg, n, 9)
    logits, am = gm.step(toks, 200, graph=graph)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 200)
    assert_close(logits, ref, what=f"toy vrow logits n={n}")
    check_argmax(logits, am, ref, 4e-3)
    for l, L in enumerate(gm.layers):
        names = ("v_cache",) if cfg.is_full(l) else ("k_cache", "v_cache")
        for nm in names:
            g = L[nm].float().cpu().numpy()
            r = getattr(om.layers[l], nm).view(np.float16).astype(np.float32)
            assert_close(g, r, atol=2e-3, rtol=2e-3, what=f"vrow layer {l} {nm}")


def test_toy_vrow_stateful_steps_vs_oracle(orc, stream):
    """Greedy steps from an empty cache: every full-layer key of the context
    is formed from rows this step sequence wrote."""
    cfg = synth.TOY
    gm, om = build_vrow_pair(orc, cfg, 10, 0)
    tok = int(synth.tokens(cfg, 1, 10)[0])
    for p in range(8):
        logits, am = gm.step([tok], p)
        torch.cuda.synchronize()
        ref, ram = om.decode_step([tok], p)
        assert_close(logits, ref, what=f"vrow step {p}")
        tok = int(ram[0])


@pytest.mark.parametrize("n", [1, 4])
def test_12b_vrow_full_layer_vs_oracle(orc, stream, n):
    """A 12B-shape full layer (layer 5 of a 6-layer model, context 32768) in
    the one-row layout, run as a one-layer step from the token embedding,
    against the oracle under the composed-output bar; the V rows it wrote
    under the elementwise bar."""
    print(f"12B vrow full layer n={n}", flush=True)
    cfg = dataclasses.replace(synth.FULL48, n_layers=6, full_cap=32768 + 8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gm, om = build_vrow_pair(orc, cfg, 5, 32768 - 4, gen_device=DEV)
    torch.cuda.synchronize()
    pos = 32768 - n
    toks = synth.tokens(cfg, n, 5)
    for l in (5, 0):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        logits, am = g1.step(toks, pos, graph=False)
        h = g1.hidden(n)
        torch.cuda.synchronize()
        ref_h = o1.run_layer(0, o1.embed_tokens(toks), pos)
        ref_logits, _ = o1.run_head(ref_h)
        assert_close_composed(logits, ref_logits, what=f"vrow layer {l} alone: logits (n={n})")
        assert_close_composed(h, ref_h, what=f"vrow layer {l} alone: residual (n={n})")
        check_argmax(logits, am, ref_logits, 1.6e-2)
        if l == 5:
            g = gm.layers[l]["v_cache"].float().cpu().numpy()[pos:pos + n]
            r = o1.layers[0].v_cache.view(np.float16).astype(np.float32)[pos:pos + n]
            assert_close(g, r, atol=2e-3, rtol=2e-3, what="vrow layer 5 rows")
    del gm
    torch.cuda.empty_cache()
