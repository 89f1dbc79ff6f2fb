"""GPU parity of decode_step against the oracle: the toy 2-layer step (batch
1 and the width-4 verify block), graph replay, stateful stepping, and the
full 48-layer 12B-shape step at context 32768."""
import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import assert_close, check_argmax, oracle_model_from_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def build_pair(orc, cfg, seed, ctx, gen_device="cpu"):
    blocks = {}

    def check(name, l, w, packed):
        ref = orc.q4_pack(w.float().cpu().numpy())
        N, K = w.shape
        got = q4.q4_unpack(packed, N, K).cpu().numpy()
        assert np.array_equal(got, ref), (name, l)
        blocks.setdefault(l, {})[name] = ref

    gm = q4.build_decode_model(cfg, seed, ctx, device=DEV, pack_check=check, gen_device=gen_device)
    om = oracle_model_from_device(orc, cfg, gm, blocks)
    return gm, om


@pytest.fixture(scope="module")
def stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yield s


@pytest.mark.parametrize("n", [1, 4])
@pytest.mark.parametrize("graph", [False, True])
def test_toy_step_vs_oracle(orc, stream, n, graph):
    print(f"toy step n={n} graph={graph}", flush=True)
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 0, 200)
    toks = synth.tokens(cfg, n, 0)
    logits, am = gm.step(toks, 200, graph=graph)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 200)
    assert_close(logits, ref, what=f"toy logits n={n}")
    check_argmax(logits, am, ref, 4e-3)
    # the caches the step wrote match the oracle's (fp16 rows)
    for l, L in enumerate(gm.layers):
        for nm in ("k_cache", "v_cache"):
            g = L[nm].float().cpu().numpy()
            r = getattr(om.layers[l], nm).view(np.float16).astype(np.float32)
            assert_close(g, r, atol=2e-3, rtol=2e-3, what=f"layer {l} {nm}")


def test_toy_graph_replay_matches_eager(orc, stream):
    cfg = synth.TOY
    gm1, _ = build_pair(orc, cfg, 1, 150)
    gm2, _ = build_pair(orc, cfg, 1, 150)
    toks = synth.tokens(cfg, 6, 1)
    for i in range(6):     # several replays of one captured graph, eager work between them
        la, aa = gm1.step(toks[i:i + 1], 150 + i, graph=True)
        lb, ab = gm2.step(toks[i:i + 1], 150 + i, graph=False)
        torch.cuda.synchronize()
        assert torch.equal(la, lb) and torch.equal(aa, ab), i


def test_toy_stateful_steps_vs_oracle(orc, stream):
    """Greedy decoding for 8 steps from an empty cache; the ring wraps nothing
    yet but the full cache grows; every step compared with the oracle."""
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 2, 0)
    tok = int(synth.tokens(cfg, 1, 2)[0])
    for p in range(8):
        logits, am = gm.step([tok], p)
        torch.cuda.synchronize()
        ref, ram = om.decode_step([tok], p)
        assert_close(logits, ref, what=f"step {p}")
        tok = int(ram[0])          # follow the oracle's token stream


def test_toy_ring_wrap_and_verify(orc, stream):
    """Positions past the ring size (128) with a 4-row verify block."""
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 3, 250)
    toks = synth.tokens(cfg, 4, 3)
    logits, am = gm.step(toks, 250)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 250)
    assert_close(logits, ref, what="toy wrap verify")


def test_verify_block_rows_equal_sequential_rows(orc, stream):
    cfg = synth.TOY
    gb, _ = build_pair(orc, cfg, 4, 180)
    gs, _ = build_pair(orc, cfg, 4, 180)
    toks = synth.tokens(cfg, 4, 4)
    lb, _ = gb.step(toks, 180)
    rows = [gs.step(toks[i:i + 1], 180 + i)[0].clone() for i in range(4)]
    torch.cuda.synchronize()
    for i in range(4):
        assert_close(lb[i], rows[i][0].cpu().double().numpy(), atol=1e-3, rtol=1e-3, what=f"row {i}")


@pytest.mark.parametrize("n", [1, 4])
def test_48_layers_ctx32k_vs_oracle(orc, stream, n):
    """The 48-layer 12B-shape step at context 32768 (the benchmark's workload
    and launch configuration), every logit against the oracle."""
    print(f"48-layer step n={n}", flush=True)
    cfg = synth.FULL48
    pos = 32768 - n
    gm, om = build_pair(orc, cfg, 5, pos, gen_device=DEV)
    toks = synth.tokens(cfg, n, 5)
    logits, am = gm.step(toks, pos)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, pos)
    assert_close(logits, ref, what=f"48-layer logits n={n}")
    check_argmax(logits, am, ref, 4e-3)
    del gm
    torch.cuda.empty_cache()
