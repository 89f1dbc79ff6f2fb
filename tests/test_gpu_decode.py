"""GPU parity of decode_step against the oracle: the toy 2-layer step (batch
1 and the width-4 verify block), graph replay, stateful stepping, and the
full 48-layer 12B-shape step at context 32768."""
import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import (assert_close, assert_close_composed, check_argmax, check_layer_stages, composed_stats,
                     oracle_model_from_device)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def build_pair(orc, cfg, seed, ctx, gen_device="cpu", weights="q4", kv="pair"):
    blocks = {}
    opack, unpack = (orc.q4_pack, q4.q4_unpack) if weights == "q4" else (orc.q8_pack, q4.q8_unpack)

    def check(name, l, w, packed):
        ref = opack(w.float().cpu().numpy())
        N, K = w.shape
        got = unpack(packed, N, K).cpu().numpy()
        assert np.array_equal(got, ref), (name, l)
        blocks.setdefault(l, {})[name] = ref

    gm = q4.build_decode_model(cfg, seed, ctx, device=DEV, pack_check=check, gen_device=gen_device,
                               weights=weights, kv=kv)
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


@pytest.mark.parametrize("n", [1, 4])
def test_toy_int8_step_vs_oracle(orc, stream, n):
    """The step over int8 (int8lin) weights: packs bit-exact, logits and the
    K/V rows written against the oracle's int8 step."""
    print(f"toy int8 step n={n}", flush=True)
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 8, 200, weights="q8")
    assert gm.weight_format == 1 and om.weight_format == 1
    toks = synth.tokens(cfg, n, 8)
    logits, am = gm.step(toks, 200)
    torch.cuda.synchronize()
    ref, _ = om.decode_step(toks, 200)
    assert_close(logits, ref, what=f"toy int8 logits n={n}")
    check_argmax(logits, am, ref, 4e-3)
    for l, L in enumerate(gm.layers):
        for nm in ("k_cache", "v_cache"):
            g = L[nm].float().cpu().numpy()
            r = getattr(om.layers[l], nm).view(np.float16).astype(np.float32)
            assert_close(g, r, atol=2e-3, rtol=2e-3, what=f"int8 layer {l} {nm}")


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


def test_speculative_greedy_equals_plain_greedy(stream):
    """Single-pass width-4 verify blocks (decode_step n = 4 at R = 2W) with
    the host acceptance rule emit exactly the tokens of plain batch-1 greedy
    decoding on the same device model; drafts are the greedy stream with an
    error at every position divisible by 5."""
    cfg = synth.TOY
    print("speculative greedy toy", flush=True)
    ga = q4.build_decode_model(cfg, 6, 200, device=DEV, gen_device="cpu")
    gb = q4.build_decode_model(cfg, 6, 200, device=DEV, gen_device="cpu")
    tok0 = int(synth.tokens(cfg, 1, 6)[0])
    n_new = 40
    stream_g, tok = [], tok0
    for p in range(200, 200 + n_new):
        _, am = ga.step([tok], p, want_logits=False)
        tok = int(am.cpu()[0])
        stream_g.append(tok)
    truth = {201 + i: t for i, t in enumerate(stream_g)}

    def drafter(pos, tok, k):
        out = []
        for j in range(1, k + 1):
            t = truth.get(pos + j, 0)
            out.append((t + 1) % cfg.vocab if (pos + j) % 5 == 0 else t)
        return out

    out, blocks = q4.speculative_greedy(gb, tok0, 200, n_new, drafter)
    assert out == stream_g
    assert blocks < n_new


def test_speculative_stream_matches_oracle_greedy(orc, stream):
    """The GPU's speculative stream (width-4 verify blocks accepted by
    q4_spec_accept, drafts = the oracle's greedy stream with an error at every
    position divisible by 5) equals the ORACLE's plain greedy stream, up to the
    first step whose top-2 margin is within twice the parity bar (where two
    correct implementations may pick different tokens)."""
    cfg = synth.TOY
    print("speculative vs oracle greedy toy", flush=True)
    gm, om = build_pair(orc, cfg, 7, 200)          # a seed whose 40 greedy margins are all clear
    tok0 = int(synth.tokens(cfg, 1, 7)[0])
    n_new = 40
    ref, clear, tok = [], None, tok0
    for i, p in enumerate(range(200, 200 + n_new)):
        lg, am = om.decode_step([tok], p)
        top = np.sort(lg[0])[-2:]
        if clear is None and top[1] - top[0] <= 2 * (2e-3 + 1e-3 * abs(top[1])):
            clear = i
        tok = int(am[0])
        ref.append(tok)
    clear = n_new if clear is None else clear
    assert clear >= 20, clear
    truth = {201 + i: t for i, t in enumerate(ref)}

    def drafter(pos, tok, k):
        out = []
        for j in range(1, k + 1):
            t = truth.get(pos + j, 0)
            out.append((t + 1) % cfg.vocab if (pos + j) % 5 == 0 else t)
        return out

    out, blocks = q4.speculative_greedy(gm, tok0, 200, n_new, drafter)
    assert out[:clear] == ref[:clear]
    assert blocks < n_new


@pytest.mark.parametrize("pos0", [126, 254])
def test_toy_verify_block_across_the_ring_end(orc, stream, pos0):
    """A width-4 verify block whose rows sit at ring slots 126, 127, 0, 1
    (first and second wrap): the sliding layer alone, stage by stage against
    the oracle fed the GPU's values, then the 2-layer step's logits and the
    K/V rows it wrote."""
    import dataclasses
    print(f"toy verify across the ring end pos0={pos0}", flush=True)
    cfg = dataclasses.replace(synth.TOY, full_cap=512)
    gm, om = build_pair(orc, cfg, 12, pos0)
    toks = synth.tokens(cfg, 4, 12)
    g0 = sub_model(gm, [0])
    o0 = sub_oracle(om, [0])
    logits, _ = g0.step(toks, pos0, graph=False)
    torch.cuda.synchronize()
    check_layer_stages(orc, g0, o0, 0, o0.embed_tokens(toks), pos0, 4, logits, what=f"ring layer pos0={pos0}")
    gm2, om2 = build_pair(orc, cfg, 12, pos0)
    logits, am = gm2.step(toks, pos0)
    torch.cuda.synchronize()
    ref, _ = om2.decode_step(toks, pos0)
    assert_close(logits, ref, what=f"toy verify across the ring end pos0={pos0}")
    check_argmax(logits, am, ref, 4e-3)
    for l, L in enumerate(gm2.layers):
        for nm in ("k_cache", "v_cache"):
            g = L[nm].float().cpu().numpy()
            r = getattr(om2.layers[l], nm).view(np.float16).astype(np.float32)
            assert_close(g, r, atol=2e-3, rtol=2e-3, what=f"layer {l} {nm}")


@pytest.mark.parametrize("n", [1, 4])
def test_toy_layer_stages_vs_oracle(orc, stream, n):
    """Each layer of the toy model alone, stage by stage (elementwise)."""
    cfg = synth.TOY
    gm, om = build_pair(orc, cfg, 13, 200)
    toks = synth.tokens(cfg, n, 13)
    for l in range(cfg.n_layers):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        logits, _ = g1.step(toks, 200, graph=(l == 0))
        torch.cuda.synchronize()
        check_layer_stages(orc, g1, o1, 0, o1.embed_tokens(toks), 200, n, logits, what=f"toy layer {l} n={n}")


def test_graph_cache_bounded_and_output_independent(orc, stream):
    """Captured step graphs do not depend on the output buffers: 100 steps
    into fresh logits/argmax tensors replay one graph with identical results;
    more than 16 workspaces (so more than 16 graph keys) keep at most 16
    graphs, each step still equal to the eager one."""
    cfg = synth.TOY
    gm, _ = build_pair(orc, cfg, 9, 150)
    q4.release()
    tok = [int(synth.tokens(cfg, 1, 9)[0])]
    first = None
    for i in range(100):
        lg = torch.empty((1, cfg.vocab), dtype=torch.float32, device=DEV)
        am = torch.empty(1, dtype=torch.int32, device=DEV)
        gm.step(tok, 150, logits=lg, argmax=am)          # rewrites the same row: same result
        if first is None:
            torch.cuda.synchronize()
            first = (lg.clone(), am.clone())
        elif i % 10 == 0:
            torch.cuda.synchronize()
            assert torch.equal(lg, first[0]) and torch.equal(am, first[1]), i
    torch.cuda.synchronize()
    assert q4.graph_count() == 1
    eager, _ = gm.step(tok, 150, graph=False)
    torch.cuda.synchronize()
    assert torch.equal(eager, first[0])
    keep = []                                            # live models: distinct workspaces
    for j in range(20):
        gj = sub_model(gm, list(range(cfg.n_layers)))    # a new workspace: a new key
        keep.append(gj)
        lj, aj = gj.step(tok, 150)
        torch.cuda.synchronize()
        assert torch.equal(lj, first[0]) and torch.equal(aj, first[1]), j
        assert q4.graph_count() <= 16
    assert q4.graph_count() == 16
    q4.release()
    assert q4.graph_count() == 0


def test_stream_read_xor(stream):
    print("stream read", flush=True)
    g = torch.Generator(device="cpu").manual_seed(11)
    for nbytes in (16, 1 << 20, (5 << 20) + 48):
        src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
        sink = q4.stream_read(src.to(DEV))
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
        assert got == want, nbytes


def sub_model(gm, layer_ids, cfg=None, scalars=None):
    """A device model over a subset of gm's layers (shared tensors)."""
    import dataclasses
    cfg = dataclasses.replace(cfg or gm.cfg, n_layers=len(layer_ids))
    layers = []
    for i, l in enumerate(layer_ids):
        L = dict(gm.layers[l])
        if scalars is not None:
            L["layer_scalar"] = scalars[i]
        layers.append(L)
    return q4.DecodeModel(cfg, layers, gm.embed, gm.final_norm, gm.weight_format, gm.kv_format)


def sub_oracle(om, layer_ids, scalars=None):
    import copy
    m = copy.copy(om)
    m.layers = []
    for i, l in enumerate(layer_ids):
        L = copy.copy(om.layers[l])
        L.k_cache = None if L.k_cache is None else L.k_cache.copy()
        L.v_cache = L.v_cache.copy()
        if scalars is not None:
            L.layer_scalar = scalars[i]
        m.layers.append(L)
    return m


@pytest.fixture(scope="module")
def full48(orc):
    """The 48-layer 12B-shape model at context 32768 (the benchmark's
    workload), on the GPU and in the oracle, from the same synthetic inputs."""
    print("building the 48-layer model", flush=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gm, om = build_pair(orc, synth.FULL48, 5, 32768 - 4, gen_device=DEV)
        gm.pristine = [(L["k_cache"].clone(), L["v_cache"].clone()) for L in gm.layers]
    torch.cuda.synchronize()
    yield gm, om
    del gm
    torch.cuda.empty_cache()


def restore_caches(gm):
    """Put back the caches the oracle holds: every step writes its K/V rows
    into the shared device caches, which a later test must not attend to."""
    for L, (k, v) in zip(gm.layers, gm.pristine):
        L["k_cache"].copy_(k)
        L["v_cache"].copy_(v)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n", [1, 4])
def test_48_layer_step_properties(full48, stream, n):
    """Properties of the full step that hold at any size: graph replay equals
    eager launches bit for bit, repeated steps are identical, logits are
    bounded by the softcap and the greedy id is their first maximum."""
    gm, _ = full48
    restore_caches(gm)
    cfg = gm.cfg
    pos = 32768 - n
    toks = synth.tokens(cfg, n, 5)
    la, aa = gm.step(toks, pos, graph=True)
    la = la.clone(); aa = aa.clone()
    lb, ab = gm.step(toks, pos, graph=True)
    lc, ac = gm.step(toks, pos, graph=False)
    torch.cuda.synchronize()
    assert torch.equal(la, lb) and torch.equal(la, lc) and torch.equal(aa, ab) and torch.equal(aa, ac)
    assert torch.isfinite(la).all() and (la.abs() < cfg.softcap).all()
    assert torch.equal(aa.long(), la.argmax(dim=1))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("n", [1, 4])
def test_48_layer_each_layer_vs_oracle(orc, full48, stream, n):
    """Every layer of the 48-layer model at full size and in the benchmark's
    launch configuration, run as a one-layer step from the token embedding.
    Stage by stage (elementwise bar): the oracle's stage fed the GPU's own
    values at that stage's input (attention input, q/k/v projections, finished
    queries, K/V rows written, attention over the GPU's caches, o-proj
    residual, MLP input, GELU * up, down residual, head input, logits).  End
    of layer: logits and residual stream against the oracle's whole layer
    from the embedding, under the composed-output bar (fp16 rounding points
    inside a layer flip where the two sides' fp32/fp64 sums straddle them)."""
    gm, om = full48
    restore_caches(gm)
    cfg = gm.cfg
    pos = 32768 - n
    toks = synth.tokens(cfg, n, 5)
    layers = range(cfg.n_layers) if n == 1 else [0, 4, 5, 6, 11, 23, 41, 47]
    for l in layers:
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        o2 = sub_oracle(om, [l])
        logits, am = g1.step(toks, pos, graph=False)
        h = g1.hidden(n)
        torch.cuda.synchronize()
        h0 = o1.embed_tokens(toks)
        check_layer_stages(orc, g1, o1, 0, h0, pos, n, logits, what=f"layer {l} (n={n})")
        ref_h = o2.run_layer(0, h0, pos)
        ref_logits, _ = o2.run_head(ref_h)
        assert_close_composed(logits, ref_logits, what=f"layer {l} alone: logits (n={n})")
        assert_close_composed(h, ref_h, what=f"layer {l} alone: residual (n={n})")
        check_argmax(logits, am, ref_logits, 1.6e-2)
        if l % 8 == 0:
            print(f"  layer {l} ok", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n", [1, 4])
def test_12b_two_layer_composition(orc, full48, stream, n):
    """Layers 4 -> 5 (sliding into full) of the 12B model as a 2-layer step.
    Elementwise: layer 4's stages from the embedding, and layer 5's stages
    fed the GPU's residual after layer 4 (from a 1-layer step of layer 4,
    which computes it bit for bit as the 2-layer step does).  Composed, one
    layer deep: the step's logits and residual against the oracle's layer 5
    run on the GPU's layer-4 output, and layer 4's residual against the
    oracle's layer 4 from the embedding (the one-layer composed bar).
    Composed, two layers deep from the embedding: RMS within two one-layer
    bars.  Layer 5's full attention (scale-1 scores over 32768 positions)
    magnifies the few fp16 flips of layer 4 (13-19 of 4096 attention outputs,
    one ulp each, for either ring kernel), so two equally accurate kernels
    give 2-deep logits RMS 1.3e-3 and 1.9e-3 against a one-layer bar of
    1.75e-3, and 0.86-0.97 of the elements within the elementwise bar
    (printed, not asserted)."""
    gm, om = full48
    restore_caches(gm)
    cfg = gm.cfg
    pos = 32768 - n
    toks = synth.tokens(cfg, n, 5)
    g4 = sub_model(gm, [4])
    o4 = sub_oracle(om, [4])
    l4, _ = g4.step(toks, pos, graph=False)
    torch.cuda.synchronize()
    check_layer_stages(orc, g4, o4, 0, o4.embed_tokens(toks), pos, n, l4, what=f"layers 4->5, layer 4 (n={n})")
    h4 = g4.hidden(n).double().cpu().numpy()
    r4 = sub_oracle(om, [4])
    assert_close_composed(h4, r4.run_layer(0, r4.embed_tokens(toks), pos),
                          what=f"layer 4 from the embedding: residual (n={n})")
    restore_caches(gm)
    g45 = sub_model(gm, [4, 5])
    logits, am = g45.step(toks, pos)
    h = g45.hidden(n)
    torch.cuda.synchronize()
    o45 = sub_oracle(om, [4, 5])
    check_layer_stages(orc, g45, o45, 1, h4, pos, n, logits, what=f"layers 4->5, layer 5 (n={n})")
    one = sub_oracle(om, [4, 5])
    h5 = one.run_layer(1, h4, pos)
    l5, _ = one.run_head(h5)
    assert_close_composed(logits, l5, what=f"layer 5 on the GPU's layer-4 output: logits (n={n})")
    assert_close_composed(h, h5, what=f"layer 5 on the GPU's layer-4 output: residual (n={n})")
    ref = sub_oracle(om, [4, 5])
    rh = ref.run_layer(1, ref.run_layer(0, ref.embed_tokens(toks), pos), pos)
    rl, _ = ref.run_head(rh)
    for g, r, nm in ((logits, rl, "logits"), (h, rh, "residual")):
        inside, worst, rms, rms_bar = composed_stats(g, r, what=f"layers 4->5 from the embedding: {nm}")
        print(f"  layers 4->5 from the embedding, {nm}: {inside:.4f} within the elementwise bar, "
              f"worst {worst:.2f} times it, rms {rms:.3e} (one-layer bar {rms_bar:.3e})", flush=True)
        assert rms <= 2 * rms_bar, (nm, n, rms, rms_bar)
    check_argmax(logits, am, rl, 1.6e-2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("pos", [2046, 1022, 0])
def test_12b_verify_block_across_the_ring_end(orc, full48, stream, pos):
    """A width-4 verify block through 12B sliding layers and a full layer,
    stage by stage: at positions 2046 .. 2049 (ring slots 2046, 2047, 0, 1);
    at 1022 .. 1025 (the first two rows see every earlier position, the last
    two windows start at 1 and 2: the splits divide a union of unequal
    windows); at 0 .. 3 (most splits empty)."""
    gm, om = full48
    restore_caches(gm)
    cfg = gm.cfg
    n = 4
    print(f"12b verify block at {pos}", flush=True)
    toks = synth.tokens(cfg, n, 7)
    for l in (0, 4, 5):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        logits, _ = g1.step(toks, pos)
        torch.cuda.synchronize()
        check_layer_stages(orc, g1, o1, 0, o1.embed_tokens(toks), pos, n, logits, what=f"layer {l} at {pos}")
    restore_caches(gm)


@pytest.mark.parametrize("n", [1, 4])
def test_12b_int8_layers_vs_oracle(orc, stream, n):
    """The int8 step at the 12B shapes and context 32768, in the benchmark's
    launch configuration: a sliding and a full layer (layers 0 and 5 of a
    6-layer model), each run as a one-layer step from the token embedding,
    against the oracle's int8 step under the composed-output bar."""
    import dataclasses
    print(f"12B int8 layers n={n}", flush=True)
    cfg = dataclasses.replace(synth.FULL48, n_layers=6, full_cap=32768 + 8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gm, om = build_pair(orc, cfg, 5, 32768 - 4, gen_device=DEV, weights="q8")
    torch.cuda.synchronize()
    pos = 32768 - n
    toks = synth.tokens(cfg, n, 5)
    for l in (0, 5):
        g1 = sub_model(gm, [l])
        o1 = sub_oracle(om, [l])
        logits, am = g1.step(toks, pos, graph=False)
        h = g1.hidden(n)
        torch.cuda.synchronize()
        ref_h = o1.run_layer(0, o1.embed_tokens(toks), pos)
        ref_logits, _ = o1.run_head(ref_h)
        assert_close_composed(logits, ref_logits, what=f"int8 layer {l} alone: logits (n={n})")
        assert_close_composed(h, ref_h, what=f"int8 layer {l} alone: residual (n={n})")
        check_argmax(logits, am, ref_logits, 1.6e-2)
    del gm
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_48_layer_identity_and_zero_scalar(orc, full48, stream):
    """All 48 layers at full size: with zero output and down projections every
    layer leaves the residual alone, so the logits are the oracle's head of
    the embedding; with a zero scalar on the last layer they are exactly 0."""
    gm, om = full48
    restore_caches(gm)
    cfg = gm.cfg
    n, pos = 1, 32767
    toks = synth.tokens(cfg, n, 5)
    zo = q4.q4_pack(torch.zeros(cfg.hidden, cfg.n_heads * cfg.sl_head_dim, device=DEV))
    zof = q4.q4_pack(torch.zeros(cfg.hidden, cfg.n_heads * cfg.full_head_dim, device=DEV))
    zd = q4.q4_pack(torch.zeros(cfg.hidden, cfg.inter, device=DEV))
    import dataclasses
    layers = []
    for l in range(cfg.n_layers):
        L = dict(gm.layers[l])
        L["wo"] = zof if cfg.is_full(l) else zo
        L["wd"] = zd
        layers.append(L)
    gid = q4.DecodeModel(cfg, layers, gm.embed, gm.final_norm)
    logits, am = gid.step(toks, pos, graph=True)
    torch.cuda.synchronize()
    h0 = om.embed_tokens(toks)
    ref_logits, _ = om.run_head(h0)
    assert_close(logits, ref_logits, what="identity layers: logits")
    check_argmax(logits, am, ref_logits, 4e-3)
    scal = [1.0] * (cfg.n_layers - 1) + [0.0]
    gz = sub_model(gm, list(range(cfg.n_layers)), scalars=scal)
    lz, az = gz.step(toks, pos, graph=True)
    torch.cuda.synchronize()
    assert torch.all(lz == 0.0) and int(az[0]) == 0


@pytest.mark.timeout(600)
def test_48_layer_capacity_independence(full48, stream):
    """The full layers' padded capacity is never read: a copy of the model
    whose full-layer caches are twice as long (NaN past the old capacity)
    gives the same bits."""
    import dataclasses
    gm, _ = full48
    restore_caches(gm)
    cfg = gm.cfg
    n, pos = 1, 32767
    toks = synth.tokens(cfg, n, 5)
    base, _ = gm.step(toks, pos, graph=False)
    base = base.clone()
    big = dataclasses.replace(cfg, full_cap=2 * cfg.full_cap)
    layers = []
    for l in range(cfg.n_layers):
        L = dict(gm.layers[l])
        if cfg.is_full(l):
            for nm in ("k_cache", "v_cache"):
                t = torch.full((big.full_cap, cfg.full_head_dim), float("nan"), dtype=torch.float16, device=DEV)
                t[: cfg.full_cap] = L[nm]
                L[nm] = t
        layers.append(L)
    gb = q4.DecodeModel(big, layers, gm.embed, gm.final_norm)
    lb, _ = gb.step(toks, pos, graph=False)
    torch.cuda.synchronize()
    assert torch.equal(base, lb)
