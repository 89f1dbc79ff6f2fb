#!/usr/bin/env python3
"""Benchmark: batch-1 48-layer decode step (12B shapes, int4 q4_0 weights,
fp16 KV) at context 32768 on one MI355X.

Prints ONE JSON line.  `value` = decode tokens/s (one token per step, inputs
resident in HBM).  Extra fields: whole-step achieved HBM bandwidth from the
algorithmic byte model, the dominant kernel's roofline (k_q4_gemv<1,0,4,0>,
the step's q/k/v, output and down products in the step's own launch
configuration, timed live with HIP events on its stream), the q4 GEMV alone
at three shapes, context-131072 and width-4 verify figures, the attention
kernels alone, and the CPU oracle timed on the host cores on a bounded
sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode full|gemv|step|verify|traffic|prefill|attn_traffic|gemv_lds]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="full", choices=["full", "gemv", "step", "verify", "traffic", "prefill", "attn_traffic", "gemv_lds"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_gemv_bytes(cfg):
    """Algorithmic bytes of the step's q/k/v, output and down products (the
    launches decode_step_gemvs makes: three per layer)."""
    from int4_q4_gemv_amd import bytemodel
    return sum(bytemodel.q4_matrix_bytes(N, K) for l in range(cfg.n_layers)
               for nm, N, K in cfg.layer_shapes(l) if nm in ("wq", "wk", "wv", "wo", "wd"))


def time_step_gemvs(q4, torch, model, reps=10, warm=5):
    """The step's most launched kernel, k_q4_gemv<1,0,4,0>, in the step's own
    launch configuration: decode_step_gemvs enqueues the q/k/v, output and
    down products of all 48 layers (144 launches, 2.95 GB: every launch
    streams from HBM), captured once into a graph and replayed back to back
    between two HIP events on the launch stream after `warm` untimed replays.
    Returns (average seconds per launch, launches timed, average algorithmic
    bytes per launch)."""
    cfg = model.cfg
    model.step([1], 32767, want_logits=False)          # the workspace holds a step's activations
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.current_stream()):
        model.step_gemvs(1)
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    e1.synchronize()
    per_step = 3 * cfg.n_layers
    launches = reps * per_step
    return e0.elapsed_time(e1) * 1e-3 / launches, launches, step_gemv_bytes(cfg) / per_step


def time_gemv_shapes(q4, torch, model):
    """q4_gemv on its own: 3840 -> 15360 (gate/up shape) at batch 1 and 4,
    15360 -> 3840 (down shape) at batch 1, each over the 48 layers' matrices
    of that shape (no launch finds its weights in the last-level cache)."""
    cfg = model.cfg
    res = {}
    for name, nm, B in (("gate_3840x15360_b1", ("wg", "wu"), 1), ("gate_3840x15360_b4", ("wg", "wu"), 4),
                        ("down_15360x3840_b1", ("wd",), 1)):
        N, K = (cfg.inter, cfg.hidden) if nm[0] != "wd" else (cfg.hidden, cfg.inter)
        mats = [L[k] for L in model.layers for k in nm]
        x = torch.randn(B, K, device="cuda", generator=torch.Generator("cuda").manual_seed(7)).half()
        y = torch.empty(B, N, device="cuda")
        g = q4.Gemv(N, K, B)
        t = time_graph_calls(torch, lambda i: g(mats[i % len(mats)], x, y), len(mats), replays=10)
        nb = q4.packed_bytes(N, K)
        res[name] = {"us": round(t * 1e6, 3), "bytes": nb, "GBps": round(nb / t / 1e9, 1),
                     "frac": round(nb / t / 1e9 / PEAK_GBPS, 4)}
    return res


def time_stream_read(q4, torch, nbytes=4 << 30, reps=5):
    """Achievable read bandwidth on this GPU: the library's plain streaming
    read (16-byte loads, 8 in flight per thread) over a 4 GiB buffer, two
    untimed calls, then `reps` calls between two HIP events."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = None
    for _ in range(2):
        sink = q4.stream_read(src, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        q4.stream_read(src, sink)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src
    return nbytes / t / 1e9


def time_graph_calls(torch, fn, reps, replays=5):
    """Average device time of fn(i), captured reps times into one graph and
    replayed between two HIP events on the current stream."""
    fn(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.current_stream()):
        for i in range(reps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * replays)


def time_attention(q4, torch):
    """The two attention kernels on their own, on the synthetic inputs of the
    scope table: full attention (16 q heads over one KV head, D 512, scale 1)
    at contexts 32768 and 131072 in a 131076-row buffer, rotating 6 buffers
    so that no call finds its keys in the last-level cache; the ring (8 KV
    heads, D 256, W 1024, R 2048, position 100000) as one call and as 40
    independent rings in one call.  Bytes per call: 2048 per full position,
    1024 per admitted ring position and KV head."""
    from int4_q4_gemv_amd import synth
    res = {}
    cap = 131076
    bufs = [synth.full_attn_inputs(131072, cap, seed=3 + i, device="cuda") for i in range(6)]
    ws = q4._fd_ws(1, 1, 16, 512, "cuda")
    for ctx in (32768, 131072):
        t = time_graph_calls(torch, lambda i: q4.flash_decode_full(*bufs[i % 6], ctx - 1, 1.0, ws=ws), 24)
        nb = ctx * 2048
        res[f"full_attention_ctx{ctx}"] = {"us": round(t * 1e6, 2), "bytes": nb,
                                          "GBps": round(nb / t / 1e9, 1), "frac": round(nb / t / 1e9 / PEAK_GBPS, 4)}
    # the one-row layout over the same V rows: 1024 bytes per position
    kw = synth.normal((512,), 0.1, synth.gen(3), mean=1.0).to("cuda")
    for ctx in (32768, 131072):
        t = time_graph_calls(torch, lambda i: q4.flash_decode_full_vrow(bufs[i % 6][0], bufs[i % 6][2], kw, 1e6,
                                                                        64, ctx - 1, 1.0, ws=ws), 24)
        nb = ctx * 1024
        res[f"full_attention_vrow_ctx{ctx}"] = {"us": round(t * 1e6, 2), "bytes": nb,
                                               "GBps": round(nb / t / 1e9, 1),
                                               "frac": round(nb / t / 1e9 / PEAK_GBPS, 4)}
    del bufs
    q, k, v = (t.to("cuda") for t in synth.ring_inputs(100000, n_rows=1, n_rejected=4))
    ws = q4._fd_ws(1, 1, 16, 256, "cuda")
    t = time_graph_calls(torch, lambda i: q4.flash_decode_ring(q, k, v, 1024, 100000, 1.0, ws=ws), 40)
    res["ring_attention_1seq_us"] = round(t * 1e6, 2)
    # two sets of 40 rings (2 x 671 MB of K/V, above the last-level cache), alternated
    sets = []
    for k in range(2):
        rings = [synth.ring_inputs(100000, n_rows=1, n_rejected=4, seed=100 + 40 * k + s, device="cuda")
                 for s in range(40)]
        sets.append(tuple(torch.stack([r[j] for r in rings]).to("cuda") for j in range(3)))
        del rings
    ws = q4._fd_ws(40, 1, 16, 256, "cuda")
    t = time_graph_calls(torch, lambda i: q4.flash_decode_ring(*sets[i % 2], 1024, [100000] * 40, 1.0, ws=ws), 10)
    del sets
    nb = 40 * 8 * 1024 * 1024
    res["ring_attention_40seq"] = {"us": round(t * 1e6, 2), "bytes": nb,
                                   "GBps": round(nb / t / 1e9, 1), "frac": round(nb / t / 1e9 / PEAK_GBPS, 4)}
    return res


def time_q8_gemv(q4, torch, N=15360, K=3840, copies=16, launches=96, reps=10, warm=5):
    """The int8 (int8lin) product at the gate/up shape, batch 1: one random
    N(0, 0.02) matrix packed into `copies` separate buffers (1 GB, above the
    last-level cache), launches rotating over them captured into a graph and
    replayed between two HIP events.  Bytes per launch: 1.0625 B per weight."""
    gen = torch.Generator(device="cuda").manual_seed(21)
    w = torch.randn(N, K, device="cuda", generator=gen) * 0.02
    mats = [q4.q8_pack(w) for _ in range(copies)]
    del w
    x = torch.randn(1, K, device="cuda", generator=gen).half()
    y = torch.empty(1, N, device="cuda")
    avg = time_graph_calls(torch, lambda i: q4.q8_gemv(mats[i % copies], N, K, x, y), launches,
                           replays=reps)
    nb = q4.q8_packed_bytes(N, K)
    del mats
    return {"us": round(avg * 1e6, 3), "bytes": nb, "GBps": round(nb / avg / 1e9, 1),
            "frac": round(nb / avg / 1e9 / PEAK_GBPS, 4), "shape": f"{N}x{K}, batch 1"}


def time_int8_step(q4, torch, bytemodel, synth, toks, steps):
    """The same 48-layer step over int8 (int8lin) weights, batch 1 at context
    32768: a second model from the same synthetic weights packed with q8_pack,
    timed like the main figure.  Bytes: the int4 byte model with 34 instead of
    18 bytes per 32-weight block."""
    from dataclasses import replace
    cfg = replace(synth.FULL48, full_cap=32768 + 8)
    m8 = q4.build_decode_model(cfg, 5, 32767, device="cuda", gen_device="cuda", weights="q8")
    torch.cuda.synchronize()
    secs = time_steps(torch, m8, toks, 32767, steps, 2)
    nb = bytemodel.step_bytes(cfg, 32767) + bytemodel.weight_bytes(cfg) * 16 // 18
    del m8
    torch.cuda.empty_cache()
    return {"ms_per_step": round(secs * 1e3 / steps, 4), "tokens_per_s": round(steps / secs, 2),
            "algorithmic_bytes": nb, "achieved_GBps": round(nb * steps / secs / 1e9, 1)}


def time_vrow_steps(q4, torch, bytemodel, model, toks, steps, ctx_hi):
    """The same step with the full layers caching only the V row (the key
    formed from it): the bench model's layers and V caches, kv_format 1, at
    positions 32767 and ctx_hi - 1."""
    layers = [dict(L, k_cache=None) if L["is_full"] else L for L in model.layers]
    mv = q4.DecodeModel(model.cfg, layers, model.embed, model.final_norm, 0, 1)
    res = {}
    for pos in (32767, ctx_hi - 1):
        secs = time_steps(torch, mv, toks, pos, steps, 2)
        nb = bytemodel.step_bytes(model.cfg, pos, kv_format=1)
        res[f"ctx{pos + 1}"] = {"ms_per_step": round(secs * 1e3 / steps, 4), "tokens_per_s": round(steps / secs, 2),
                                "algorithmic_bytes": nb, "achieved_GBps": round(nb * steps / secs / 1e9, 1)}
    return res


def time_prefill(q4, torch, bytemodel, model, reps=3):
    """Prefill chunks of 64 tokens on the bench model (the caches are those
    of the decode figures): a chunk at positions 0 .. 63 and one ending at
    position 32767 (every row attends up to 32K positions on the full
    layers), each timed over `reps` eager calls between HIP events.  Bytes:
    the weights and head once per chunk, and every cached position the
    chunk's rows attend once (they share each K/V tile)."""
    from int4_q4_gemv_amd import synth
    cfg = model.cfg
    toks = [int(t) for t in synth.tokens(cfg, 64, 9)]
    res = {}
    for name, pos0 in (("pos0", 0), ("ctx32768", 32768 - 64)):
        model.prefill(toks, pos0, want_logits=False)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            model.prefill(toks, pos0, want_logits=False)
        e1.record()
        e1.synchronize()
        secs = e0.elapsed_time(e1) * 1e-3 / reps
        nb = bytemodel.chunk_bytes(cfg, pos0, 64)
        res[name] = {"ms_per_chunk": round(secs * 1e3, 3), "tokens_per_s": round(64 / secs, 1),
                     "algorithmic_bytes": nb, "achieved_GBps": round(nb / secs / 1e9, 1)}
    return res


def time_gemm(q4, torch, N=15360, K=3840, n=64, copies=16, launches=48):
    """The chunk product alone at the gate/up shape with 64 rows (16 packed
    copies rotated, above the last-level cache), as q4_gemm launches it (one
    run of K).  Work: 2 n N K flops; bytes: the q4 weights."""
    gen = torch.Generator(device="cuda").manual_seed(31)
    w = torch.randn(N, K, device="cuda", generator=gen) * 0.02
    mats = [q4.q4_pack(w) for _ in range(copies)]
    del w
    x = torch.randn(n, K, device="cuda", generator=gen).half()
    y = torch.empty(n, N, device="cuda")
    avg = time_graph_calls(torch, lambda i: q4.q4_gemm(mats[i % copies], N, K, x, y), launches)
    del mats
    nb = N * K // 32 * 18
    return {"us": round(avg * 1e6, 2), "TFLOPs": round(2 * n * N * K / avg / 1e12, 1),
            "GBps": round(nb / avg / 1e9, 1), "shape": f"{N}x{K}, {n} rows"}


COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4_gemv_step_launches_traffic.txt")
GEMV_SOURCES = ("int4_q4_gemv_amd/csrc/gemv_kernels.h", "int4_q4_gemv_amd/csrc/device_common.h",
                "int4_q4_gemv_amd/csrc/q4dec.hip")


def gemv_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_launches(q4, torch, model):
    """What the two counter runs profile: a plain device copy of COPY_BYTES
    (its FETCH_SIZE / WRITE_SIZE calibrate the counters to bytes), then the
    step's q/k/v, output and down products (decode_step_gemvs), twice."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    model.step([1], 32767, want_logits=False)
    for _ in range(2):
        model.step_gemvs(1)
    torch.cuda.synchronize()


def gemv_lds_launches(q4, torch):
    """What the GEMV LDS counter run profiles, eagerly: the standalone
    15360 x 3840 product at batch 1, then at batch 4, three dispatches each."""
    N, K = 15360, 3840
    g = torch.Generator(device="cuda").manual_seed(1)
    w = torch.randn(N, K, device="cuda", generator=g) * 0.05
    packed = q4.q4_pack(w)
    del w
    for B in (1, 4):
        x = (torch.randn(B, K, device="cuda", generator=g) * 0.5).half()
        for _ in range(3):
            q4.q4_gemv(packed, N, K, x)
    torch.cuda.synchronize()


def attention_traffic_launches(q4, torch):
    """What the attention counter runs profile, eagerly (one dispatch per
    kernel): a plain device copy of COPY_BYTES (calibration), then twice each
    full attention at context 32768 (16 q heads, D 512; the K/V pair layout
    and the one-row layout, in buffers larger than the last-level cache), the
    ring (8 KV heads, D 256, W 1024, R 2048) for one sequence, and 40 rings
    in one call."""
    from int4_q4_gemv_amd import synth
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    del src, dst
    cap = 131076
    bufs = [synth.full_attn_inputs(131072, cap, seed=3 + i, device="cuda") for i in range(4)]
    kw = synth.normal((512,), 0.1, synth.gen(3), mean=1.0).to("cuda")
    ws = q4._fd_ws(1, 1, 16, 512, "cuda")
    for i in range(2):
        q4.flash_decode_full(*bufs[i], 32767, 1.0, ws=ws)
    for i in range(2):
        q4.flash_decode_full_vrow(bufs[2 + i][0], bufs[2 + i][2], kw, 1e6, 64, 32767, 1.0, ws=ws)
    torch.cuda.synchronize()
    del bufs
    q, k, v = (t.to("cuda") for t in synth.ring_inputs(100000, n_rows=1, n_rejected=4))
    ws = q4._fd_ws(1, 1, 16, 256, "cuda")
    for _ in range(2):
        q4.flash_decode_ring(q, k, v, 1024, 100000, 1.0, ws=ws)
    rings = [synth.ring_inputs(100000, n_rows=1, n_rejected=4, seed=100 + s, device="cuda") for s in range(40)]
    qs, ks, vs = (torch.stack([r[j] for r in rings]).to("cuda") for j in range(3))
    del rings
    ws = q4._fd_ws(40, 1, 16, 256, "cuda")
    q4.flash_decode_ring(qs, ks, vs, 1024, [100000] * 40, 1.0, ws=ws)
    torch.cuda.synchronize()


def stored_traffic():
    """Per-launch HBM bytes of the roofline kernel from the committed counter
    summary, or None when the summary is absent or was taken on other GEMV
    sources than the ones built now."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("gemv_source_sha256_16") != gemv_source_hash():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def time_steps(torch, model, toks, pos, steps, warmup):
    for i in range(warmup):
        model.step(toks[i % len(toks)], pos, want_logits=False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        model.step(toks[i % len(toks)], pos, want_logits=False)
    e1.record()
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def cpu_baseline(model, torch):
    """The oracle on the host cores, on a bounded sample of the same workload:
    layer 0 (sliding) and layer 5 (full, context 32768) of the same weights,
    plus the vocab head; per-token time = 40 t_sliding + 8 t_full + t_head."""
    import numpy as np
    import oracle
    from int4_q4_gemv_amd import synth
    cfg = model.cfg
    seed = 5
    blk = {}
    for l in (0, 5):
        lp = synth.layer_params(cfg, l, seed, device="cuda")
        blk[l] = {n: oracle.q4_pack(w.cpu().numpy()) for n, w in lp.mats.items()}
        del lp
    f16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()
    emb = f16(model.embed)

    def om(ls):
        layers = []
        for l in ls:
            L = model.layers[l]
            layers.append(oracle.OracleLayer(
                is_full=bool(L["is_full"]), v_norm=bool(L["v_norm"]), wq=blk[l]["wq"], wk=blk[l]["wk"],
                wv=blk[l].get("wv"), wo=blk[l]["wo"], wg=blk[l]["wg"], wu=blk[l]["wu"], wd=blk[l]["wd"],
                attn_norm=L["attn_norm"].cpu().numpy(), q_norm=L["q_norm"].cpu().numpy(),
                k_norm=L["k_norm"].cpu().numpy(), post_attn_norm=L["post_attn_norm"].cpu().numpy(),
                pre_ff_norm=L["pre_ff_norm"].cpu().numpy(), post_ff_norm=L["post_ff_norm"].cpu().numpy(),
                layer_scalar=1.0, k_cache=f16(L["k_cache"]), v_cache=f16(L["v_cache"])))
        return oracle.OracleModel(
            hidden=cfg.hidden, n_heads=cfg.n_heads, inter=cfg.inter, vocab=cfg.vocab,
            sl_kv_heads=cfg.sl_kv_heads, sl_head_dim=cfg.sl_head_dim, full_head_dim=cfg.full_head_dim,
            window=cfg.window, ring=cfg.ring, full_cap=cfg.full_cap, sl_theta=cfg.sl_theta,
            full_theta=cfg.full_theta, sl_rot_pairs=cfg.sl_rot_pairs, full_rot_pairs=cfg.full_rot_pairs,
            sl_scale=cfg.sl_scale, full_scale=cfg.full_scale, eps=cfg.eps, softcap=cfg.softcap,
            embed=emb, final_norm=model.final_norm.cpu().numpy(), layers=layers)

    tok = [1234]
    pos = 32767
    m = om([0, 5])                  # its layer 0 is model layer 0 (sliding), layer 1 is layer 5 (full)
    h = m.embed_tokens(tok)
    wall = time.perf_counter()

    def med(f, k):
        ts = []
        for _ in range(k):
            t = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[k // 2]

    def parts(k):
        return (med(lambda: m.run_layer(0, h, pos), k), med(lambda: m.run_layer(1, h, pos), k),
                med(lambda: m.run_head(h, want_logits=False), k))

    cores = oracle.num_threads()
    t_s, t_f, t_h = parts(5)
    oracle.set_num_threads(1)
    t1_s, t1_f, t1_h = parts(1)
    oracle.set_num_threads(cores)
    per_tok = 40 * t_s + 8 * t_f + t_h
    per_tok1 = 40 * t1_s + 8 * t1_f + t1_h
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": ("the oracle's layer 0 (sliding) and layer 5 (full, context 32768) of the same "
                       "12B-shape weights at position 32767, and its vocab head, each timed 5 times "
                       "(median) on all threads and once on one thread; tokens/s = "
                       "1/(40 t_sliding + 8 t_full + t_head)"),
            "cpu_model": cpu, "t_sliding_s": t_s, "t_full_s": t_f, "t_head_s": t_h,
            "one_thread": {"value": 1.0 / per_tok1, "t_sliding_s": t1_s, "t_full_s": t1_f, "t_head_s": t1_h},
            "wall_s": round(time.perf_counter() - wall, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_q4_gemv_amd as q4
    from int4_q4_gemv_amd import bytemodel, synth
    from dataclasses import replace

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.mode == "gemv_lds":
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            gemv_lds_launches(q4, torch)
        print(json.dumps({"mode": "gemv_lds"}))
        return
    if args.mode == "attn_traffic":
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            attention_traffic_launches(q4, torch)
        print(json.dumps({"mode": "attn_traffic", "copy_bytes": COPY_BYTES}))
        return
    ctx_hi = 131072
    cfg = replace(synth.FULL48, full_cap=ctx_hi + 8)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        log("building the 48-layer model on the GPU ...")
        model = q4.build_decode_model(cfg, 5, ctx_hi - 1, device="cuda", gen_device="cuda")
        torch.cuda.synchronize()
        log(f"model ready in {time.perf_counter() - t0:.1f} s")
        toks = [[int(t)] for t in synth.tokens(cfg, 64, 5)]
        out = {}
        if args.mode == "traffic":
            traffic_launches(q4, torch, model)
            print(json.dumps({"mode": "traffic", "copy_bytes": COPY_BYTES,
                              "gemv_source_sha256_16": gemv_source_hash()}))
            return
        if args.mode == "prefill":
            print(json.dumps({"mode": "prefill", "prefill64": time_prefill(q4, torch, bytemodel, model)}))
            return
        if args.mode in ("full", "gemv"):
            avg_s, launches, nbytes = time_step_gemvs(q4, torch, model)
            ach = nbytes / avg_s / 1e9
            out["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                               "frac": round(ach / PEAK_GBPS, 4), "traffic": stored_traffic(),
                               "kernel": "k_q4_gemv<1,0,4,0>: the step's q/k/v, output and down products in the "
                                         "step's launch configuration (decode_step_gemvs, 144 launches per step)",
                               "bytes_per_launch": round(nbytes), "avg_launch_us": round(avg_s * 1e6, 3),
                               "launches": launches}
            log(f"step q/k/v, o, down products: {avg_s * 1e6:.2f} us/launch, {ach:.0f} GB/s")
            out["gemv_standalone"] = time_gemv_shapes(q4, torch, model)
            log(f"q4_gemv alone: {out['gemv_standalone']}")
            peak_meas = time_stream_read(q4, torch)
            out["roofline"]["achievable"] = {
                "GBps": round(peak_meas, 1), "kernel": "q4_stream_read over 4 GiB (plain 16-byte streaming read)",
                "frac_of_peak": round(peak_meas / PEAK_GBPS, 4), "gemv_frac_of_achievable": round(ach / peak_meas, 4)}
            log(f"plain streaming read, 4 GiB: {peak_meas:.0f} GB/s")
            if args.mode == "gemv":
                print(json.dumps(out))
                return
        if args.mode == "verify":
            blocks = [[int(t) for t in synth.tokens(cfg, 4, 50 + i)] for i in range(8)]
            sv = time_steps(torch, model, blocks, 32764, args.steps, args.warmup)
            print(json.dumps({"mode": "verify", "verify4_ctx32768_ms_per_block": round(sv * 1e3 / args.steps, 4)}))
            return
        pos = 32767
        secs = time_steps(torch, model, toks, pos, args.steps, args.warmup)
        ms = secs * 1e3 / args.steps
        tok_s = args.steps / secs
        step_bytes = bytemodel.step_bytes(cfg, pos)
        log(f"decode ctx 32768: {ms:.3f} ms/step, {tok_s:.1f} tok/s")
        extra = {}
        if args.mode == "full":
            k2 = max(5, args.steps // 5)
            s131 = time_steps(torch, model, toks, ctx_hi - 1, k2, 2)
            extra["ctx131072"] = {"ms_per_step": round(s131 * 1e3 / k2, 4),
                                  "tokens_per_s": round(k2 / s131, 2),
                                  "achieved_GBps": round(bytemodel.step_bytes(cfg, ctx_hi - 1) * k2 / s131 / 1e9, 1)}
            blocks = [[int(t) for t in synth.tokens(cfg, 4, 50 + i)] for i in range(8)]
            sv = time_steps(torch, model, blocks, 32764, k2, 2)
            extra["verify4_ctx32768"] = {"ms_per_block": round(sv * 1e3 / k2, 4),
                                         "rows_per_s": round(4 * k2 / sv, 2),
                                         "achieved_GBps": round(step_bytes * k2 / sv / 1e9, 1)}
            log(f"ctx 131072: {extra['ctx131072']}; verify4: {extra['verify4_ctx32768']}")
            extra["attention_kernels"] = time_attention(q4, torch)
            log(f"attention kernels: {extra['attention_kernels']}")
            extra["vrow_kv"] = time_vrow_steps(q4, torch, bytemodel, model, toks, k2, ctx_hi)
            log(f"one-row full-layer KV: {extra['vrow_kv']}")
            extra["prefill64"] = time_prefill(q4, torch, bytemodel, model)
            log(f"prefill chunks: {extra['prefill64']}")
            extra["chunk_gemm"] = time_gemm(q4, torch)
            log(f"chunk product: {extra['chunk_gemm']}")
            extra["q8_gemv"] = time_q8_gemv(q4, torch)
            log(f"q8 (int8lin) gemv: {extra['q8_gemv']}")
            extra["int8_ctx32768"] = time_int8_step(q4, torch, bytemodel, synth, toks, k2)
            log(f"int8 (int8lin) step: {extra['int8_ctx32768']}")
    res = {
        "metric": "decode tokens/s (batch 1, 48 layers) + achieved HBM GB/s as % of peak",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4(q4_0) x f16 -> f32", "data": "synthetic",
        "config": {"workload": "48-layer 12B-shape decode step (40 sliding + 8 full layers), batch 1, "
                               "context 32768 (every timed step decodes position 32767)",
                   "layers": 48, "hidden": 3840, "inter": 15360, "vocab": 262144, "ctx": 32768,
                   "batch": 1, "window": 1024, "ring": 2048},
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_GBPS, 4)},
    }
    res.update(out)
    res.update(extra)
    if args.mode == "full" and not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(model, torch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
