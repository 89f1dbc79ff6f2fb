"""Shared helpers for the GPU parity tests (comparison bar, oracle models)."""
import numpy as np
import torch

# Tolerance on fp32-accumulated outputs: |gpu - oracle| <= ATOL + RTOL * |oracle|
ATOL = 2e-3
RTOL = 1e-3


def assert_close(gpu, ref, atol=ATOL, rtol=RTOL, what=""):
    g = gpu.detach().double().cpu().numpy() if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {g[i]!r} oracle {r[i]!r}")


def assert_close_composed(gpu, ref, atol=ATOL, rtol=RTOL, frac=0.98, factor=4.0, what=""):
    """The bar for outputs of a composition with fp16 rounding points inside
    it (a whole layer and the 262144-row head): the RMS error within the
    relative bar of the reference's RMS plus a quarter of the absolute bar,
    at least ``frac`` of the elements within the elementwise bar and none
    beyond ``factor`` times it.  In scale-1 attention the fp32-vs-fp64
    accumulation error of the scores flips fp16 roundings of the attention
    output, so two correct fp32 implementations (two summation orders of the
    same kernels) already differ by about the elementwise bar on a few
    elements; kernel-level outputs keep the elementwise bar (assert_close)."""
    inside, worst, rms, rms_bar = composed_stats(gpu, ref, atol, rtol, what)
    assert inside >= frac and worst <= factor and rms <= rms_bar, (
        f"{what}: {inside:.5f} of elements within the bar (need {frac}), worst error/bound {worst:.2f} "
        f"(need <= {factor}), rms error {rms:.2e} (need <= {rms_bar:.2e})")
    return inside


def composed_stats(gpu, ref, atol=ATOL, rtol=RTOL, what=""):
    """(fraction of elements within the elementwise bar, worst error / bar,
    RMS error, the composed RMS bar: rtol * RMS(ref) + atol / 4)."""
    g = gpu.detach().double().cpu().numpy() if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    inside = float((err <= bound).mean())
    worst = float((err / bound).max())
    rms = float(np.sqrt((err ** 2).mean()))
    rms_bar = rtol * float(np.sqrt((r ** 2).mean())) + atol / 4
    return inside, worst, rms, rms_bar


def f16bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_model_from_device(orc, cfg, gm, blocks):
    """Oracle model over the same inputs as the GPU model ``gm``: the oracle's
    own blocks (``blocks[l][name]``, q4_0 or int8 as ``gm``'s weight format,
    packed by the oracle from the fp32 weights), host copies of the norms,
    table and caches."""
    layers = []
    for l, L in enumerate(gm.layers):
        layers.append(orc.OracleLayer(
            is_full=bool(L["is_full"]), v_norm=bool(L["v_norm"]),
            wq=blocks[l]["wq"], wk=blocks[l]["wk"], wv=blocks[l].get("wv"), wo=blocks[l]["wo"],
            wg=blocks[l]["wg"], wu=blocks[l]["wu"], wd=blocks[l]["wd"],
            attn_norm=L["attn_norm"].cpu().numpy(), q_norm=L["q_norm"].cpu().numpy(),
            k_norm=L["k_norm"].cpu().numpy(), post_attn_norm=L["post_attn_norm"].cpu().numpy(),
            pre_ff_norm=L["pre_ff_norm"].cpu().numpy(), post_ff_norm=L["post_ff_norm"].cpu().numpy(),
            layer_scalar=float(L["layer_scalar"]),
            k_cache=None if L.get("k_cache") is None else f16bits(L["k_cache"]).copy(),
            v_cache=f16bits(L["v_cache"]).copy()))
    return orc.OracleModel(
        hidden=cfg.hidden, n_heads=cfg.n_heads, inter=cfg.inter, vocab=cfg.vocab,
        sl_kv_heads=cfg.sl_kv_heads, sl_head_dim=cfg.sl_head_dim, full_head_dim=cfg.full_head_dim,
        window=cfg.window, ring=cfg.ring, full_cap=cfg.full_cap,
        sl_theta=cfg.sl_theta, full_theta=cfg.full_theta,
        sl_rot_pairs=cfg.sl_rot_pairs, full_rot_pairs=cfg.full_rot_pairs,
        sl_scale=cfg.sl_scale, full_scale=cfg.full_scale, eps=cfg.eps, softcap=cfg.softcap,
        embed=f16bits(gm.embed), final_norm=gm.final_norm.cpu().numpy(), layers=layers,
        weight_format=int(getattr(gm, "weight_format", 0)), kv_format=int(getattr(gm, "kv_format", 0)))


def check_argmax(gpu_logits, gpu_argmax, ref_logits, tol_margin):
    """The greedy id is unique only where the oracle's top-2 margin is clear;
    otherwise it must be a valid near-maximum.  Always: the GPU id is the
    lowest index of the GPU logits' maximum."""
    gl = gpu_logits.detach().cpu().numpy()
    ga = gpu_argmax.detach().cpu().numpy()
    for i in range(ga.shape[0]):
        assert ga[i] == int(np.argmax(gl[i])), "argmax is not the first maximum of the logits"
        r = ref_logits[i]
        top = np.sort(r)[-2:]
        if top[1] - top[0] > tol_margin:
            assert ga[i] == int(np.argmax(r)), (i, ga[i], int(np.argmax(r)))
        else:
            assert r[ga[i]] >= top[1] - tol_margin


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def check_layer_stages(orc, gm, om, l, h_in, pos0, n, logits, what=""):
    """Every stage of the last layer of the step ``gm`` just ran (width n at
    pos0, its last layer being the oracle's layer ``l``; ``h_in`` the residual
    stream entering it), each against the oracle's stage fed the GPU's own
    values at the stage's input, so every comparison is elementwise:
    attention input, raw q/k/v projections, finished queries, the K/V rows
    written, attention (over the GPU's own caches), o-proj residual, MLP
    input, GELU * up, down residual, head input and logits.  Writes the
    GPU's K/V rows into the oracle layer's cache."""
    import int4_q4_gemv_amd as q4
    L = om.layers[l]
    D, Hkv = om._dims(l)
    Hq = om.n_heads
    st = lambda s: gm.stage(n, s)
    h_in = np.asarray(h_in, dtype=np.float64).reshape(n, -1)

    xa = f16bits(st(q4.STAGE_X_ATTN))
    assert_close(_f16(xa), _f16(om.stage_attn_in(l, h_in)), what=f"{what} attention input")
    qkv = st(q4.STAGE_QKV).double().cpu().numpy()
    q_r, k_r, v_r = om.stage_qkv(l, xa)
    qg, kg = qkv[:, :Hq * D], qkv[:, Hq * D:(Hq + Hkv) * D]
    vg = kg if L.is_full else qkv[:, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D]
    assert_close(qg, q_r, what=f"{what} q projection")
    assert_close(kg, k_r, what=f"{what} k projection")
    if not L.is_full:
        assert_close(vg, v_r, what=f"{what} v projection")

    # finishing from the GPU's raw projections (writes the oracle's cache rows)
    q16_ref = om.stage_finish(l, qg, kg, vg, pos0)
    q16 = f16bits(st(q4.STAGE_Q16)).reshape(n, Hq, D)
    assert_close(_f16(q16), _f16(q16_ref), what=f"{what} finished queries")
    gl = gm.layers[-1]
    for nm in ("k_cache", "v_cache"):
        oc = getattr(L, nm)
        if oc is None or gl.get(nm) is None:
            continue
        gc = f16bits(gl[nm])
        if L.is_full:
            sel = (slice(pos0, pos0 + n),)
        else:
            sel = (slice(None), [(pos0 + i) % om.ring for i in range(n)])
        assert_close(_f16(gc[sel]), _f16(oc[sel]), what=f"{what} {nm} rows written")
        oc[sel] = gc[sel]                                 # attention over the GPU's own caches
    att_ref = om.stage_attend(l, q16, pos0)
    o16 = f16bits(st(q4.STAGE_O16)).reshape(n, Hq, D)
    assert_close(_f16(o16), att_ref, what=f"{what} attention output")

    hm = st(q4.STAGE_H_MID).double().cpu().numpy()
    assert_close(hm, om.stage_oproj(l, o16, h_in), what=f"{what} residual after attention")
    xm = f16bits(st(q4.STAGE_X_MLP))
    assert_close(_f16(xm), _f16(om.stage_mlp_in(l, hm)), what=f"{what} MLP input")
    a16 = f16bits(st(q4.STAGE_A16))
    assert_close(_f16(a16), _f16(om.stage_gateup(l, xm)), what=f"{what} gelu(gate) * up")
    ho = st(q4.STAGE_H_OUT).double().cpu().numpy()
    assert_close(ho, om.stage_down(l, a16, hm), what=f"{what} residual after the layer")
    xh = f16bits(st(q4.STAGE_X_HEAD))
    assert_close(_f16(xh), _f16(om.head_input(ho)), what=f"{what} head input")
    if logits is not None:
        ref, _ = om.head_logits(xh)
        assert_close(logits, ref, what=f"{what} logits")
    return ho
