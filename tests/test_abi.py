"""The C-ABI library loads and exports every entry point include/q4dec.h
declares; host-side argument checks reject bad calls before any HIP work.
No compute call is made here (this runs without a GPU)."""
import ctypes as C
import os
import re

import pytest

import int4_q4_gemv_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "q4dec.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+([a-z_0-9]+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ("q4_pack", "q4_gemv", "flash_decode_full", "flash_decode_ring", "decode_step"):
        assert name in fns
    assert set(fns) == set(q4.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_sizes():
    L = q4.lib()
    assert L.q4dec_status_str(0) == b"Q4_OK"
    for s in (-1, -2, -3, -4, -5, -6):
        assert L.q4dec_status_str(s).startswith(b"Q4_E")
    assert q4.packed_bytes(3840, 15360) == 33_177_600
    assert q4.packed_bytes(100, 64) == 112 * 4 * 18         # 16-row tiles, 4-block quads
    assert q4.packed_bytes(10, 48) == 0                     # K not a multiple of 32
    assert L.flash_decode_workspace_size(1, 1, 16, 96) == 0  # unsupported head_dim


def test_argument_checks_fail_before_launch():
    L = q4.lib()
    fake = C.c_void_p(0x10000)      # never dereferenced: every call below fails its checks
    odd = C.c_void_p(0x10008)
    assert L.q4_pack(None, 0, 64, 64, fake, 1 << 20, None, None) == q4.Q4_EINVAL
    assert L.q4_pack(fake, 7, 64, 64, fake, 1 << 20, None, None) == q4.Q4_EINVAL
    assert L.q4_pack(fake, 0, 64, 48, fake, 1 << 20, None, None) == q4.Q4_ESHAPE
    assert L.q4_pack(fake, 0, 64, 64, fake, 10, None, None) == q4.Q4_ENOSPACE
    assert L.q4_pack(odd, 0, 64, 64, fake, 1 << 20, None, None) == q4.Q4_EALIGN
    assert L.q4_gemv(fake, 64, 64, fake, 5, fake, None) == q4.Q4_ESHAPE
    assert L.q4_gemv(fake, 64, 40, fake, 1, fake, None) == q4.Q4_ESHAPE
    assert L.q4_gemv(fake, 64, 65536, fake, 1, fake, None) == q4.Q4_ESHAPE
    assert L.q4_gemv(None, 64, 64, fake, 1, fake, None) == q4.Q4_EINVAL
    assert L.q4_gemv(odd, 64, 64, fake, 1, fake, None) == q4.Q4_EALIGN
    pos = (C.c_int32 * 1)(100)
    ws = 1 << 30
    # position beyond capacity
    assert L.flash_decode_full(fake, fake, fake, 0, 100, 16, 512, pos, 1, 1, C.c_float(1.0),
                               fake, fake, ws, None) == q4.Q4_ERANGE
    # ring too short for a 4-row verify block: R < W + n - 1
    assert L.flash_decode_ring(fake, fake, fake, 0, 16, 8, 256, 1026, 1024, pos, 1, 4,
                               C.c_float(1.0), fake, fake, ws, None) == q4.Q4_ERANGE
    assert L.flash_decode_ring(fake, fake, fake, 0, 16, 8, 256, 2048, 4096, pos, 1, 1,
                               C.c_float(1.0), fake, fake, ws, None) == q4.Q4_ERANGE
    assert L.flash_decode_ring(fake, fake, fake, 0, 16, 5, 256, 2048, 1024, pos, 1, 1,
                               C.c_float(1.0), fake, fake, ws, None) == q4.Q4_ESHAPE
    # a ring holds at least one 32-position tile
    assert L.flash_decode_ring(fake, fake, fake, 0, 16, 8, 256, 16, 8, pos, 1, 1,
                               C.c_float(1.0), fake, fake, ws, None) == q4.Q4_ESHAPE
    # one-row full layers: D in {128, 512}, at most 64 rotated pairs, theta > 0, kw given and aligned
    fv = L.flash_decode_full_vrow
    ok = (fake, fake, 0, 200, 16, 512, fake, C.c_double(1e6), 64, pos, 1, 1, C.c_float(1.0), fake, fake, ws, None)
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[{"D": 5, "kw": 6, "theta": 7, "rot": 8, "cap": 3}[k]] = v
        return fv(*a)
    assert call(D=256) == q4.Q4_ESHAPE
    assert call(rot=65) == q4.Q4_ESHAPE
    assert call(theta=C.c_double(0.0)) == q4.Q4_ESHAPE
    assert call(kw=None) == q4.Q4_EINVAL
    assert call(kw=odd) == q4.Q4_EALIGN
    assert call(cap=100) == q4.Q4_ERANGE


def test_decode_step_checks():
    from int4_q4_gemv_amd import synth
    cfg = synth.TOY
    L = q4.lib()
    fake = 0x10000
    lay = (q4.Layer * 2)()
    for i in range(2):
        lay[i] = q4.Layer(int(cfg.is_full(i)), 1, *([fake] * 13), 1.0, fake, fake)
    m = q4.Model(cfg.hidden, cfg.n_heads, cfg.inter, cfg.vocab, 2, cfg.sl_kv_heads, cfg.sl_head_dim,
                 cfg.full_head_dim, cfg.window, cfg.ring, cfg.full_cap, cfg.sl_rot_pairs,
                 cfg.full_rot_pairs, cfg.sl_theta, cfg.full_theta, 1.0, 1.0, 1e-6, 30.0, fake, fake, lay)
    need = L.decode_step_workspace_size(C.byref(m), 1)
    assert need > 0
    tok = (C.c_int32 * 4)(1, 2, 3, 4)
    big = C.c_size_t(need * 2)
    f = C.c_void_p(fake)
    assert L.decode_step(C.byref(m), tok, 5, 0, f, f, f, big, None) == q4.Q4_ESHAPE
    assert L.decode_step(C.byref(m), tok, 1, -1, f, f, f, big, None) == q4.Q4_ERANGE
    assert L.decode_step(C.byref(m), tok, 1, cfg.full_cap, f, f, f, big, None) == q4.Q4_ERANGE
    assert L.decode_step(C.byref(m), tok, 1, 5, f, f, f, C.c_size_t(16), None) == q4.Q4_ENOSPACE
    bad = (C.c_int32 * 1)(cfg.vocab)
    assert L.decode_step(C.byref(m), bad, 1, 5, f, f, f, big, None) == q4.Q4_ERANGE
    assert L.decode_step_hidden(C.byref(m), f, C.c_size_t(16), 1, f, None) == q4.Q4_ENOSPACE
    assert L.decode_step_hidden(C.byref(m), f, big, 5, f, None) == q4.Q4_ESHAPE
    # kv_format: 0 or 1; the one-row layout needs the V norm on full layers and
    # does not need their K cache
    m.kv_format = 2
    assert L.decode_step(C.byref(m), tok, 1, 5, f, f, f, big, None) == q4.Q4_ESHAPE
    m.kv_format = 1
    lay[1].k_cache = None
    assert L.decode_step(C.byref(m), bad, 1, 5, f, f, f, big, None) == q4.Q4_ERANGE   # passes the layer checks
    lay[1].v_norm = 0
    assert L.decode_step(C.byref(m), tok, 1, 5, f, f, f, big, None) == q4.Q4_EINVAL
    m.kv_format = 0
    assert L.decode_step(C.byref(m), tok, 1, 5, f, f, f, big, None) == q4.Q4_EINVAL  # K cache missing
    lay[1].v_norm, lay[1].k_cache = 1, fake
    m.ring = cfg.window + 2      # a 4-row block needs R >= W + 3
    assert L.decode_step(C.byref(m), tok, 4, 5, f, f, f, big, None) == q4.Q4_ERANGE
    m.ring, m.window = 16, 8     # a ring holds at least one 32-position tile
    assert L.decode_step(C.byref(m), tok, 1, 5, f, f, f, big, None) == q4.Q4_ESHAPE


def test_stage_export_sizes_and_checks():
    from int4_q4_gemv_amd import synth
    cfg = synth.TOY
    L = q4.lib()
    fake = 0x10000
    lay = (q4.Layer * 2)()
    for i in range(2):
        lay[i] = q4.Layer(int(cfg.is_full(i)), 1, *([fake] * 13), 1.0, fake, fake)
    m = q4.Model(cfg.hidden, cfg.n_heads, cfg.inter, cfg.vocab, 2, cfg.sl_kv_heads, cfg.sl_head_dim,
                 cfg.full_head_dim, cfg.window, cfg.ring, cfg.full_cap, cfg.sl_rot_pairs,
                 cfg.full_rot_pairs, cfg.sl_theta, cfg.full_theta, 1.0, 1.0, 1e-6, 30.0, fake, fake, lay)
    H, I, Hq = cfg.hidden, cfg.inter, cfg.n_heads
    D = cfg.full_head_dim if cfg.is_full(1) else cfg.sl_head_dim       # the last layer's head size
    ld = max(Hq * cfg.sl_head_dim + 2 * cfg.sl_kv_heads * cfg.sl_head_dim, Hq * cfg.full_head_dim + cfg.full_head_dim)
    want = {q4.STAGE_H_OUT: 4 * H, q4.STAGE_H_MID: 4 * H, q4.STAGE_X_ATTN: 2 * H, q4.STAGE_QKV: 4 * ld,
            q4.STAGE_Q16: 2 * Hq * D, q4.STAGE_O16: 2 * Hq * D, q4.STAGE_X_MLP: 2 * H,
            q4.STAGE_A16: 2 * I, q4.STAGE_X_HEAD: 2 * H}
    for n in (1, 4):
        for st, b in want.items():
            assert L.decode_step_stage_bytes(C.byref(m), n, st) == n * b, (n, st)
    assert L.decode_step_stage_bytes(C.byref(m), 1, 9) == 0
    assert L.decode_step_stage_bytes(C.byref(m), 5, 0) == 0
    need = L.decode_step_workspace_size(C.byref(m), 1)
    f = C.c_void_p(fake)
    big = C.c_size_t(need)
    assert L.decode_step_stage(C.byref(m), f, big, 1, 9, f, C.c_size_t(1 << 20), None) == q4.Q4_EINVAL
    assert L.decode_step_stage(C.byref(m), f, big, 1, 0, f, C.c_size_t(4 * H - 1), None) == q4.Q4_ENOSPACE
    assert L.decode_step_stage(C.byref(m), f, C.c_size_t(need - 1), 1, 0, f, C.c_size_t(4 * H), None) == q4.Q4_ENOSPACE
    assert L.decode_step_stage(C.byref(m), None, big, 1, 0, f, C.c_size_t(4 * H), None) == q4.Q4_EINVAL
    assert L.q4dec_graph_count() == 0


def test_version_carries_the_source_hash():
    v = q4.lib().q4dec_version().decode()
    assert v.startswith("q4dec ") and v.endswith(" src " + q4.source_hash())


def test_chunk_entry_points_check_their_arguments():
    """q4_gemm and prefill_chunk reject bad calls on the host, before any launch."""
    from int4_q4_gemv_amd import synth
    L = q4.lib()
    fake = C.c_void_p(0x10000)
    odd = C.c_void_p(0x10008)
    assert L.q4_gemm(None, 64, 128, fake, 4, fake, None) == q4.Q4_EINVAL
    assert L.q4_gemm(fake, 64, 128, fake, 0, fake, None) == q4.Q4_ESHAPE       # no rows
    assert L.q4_gemm(fake, 64, 128, fake, 65, fake, None) == q4.Q4_ESHAPE      # more than a chunk
    assert L.q4_gemm(fake, 64, 100, fake, 4, fake, None) == q4.Q4_ESHAPE      # K % 32
    assert L.q4_gemm(fake, 64, 128, odd, 4, fake, None) == q4.Q4_EALIGN
    cfg = synth.TOY
    lay = (q4.Layer * 2)()
    for i in range(2):
        lay[i] = q4.Layer(int(cfg.is_full(i)), 1, *([0x10000] * 13), 1.0, 0x10000, 0x10000)
    m = q4.Model(cfg.hidden, cfg.n_heads, cfg.inter, cfg.vocab, 2, cfg.sl_kv_heads, cfg.sl_head_dim,
                 cfg.full_head_dim, cfg.window, cfg.ring, cfg.full_cap, cfg.sl_rot_pairs,
                 cfg.full_rot_pairs, cfg.sl_theta, cfg.full_theta, 1.0, 1.0, 1e-6, 30.0, 0x10000, 0x10000, lay)
    need = L.prefill_chunk_workspace_size(C.byref(m))
    assert need > 0
    big = C.c_size_t(need * 2)
    toks = (C.c_int32 * 65)(*range(65))
    f = fake
    assert L.prefill_chunk(C.byref(m), toks, 65, 0, f, f, None, f, big, None) == q4.Q4_ESHAPE   # > 64 rows
    assert L.prefill_chunk(C.byref(m), toks, 64, -1, f, f, None, f, big, None) == q4.Q4_ERANGE
    assert L.prefill_chunk(C.byref(m), toks, 64, cfg.full_cap - 10, f, f, None, f, big, None) == q4.Q4_ERANGE
    assert L.prefill_chunk(C.byref(m), toks, 64, 0, f, f, None, f, C.c_size_t(64), None) == q4.Q4_ENOSPACE
    m.weight_format = 1                      # the chunk products take q4 weights only
    assert L.prefill_chunk(C.byref(m), toks, 64, 0, f, f, None, f, big, None) == q4.Q4_ESHAPE
    m.weight_format = 0
    m.ring = cfg.window + 62                 # R >= W + n - 1 fails for 64 rows
    assert L.prefill_chunk(C.byref(m), toks, 64, 0, f, f, None, f, big, None) == q4.Q4_ERANGE


def test_spec_accept_rule():
    """The host acceptance rule of a verify block (no device work): drafts are
    kept while they equal the target's argmax of the previous row; the
    target's own token at the first mismatch (or after the last draft) ends
    the emitted run."""
    acc = q4.spec_accept
    assert acc([5, 1, 2, 3], [1, 2, 3, 9]) == [1, 2, 3, 9]      # every draft accepted, plus one
    assert acc([5, 1, 2, 3], [1, 7, 3, 9]) == [1, 7]            # second draft rejected
    assert acc([5, 1, 2, 3], [4, 2, 3, 9]) == [4]               # first draft rejected
    assert acc([5, 1, 2, 3], [1, 2, 4, 3]) == [1, 2, 4]         # a later match does not resume
    assert acc([5], [8]) == [8]                                 # plain greedy step
    assert acc([0, 0], [0, 0]) == [0, 0]
    L = q4.lib()
    b = (C.c_int32 * 4)(1, 2, 3, 4)
    e = (C.c_int32 * 4)()
    ne = C.c_int(-1)
    assert L.q4_spec_accept(b, b, 0, e, C.byref(ne)) == q4.Q4_ESHAPE
    assert L.q4_spec_accept(b, b, 5, e, C.byref(ne)) == q4.Q4_ESHAPE
    assert L.q4_spec_accept(None, b, 4, e, C.byref(ne)) == q4.Q4_EINVAL
    assert L.q4_spec_accept(b, b, 4, e, None) == q4.Q4_EINVAL
    assert ne.value == -1


def test_stream_read_checks():
    L = q4.lib()
    fake = C.c_void_p(0x10000)
    odd = C.c_void_p(0x10008)
    assert L.q4_stream_read_sink_words() >= 256
    assert L.q4_stream_read(None, 1024, fake, None) == q4.Q4_EINVAL
    assert L.q4_stream_read(fake, 1024, None, None) == q4.Q4_EINVAL
    assert L.q4_stream_read(fake, 0, fake, None) == q4.Q4_ESHAPE
    assert L.q4_stream_read(fake, 1000, fake, None) == q4.Q4_ESHAPE
    assert L.q4_stream_read(odd, 1024, fake, None) == q4.Q4_EALIGN
