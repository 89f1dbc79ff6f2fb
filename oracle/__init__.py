"""Plain CPU oracle (fp64) for the int4 q4_0 decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``int4_q4_gemv_amd``; the two meet only through
the seeded inputs of ``int4_q4_gemv_amd.synth``.

The arithmetic lives in ``oracle.c`` (see its header for the page citations);
this module is a ctypes binding that moves numpy arrays in and out.

Parity unpinned: the readings of points the pages leave open (norm placement,
RMSNorm eps, GELU form, softcap value, embedding scale, V-norm on sliding
layers, layer_scalar placement) are pinned only by invariants and special
cases in ``tests/test_oracle_*.py``, not against a real checkpoint.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile the oracle with gcc (plain C11 + OpenMP, no fast-math)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i64 = C.c_int64
_i = C.c_int
_d = C.c_double


def _declare(L):
    L.orc_f64_to_f16.restype = C.c_uint16
    L.orc_f64_to_f16.argtypes = [_d]
    L.orc_f16_to_f64.restype = _d
    L.orc_f16_to_f64.argtypes = [C.c_uint16]
    L.orc_f64_to_f16_array.argtypes = [_p, _i64, _p]
    L.orc_q4_pack.argtypes = [_p, _i64, _i64, _p]
    L.orc_q4_dequant.argtypes = [_p, _i64, _i64, _p]
    L.orc_q4_gemv.argtypes = [_p, _i64, _i64, _p, _i, _p]
    L.orc_f16_gemv.argtypes = [_p, _i64, _i64, _p, _i, _p]
    L.orc_q8_pack.argtypes = [_p, _i64, _i64, _p]
    L.orc_q8_dequant.argtypes = [_p, _i64, _i64, _p]
    L.orc_q8_gemv.argtypes = [_p, _i64, _i64, _p, _i, _p]
    L.orc_ring_admit.argtypes = [_i64, _i64, _i64, _p]
    L.orc_attend.argtypes = [_p, _i, _i, _i, _p, _p, _i64, _p, _i64, _d, _p]
    L.orc_flash_full.argtypes = [_p, _p, _p, _i64, _i, _i, _i64, _i, _d, _p]
    L.orc_flash_full_vrow.argtypes = [_p, _p, _i64, _i, _i, _i64, _i, _p, _d, _i, _d, _p]
    L.orc_flash_ring.argtypes = [_p, _p, _p, _i, _i, _i, _i64, _i64, _i64, _i, _d, _p]
    L.orc_rmsnorm.argtypes = [_p, _p, _i64, _d, _p]
    L.orc_rope.argtypes = [_p, _i, _i64, _d, _i]
    L.orc_gelu_tanh.restype = _d
    L.orc_gelu_tanh.argtypes = [_d]
    L.orc_softcap.restype = _d
    L.orc_softcap.argtypes = [_d, _d]
    L.orc_decode_step.restype = _i
    L.orc_decode_step.argtypes = [_p, _p, _i, _i64, _p, _p]
    L.orc_num_threads.restype = _i
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [_i]
    L.orc_embed.restype = _i
    L.orc_embed.argtypes = [_p, _p, _i, _p]
    L.orc_run_layer.restype = _i
    L.orc_run_layer.argtypes = [_p, _i, _p, _i, _i64]
    L.orc_head.restype = _i
    L.orc_head.argtypes = [_p, _p, _i, _p, _p]
    L.orc_stage_attn_in.restype = _i
    L.orc_stage_attn_in.argtypes = [_p, _i, _p, _i, _p]
    L.orc_stage_qkv.restype = _i
    L.orc_stage_qkv.argtypes = [_p, _i, _p, _i, _p, _p, _p]
    L.orc_stage_mlp_in.restype = _i
    L.orc_stage_mlp_in.argtypes = [_p, _i, _p, _i, _p]
    L.orc_stage_finish.restype = _i
    L.orc_stage_finish.argtypes = [_p, _i, _p, _p, _p, _i, _i64, _p]
    L.orc_stage_attend.restype = _i
    L.orc_stage_attend.argtypes = [_p, _i, _p, _i, _i64, _p]
    L.orc_stage_oproj.restype = _i
    L.orc_stage_oproj.argtypes = [_p, _i, _p, _i, _p]
    L.orc_stage_gateup.restype = _i
    L.orc_stage_gateup.argtypes = [_p, _i, _p, _i, _p]
    L.orc_stage_down.restype = _i
    L.orc_stage_down.argtypes = [_p, _i, _p, _i, _p]
    L.orc_head_input.restype = _i
    L.orc_head_input.argtypes = [_p, _p, _i, _p]
    L.orc_head_logits.restype = _i
    L.orc_head_logits.argtypes = [_p, _p, _i, _p, _p]


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(_p)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- fp16 ----
def f64_to_f16(x) -> np.ndarray:
    """Round to IEEE binary16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f64_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = np.vectorize(lambda v: lib().orc_f16_to_f64(int(v)), otypes=[np.float64])
    return f(h) if h.size else h.astype(np.float64)


# ---------------------------------------------------------------- q4_0 ----
def q4_pack(w: np.ndarray) -> np.ndarray:
    """fp32 [N, K] -> canonical q4_0 blocks uint8 [N, K/32, 18]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 32 == 0
    out = np.empty((N, K // 32, 18), dtype=np.uint8)
    lib().orc_q4_pack(_ptr(w), N, K, _ptr(out))
    return out


def q4_dequant(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    lib().orc_q4_dequant(_ptr(blocks), N, K, _ptr(out))
    return out


def q4_gemv(blocks: np.ndarray, N: int, K: int, x16: np.ndarray) -> np.ndarray:
    """x16: uint16 fp16 bits [B, K] -> y float64 [B, N]."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
    B = x16.shape[0]
    assert x16.shape[1] == K
    y = np.empty((B, N), dtype=np.float64)
    lib().orc_q4_gemv(_ptr(blocks), N, K, _ptr(x16), B, _ptr(y))
    return y


# ------------------------------------------------------------ q8 int8lin ----
def q8_pack(w: np.ndarray) -> np.ndarray:
    """fp32 [N, K] -> canonical q8 blocks uint8 [N, K/32, 34]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 32 == 0
    out = np.empty((N, K // 32, 34), dtype=np.uint8)
    lib().orc_q8_pack(_ptr(w), N, K, _ptr(out))
    return out


def q8_dequant(blocks: np.ndarray, N: int, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    lib().orc_q8_dequant(_ptr(blocks), N, K, _ptr(out))
    return out


def q8_gemv(blocks: np.ndarray, N: int, K: int, x16: np.ndarray) -> np.ndarray:
    """x16: uint16 fp16 bits [B, K] -> y float64 [B, N]."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
    B = x16.shape[0]
    assert x16.shape[1] == K
    y = np.empty((B, N), dtype=np.float64)
    lib().orc_q8_gemv(_ptr(blocks), N, K, _ptr(x16), B, _ptr(y))
    return y


def f16_gemv(W16: np.ndarray, x16: np.ndarray) -> np.ndarray:
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
    N, K = W16.shape
    B = x16.shape[0]
    y = np.empty((B, N), dtype=np.float64)
    lib().orc_f16_gemv(_ptr(W16), N, K, _ptr(x16), B, _ptr(y))
    return y


# ----------------------------------------------------------- attention ----
def ring_admit(q: int, R: int, W: int) -> np.ndarray:
    out = np.empty(R, dtype=np.uint8)
    lib().orc_ring_admit(q, R, W, _ptr(out))
    return out.astype(bool)


def attend(q16, k16, v16, admit, scale: float) -> np.ndarray:
    """q16 [Hq, D]; k16, v16 [Hkv, S, D]; admit bool [S] -> out [Hq, D]."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    k16 = np.ascontiguousarray(k16, dtype=np.uint16)
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    admit = np.ascontiguousarray(admit, dtype=np.uint8)
    Hq, D = q16.shape
    Hkv, S, _ = k16.shape
    out = np.empty((Hq, D), dtype=np.float64)
    lib().orc_attend(_ptr(q16), Hq, Hkv, D, _ptr(k16), _ptr(v16), S * D,
                     _ptr(admit), S, scale, _ptr(out))
    return out


def flash_full(q16, k16, v16, pos0: int, scale: float) -> np.ndarray:
    """q16 [n, Hq, D]; k16, v16 [cap, D]; row i attends [0, pos0+i]."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    k16 = np.ascontiguousarray(k16, dtype=np.uint16)
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    n, Hq, D = q16.shape
    cap = k16.shape[0]
    assert pos0 + n - 1 < cap
    out = np.empty((n, Hq, D), dtype=np.float64)
    lib().orc_flash_full(_ptr(q16), _ptr(k16), _ptr(v16), cap, Hq, D, pos0, n, scale, _ptr(out))
    return out


def flash_full_vrow(q16, vrow16, kw, theta: float, rot_pairs: int, pos0: int,
                    scale: float) -> np.ndarray:
    """Full layer caching one row per position: q16 [n, Hq, D]; vrow16 [cap, D]
    (the V rows); kw [D] the k_norm multiplier; key t = RoPE_t(kw * v_t)."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    vrow16 = np.ascontiguousarray(vrow16, dtype=np.uint16)
    kw = np.ascontiguousarray(kw, dtype=np.float32)
    n, Hq, D = q16.shape
    cap = vrow16.shape[0]
    assert pos0 + n - 1 < cap and kw.shape == (D,)
    out = np.empty((n, Hq, D), dtype=np.float64)
    lib().orc_flash_full_vrow(_ptr(q16), _ptr(vrow16), cap, Hq, D, pos0, n, _ptr(kw),
                              theta, rot_pairs, scale, _ptr(out))
    return out


def flash_ring(q16, k16, v16, W: int, pos0: int, scale: float) -> np.ndarray:
    """q16 [n, Hq, D]; k16, v16 [Hkv, R, D]; row i sits at position pos0+i."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    k16 = np.ascontiguousarray(k16, dtype=np.uint16)
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    n, Hq, D = q16.shape
    Hkv, R, _ = k16.shape
    out = np.empty((n, Hq, D), dtype=np.float64)
    lib().orc_flash_ring(_ptr(q16), _ptr(k16), _ptr(v16), Hq, Hkv, D, R, W, pos0, n, scale, _ptr(out))
    return out


# ---------------------------------------------------------- elementwise ----
def rmsnorm(x, w=None, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    wp = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        wp = _ptr(w)
    lib().orc_rmsnorm(_ptr(x), wp, x.size, eps, _ptr(out))
    return out


def rope(x, pos: int, theta: float, rot_pairs: int) -> np.ndarray:
    x = np.array(x, dtype=np.float64, copy=True)
    lib().orc_rope(_ptr(x), x.size, pos, theta, rot_pairs)
    return x


def gelu_tanh(g: float) -> float:
    return float(lib().orc_gelu_tanh(float(g)))


def softcap(z: float, c: float) -> float:
    return float(lib().orc_softcap(float(z), float(c)))


# ---------------------------------------------------------- decode step ----
class _Layer(C.Structure):
    _fields_ = [("is_full", _i), ("v_norm", _i),
                ("wq", _p), ("wk", _p), ("wv", _p), ("wo", _p), ("wg", _p), ("wu", _p), ("wd", _p),
                ("attn_norm", _p), ("q_norm", _p), ("k_norm", _p), ("post_attn_norm", _p),
                ("pre_ff_norm", _p), ("post_ff_norm", _p),
                ("layer_scalar", C.c_float),
                ("k_cache", _p), ("v_cache", _p)]


class _Model(C.Structure):
    _fields_ = [("hidden", _i), ("n_heads", _i), ("inter", _i), ("vocab", _i), ("n_layers", _i),
                ("sl_kv_heads", _i), ("sl_head_dim", _i), ("full_head_dim", _i),
                ("window", _i64), ("ring", _i64), ("full_cap", _i64),
                ("sl_theta", _d), ("full_theta", _d),
                ("sl_rot_pairs", _i), ("full_rot_pairs", _i),
                ("sl_scale", _d), ("full_scale", _d), ("eps", _d), ("softcap", _d),
                ("embed", _p), ("final_norm", _p), ("layers", C.POINTER(_Layer)),
                ("weight_format", _i), ("kv_format", _i)]


@dataclass
class OracleLayer:
    is_full: bool
    v_norm: bool
    wq: np.ndarray  # canonical q4_0 (or int8) blocks
    wk: np.ndarray
    wv: np.ndarray | None
    wo: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    attn_norm: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    post_attn_norm: np.ndarray
    pre_ff_norm: np.ndarray
    post_ff_norm: np.ndarray
    layer_scalar: float
    k_cache: np.ndarray | None  # uint16 fp16 bits; sliding [Hkv, R, D], full [cap, D]
                                # (None on full layers of a kv_format 1 model)
    v_cache: np.ndarray


@dataclass
class OracleModel:
    """Host-side model for :func:`decode_step`; arrays are kept alive here."""
    hidden: int
    n_heads: int
    inter: int
    vocab: int
    sl_kv_heads: int
    sl_head_dim: int
    full_head_dim: int
    window: int
    ring: int
    full_cap: int
    sl_theta: float
    full_theta: float
    sl_rot_pairs: int
    full_rot_pairs: int
    sl_scale: float
    full_scale: float
    eps: float
    softcap: float
    embed: np.ndarray        # uint16 [vocab, hidden]
    final_norm: np.ndarray   # float32 [hidden]
    layers: list = field(default_factory=list)
    weight_format: int = 0   # 0: layer matrices are q4_0 blocks, 1: int8 (q8) blocks
    kv_format: int = 0       # 0: full layers cache K and V; 1: only the V row (key rebuilt)

    def _struct(self):
        arr = (_Layer * len(self.layers))()
        keep = []
        for i, L in enumerate(self.layers):
            def P(a):
                if a is None:
                    return None
                a = np.ascontiguousarray(a)
                keep.append(a)
                return a.ctypes.data
            for nm in ("k_cache", "v_cache"):
                c = getattr(L, nm)
                assert c is None or (c.flags["C_CONTIGUOUS"] and c.dtype == np.uint16)
            assert L.v_cache is not None and (L.k_cache is not None or (L.is_full and self.kv_format == 1))
            arr[i] = _Layer(int(L.is_full), int(L.v_norm),
                            P(L.wq), P(L.wk), P(L.wv), P(L.wo), P(L.wg), P(L.wu), P(L.wd),
                            P(L.attn_norm), P(L.q_norm), P(L.k_norm), P(L.post_attn_norm),
                            P(L.pre_ff_norm), P(L.post_ff_norm), float(L.layer_scalar),
                            None if L.k_cache is None else L.k_cache.ctypes.data, L.v_cache.ctypes.data)
        keep.append(arr)
        emb = np.ascontiguousarray(self.embed, dtype=np.uint16)
        fn = np.ascontiguousarray(self.final_norm, dtype=np.float32)
        keep += [emb, fn]
        m = _Model(self.hidden, self.n_heads, self.inter, self.vocab, len(self.layers),
                   self.sl_kv_heads, self.sl_head_dim, self.full_head_dim,
                   self.window, self.ring, self.full_cap,
                   self.sl_theta, self.full_theta, self.sl_rot_pairs, self.full_rot_pairs,
                   self.sl_scale, self.full_scale, self.eps, self.softcap,
                   emb.ctypes.data, fn.ctypes.data, arr, int(self.weight_format), int(self.kv_format))
        return m, keep

    def embed_tokens(self, tokens) -> np.ndarray:
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        m, keep = self._struct()
        h = np.empty((tokens.size, self.hidden), dtype=np.float64)
        if lib().orc_embed(C.byref(m), _ptr(tokens), tokens.size, _ptr(h)) != 0:
            raise ValueError("oracle embed rejected its arguments")
        return h

    def run_layer(self, l: int, h, pos0: int) -> np.ndarray:
        """Layer l applied to a copy of h [n, hidden] (writes layer l's cache)."""
        h = np.array(h, dtype=np.float64, copy=True, order="C")
        m, keep = self._struct()
        if lib().orc_run_layer(C.byref(m), l, _ptr(h), h.shape[0], pos0) != 0:
            raise ValueError("oracle layer rejected its arguments")
        return h

    def run_head(self, h, want_logits: bool = True):
        h = np.ascontiguousarray(h, dtype=np.float64)
        n = h.shape[0]
        m, keep = self._struct()
        logits = np.empty((n, self.vocab), dtype=np.float64) if want_logits else None
        am = np.empty(n, dtype=np.int32)
        if lib().orc_head(C.byref(m), _ptr(h), n, _ptr(logits) if logits is not None else None, _ptr(am)) != 0:
            raise ValueError("oracle head rejected its arguments")
        return logits, am

    # ---- the layer's stages and the head's two (orc_run_layer and
    # orc_head compose them); each takes the previous stage's storage values,
    # so a stage can be fed another implementation's rounding points
    def _dims(self, l: int):
        L = self.layers[l]
        D = self.full_head_dim if L.is_full else self.sl_head_dim
        Hkv = 1 if L.is_full else self.sl_kv_heads
        return D, Hkv

    def stage_attn_in(self, l: int, h):
        """-> x16 = fp16(RMSNorm(h, attn_norm)) uint16 [n, hidden]"""
        h = np.ascontiguousarray(np.atleast_2d(h), dtype=np.float64)
        x16 = np.empty((h.shape[0], self.hidden), dtype=np.uint16)
        m, keep = self._struct()
        if lib().orc_stage_attn_in(C.byref(m), l, _ptr(h), h.shape[0], _ptr(x16)) != 0:
            raise ValueError("oracle stage_attn_in rejected its arguments")
        return x16

    def stage_qkv(self, l: int, x16):
        """-> (q [n, Hq*D], k [n, Hkv*D], v [n, Hkv*D]) projections of x16"""
        x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
        n = x16.shape[0]
        D, Hkv = self._dims(l)
        q = np.empty((n, self.n_heads * D)); k = np.empty((n, Hkv * D)); v = np.empty((n, Hkv * D))
        m, keep = self._struct()
        if lib().orc_stage_qkv(C.byref(m), l, _ptr(x16), n, _ptr(q), _ptr(k), _ptr(v)) != 0:
            raise ValueError("oracle stage_qkv rejected its arguments")
        return q, k, v

    def stage_finish(self, l: int, q, k, v, pos0: int):
        """Writes the rows' K/V into layer l's cache; -> q16 uint16 [n, Hq, D]."""
        q = np.ascontiguousarray(np.atleast_2d(q), dtype=np.float64)
        k = np.ascontiguousarray(np.atleast_2d(k), dtype=np.float64)
        v = np.ascontiguousarray(np.atleast_2d(v), dtype=np.float64)
        n = q.shape[0]
        D, _ = self._dims(l)
        q16 = np.empty((n, self.n_heads, D), dtype=np.uint16)
        m, keep = self._struct()
        if lib().orc_stage_finish(C.byref(m), l, _ptr(q), _ptr(k), _ptr(v), n, pos0, _ptr(q16)) != 0:
            raise ValueError("oracle stage_finish rejected its arguments")
        return q16

    def stage_attend(self, l: int, q16, pos0: int):
        """-> att float64 [n, Hq, D] over layer l's cache."""
        q16 = np.ascontiguousarray(q16, dtype=np.uint16)
        D, _ = self._dims(l)
        q16 = q16.reshape(-1, self.n_heads, D)
        n = q16.shape[0]
        att = np.empty((n, self.n_heads, D))
        m, keep = self._struct()
        if lib().orc_stage_attend(C.byref(m), l, _ptr(q16), n, pos0, _ptr(att)) != 0:
            raise ValueError("oracle stage_attend rejected its arguments")
        return att

    def stage_oproj(self, l: int, o16, h):
        """-> h + RMSNorm(Wo o16, post_attn_norm)"""
        D, _ = self._dims(l)
        o16 = np.ascontiguousarray(o16, dtype=np.uint16).reshape(-1, self.n_heads * D)
        h = np.array(np.atleast_2d(h), dtype=np.float64, copy=True, order="C")
        m, keep = self._struct()
        if lib().orc_stage_oproj(C.byref(m), l, _ptr(o16), h.shape[0], _ptr(h)) != 0:
            raise ValueError("oracle stage_oproj rejected its arguments")
        return h

    def stage_mlp_in(self, l: int, h):
        """-> x16 = fp16(RMSNorm(h, pre_ff_norm)) uint16 [n, hidden]"""
        h = np.ascontiguousarray(np.atleast_2d(h), dtype=np.float64)
        x16 = np.empty((h.shape[0], self.hidden), dtype=np.uint16)
        m, keep = self._struct()
        if lib().orc_stage_mlp_in(C.byref(m), l, _ptr(h), h.shape[0], _ptr(x16)) != 0:
            raise ValueError("oracle stage_mlp_in rejected its arguments")
        return x16

    def stage_gateup(self, l: int, x16):
        """-> a16 = fp16(gelu_tanh(Wg x16) * Wu x16) uint16 [n, inter]"""
        x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
        n = x16.shape[0]
        a16 = np.empty((n, self.inter), dtype=np.uint16)
        m, keep = self._struct()
        if lib().orc_stage_gateup(C.byref(m), l, _ptr(x16), n, _ptr(a16)) != 0:
            raise ValueError("oracle stage_gateup rejected its arguments")
        return a16

    def stage_down(self, l: int, a16, h):
        """-> (h + RMSNorm(Wd a16, post_ff_norm)) * layer_scalar"""
        a16 = np.ascontiguousarray(a16, dtype=np.uint16).reshape(-1, self.inter)
        h = np.array(np.atleast_2d(h), dtype=np.float64, copy=True, order="C")
        m, keep = self._struct()
        if lib().orc_stage_down(C.byref(m), l, _ptr(a16), h.shape[0], _ptr(h)) != 0:
            raise ValueError("oracle stage_down rejected its arguments")
        return h

    def head_input(self, h):
        """-> x16 = fp16(RMSNorm(h, final_norm)) uint16 [n, hidden]"""
        h = np.ascontiguousarray(np.atleast_2d(h), dtype=np.float64)
        x16 = np.empty((h.shape[0], self.hidden), dtype=np.uint16)
        m, keep = self._struct()
        if lib().orc_head_input(C.byref(m), _ptr(h), h.shape[0], _ptr(x16)) != 0:
            raise ValueError("oracle head_input rejected its arguments")
        return x16

    def head_logits(self, x16, want_logits: bool = True):
        """-> (softcapped logits float64 [n, vocab] or None, argmax int32 [n])"""
        x16 = np.ascontiguousarray(np.atleast_2d(x16), dtype=np.uint16)
        n = x16.shape[0]
        logits = np.empty((n, self.vocab), dtype=np.float64) if want_logits else None
        am = np.empty(n, dtype=np.int32)
        m, keep = self._struct()
        if lib().orc_head_logits(C.byref(m), _ptr(x16), n, _ptr(logits) if logits is not None else None,
                                 _ptr(am)) != 0:
            raise ValueError("oracle head_logits rejected its arguments")
        return logits, am

    def decode_step(self, tokens, pos0: int, want_logits: bool = True):
        """Run len(tokens) rows at positions pos0.. (writes the caches).

        Returns (logits float64 [n, vocab] or None, argmax int32 [n])."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        n = tokens.size
        m, keep = self._struct()
        logits = np.empty((n, self.vocab), dtype=np.float64) if want_logits else None
        am = np.empty(n, dtype=np.int32)
        rc = lib().orc_decode_step(C.byref(m), _ptr(tokens), n, pos0,
                                   _ptr(logits) if logits is not None else None, _ptr(am))
        del keep
        if rc != 0:
            raise ValueError("oracle decode_step rejected its arguments")
        return logits, am
