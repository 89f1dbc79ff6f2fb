"""int4_q4_gemv_amd -- MI355X (gfx950) int4 q4_0 decode step.

Thin Python binding over the C ABI in ``include/q4dec.h`` (``libq4dec.so``,
built from ``csrc/`` by :func:`build`).  Every step of the path runs in the
library's HIP kernels; this module only marshals torch tensors (device memory)
and the current HIP stream into the C calls.  There is no fallback: without
the built library every entry point raises.
"""
from __future__ import annotations

import ctypes as C
import glob
import hashlib
import math
import os
import subprocess
import sys

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libq4dec.so")
SRC = os.path.join(_HERE, "csrc", "q4dec.hip")

HIPCC_FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-shared", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fhip-fp32-correctly-rounded-divide-sqrt"]

Q4_OK, Q4_EINVAL, Q4_ESHAPE, Q4_EALIGN, Q4_ERANGE, Q4_ENOSPACE, Q4_EHIP = 0, -1, -2, -3, -4, -5, -6
Q4_F32, Q4_BF16 = 0, 1


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the library's sources (csrc/
    and include/q4dec.h, in name order): compiled into the library and
    reported by q4dec_version()."""
    files = sorted(glob.glob(os.path.join(_HERE, "csrc", "*.h")) + glob.glob(os.path.join(_HERE, "csrc", "*.hip")))
    files.append(os.path.join(_ROOT, "include", "q4dec.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    """Compile csrc/ for gfx950 into libq4dec.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f'-DQ4DEC_SRC_HASH="{source_hash()}"', "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib_raw().q4dec_status_str(status).decode()}")


_lib = None


def _lib_raw():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run int4_q4_gemv_amd.build() "
                               "(or __graft_entry__.build()) first")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        built = L.q4dec_version().decode().rsplit(" ", 1)[-1]
        if built != source_hash():
            raise RuntimeError(f"{LIB_PATH} was built from other sources (library {built}, tree "
                               f"{source_hash()}); rebuild it with int4_q4_gemv_amd.build()")
        _lib = L
    return _lib


lib = _lib_raw

_p, _i, _sz, _i64, _f = C.c_void_p, C.c_int, C.c_size_t, C.c_int64, C.c_float


class Layer(C.Structure):
    _fields_ = [("is_full", C.c_int32), ("v_norm", C.c_int32),
                ("wq", _p), ("wk", _p), ("wv", _p), ("wo", _p), ("wg", _p), ("wu", _p), ("wd", _p),
                ("attn_norm", _p), ("q_norm", _p), ("k_norm", _p), ("post_attn_norm", _p),
                ("pre_ff_norm", _p), ("post_ff_norm", _p), ("layer_scalar", C.c_float),
                ("k_cache", _p), ("v_cache", _p)]


class Model(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("inter", C.c_int32),
                ("vocab", C.c_int32), ("n_layers", C.c_int32),
                ("sl_kv_heads", C.c_int32), ("sl_head_dim", C.c_int32), ("full_head_dim", C.c_int32),
                ("window", C.c_int32), ("ring", C.c_int32), ("full_cap", C.c_int32),
                ("sl_rot_pairs", C.c_int32), ("full_rot_pairs", C.c_int32),
                ("sl_theta", C.c_double), ("full_theta", C.c_double),
                ("sl_scale", C.c_float), ("full_scale", C.c_float), ("eps", C.c_float),
                ("softcap", C.c_float), ("embed", _p), ("final_norm", _p), ("layers", C.POINTER(Layer)),
                ("weight_format", C.c_int32), ("kv_format", C.c_int32)]


def _declare(L):
    L.q4dec_status_str.restype = C.c_char_p
    L.q4dec_status_str.argtypes = [_i]
    L.q4dec_version.restype = C.c_char_p
    L.q4_packed_bytes.restype = _sz
    L.q4_packed_bytes.argtypes = [_i, _i]
    L.q4_pack.restype = _i
    L.q4_pack.argtypes = [_p, _i, _i, _i, _p, _sz, _p, _p]
    L.q4_unpack.restype = _i
    L.q4_unpack.argtypes = [_p, _i, _i, _p, _p]
    L.q4_gemv.restype = _i
    L.q4_gemv.argtypes = [_p, _i, _i, _p, _i, _p, _p]
    L.q8_packed_bytes.restype = _sz
    L.q8_packed_bytes.argtypes = [_i, _i]
    L.q8_pack.restype = _i
    L.q8_pack.argtypes = [_p, _i, _i, _i, _p, _sz, _p, _p]
    L.q8_unpack.restype = _i
    L.q8_unpack.argtypes = [_p, _i, _i, _p, _p]
    L.q8_gemv.restype = _i
    L.q8_gemv.argtypes = [_p, _i, _i, _p, _i, _p, _p]
    L.flash_decode_workspace_size.restype = _sz
    L.flash_decode_workspace_size.argtypes = [_i, _i, _i, _i]
    L.flash_decode_full.restype = _i
    L.flash_decode_full.argtypes = [_p, _p, _p, _i64, _i, _i, _i, _p, _i, _i, _f, _p, _p, _sz, _p]
    L.flash_decode_noalloc_max_bytes.restype = _sz
    L.flash_decode_noalloc_max_bytes.argtypes = []
    L.flash_decode_full_noalloc.restype = _i
    L.flash_decode_full_noalloc.argtypes = [_p, _p, _p, _i64, _i, _i, _i, _p, _i, _i, _f, _p, _p]
    L.flash_decode_full_vrow.restype = _i
    L.flash_decode_full_vrow.argtypes = [_p, _p, _i64, _i, _i, _i, _p, C.c_double, _i, _p, _i, _i, _f, _p,
                                         _p, _sz, _p]
    L.flash_decode_ring.restype = _i
    L.flash_decode_ring.argtypes = [_p, _p, _p, _i64, _i, _i, _i, _i, _i, _p, _i, _i, _f, _p, _p, _sz, _p]
    L.decode_step_workspace_size.restype = _sz
    L.decode_step_workspace_size.argtypes = [C.POINTER(Model), _i]
    for fn in (L.decode_step, L.decode_step_eager):
        fn.restype = _i
        fn.argtypes = [C.POINTER(Model), _p, _i, _i, _p, _p, _p, _sz, _p]
    L.q4dec_release.restype = _i
    L.decode_step_gemvs.restype = _i
    L.decode_step_gemvs.argtypes = [C.POINTER(Model), _i, _p, _sz, _p]
    L.q4dec_graph_count.restype = _i
    L.q4dec_graph_count.argtypes = []
    L.decode_step_stage_bytes.restype = _sz
    L.decode_step_stage_bytes.argtypes = [C.POINTER(Model), _i, _i]
    L.decode_step_stage.restype = _i
    L.decode_step_stage.argtypes = [C.POINTER(Model), _p, _sz, _i, _i, _p, _sz, _p]
    L.decode_step_hidden.restype = _i
    L.decode_step_hidden.argtypes = [C.POINTER(Model), _p, _sz, _i, _p, _p]
    L.q4_gemm.restype = _i
    L.q4_gemm.argtypes = [_p, _i, _i, _p, _i, _p, _p]
    L.prefill_chunk_workspace_size.restype = _sz
    L.prefill_chunk_workspace_size.argtypes = [C.POINTER(Model)]
    L.prefill_chunk.restype = _i
    L.prefill_chunk.argtypes = [C.POINTER(Model), _p, _i, _i, _p, _p, _p, _p, _sz, _p]
    L.q4_spec_accept.restype = _i
    L.q4_spec_accept.argtypes = [_p, _p, _i, _p, _p]
    L.q4_stream_read_sink_words.restype = _i
    L.q4_stream_read_sink_words.argtypes = []
    L.q4_stream_read.restype = _i
    L.q4_stream_read.argtypes = [_p, _sz, _p, _p]


EXPORTS = ["q4dec_status_str", "q4dec_version", "q4_packed_bytes", "q4_pack", "q4_unpack",
           "q4_gemv", "q8_packed_bytes", "q8_pack", "q8_unpack", "q8_gemv", "flash_decode_workspace_size", "flash_decode_full",
           "flash_decode_full_vrow", "flash_decode_ring", "flash_decode_noalloc_max_bytes",
           "flash_decode_full_noalloc",
           "decode_step_workspace_size", "decode_step", "decode_step_hidden", "decode_step_eager",
           "decode_step_stage_bytes", "decode_step_stage", "q4dec_graph_count", "decode_step_gemvs",
           "q4_gemm", "prefill_chunk_workspace_size", "prefill_chunk",
           "q4_spec_accept", "q4_stream_read_sink_words", "q4_stream_read", "q4dec_release"]


def _check(fn: str, rc: int):
    if rc != Q4_OK:
        raise Q4Error(fn, rc)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors passed to the HIP library must live on the GPU")


# ------------------------------------------------------------------ q4_0 ----
def packed_bytes(N: int, K: int) -> int:
    return int(lib().q4_packed_bytes(N, K))


def q4_pack(w: torch.Tensor, nonfinite: torch.Tensor | None = None) -> torch.Tensor:
    """Quantise fp32/bf16 [N, K] (device) to the packed q4_0 layout (uint8)."""
    _need_cuda(w)
    w = w.contiguous()
    N, K = w.shape
    dt = {torch.float32: Q4_F32, torch.bfloat16: Q4_BF16}.get(w.dtype)
    if dt is None:
        raise ValueError("q4_pack takes fp32 or bf16 weights")
    nbytes = packed_bytes(N, K)
    if nbytes == 0:
        raise Q4Error("q4_pack", Q4_ESHAPE)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check("q4_pack", lib().q4_pack(_ptr(w), dt, N, K, _ptr(out), nbytes, _ptr(nonfinite), _stream()))
    return out


def q4_unpack(packed: torch.Tensor, N: int, K: int) -> torch.Tensor:
    """Canonical q4_0 blocks [N, K/32, 18] (uint8) of a packed matrix."""
    out = torch.empty((N, K // 32, 18), dtype=torch.uint8, device=packed.device)
    _check("q4_unpack", lib().q4_unpack(_ptr(packed), N, K, _ptr(out), _stream()))
    return out


class Gemv:
    """q4_gemv for one matrix shape (kept for call sites that reuse it)."""

    def __init__(self, N: int, K: int, B: int, device="cuda"):
        self.N, self.K, self.B = N, K, B

    def __call__(self, packed, x, y=None):
        _need_cuda(packed, x)
        x = x.contiguous()
        B = x.shape[0]
        if y is None:
            y = torch.empty((B, self.N), dtype=torch.float32, device=x.device)
        _check("q4_gemv", lib().q4_gemv(_ptr(packed), self.N, self.K, _ptr(x), B, _ptr(y), _stream()))
        return y


def q4_gemv(packed, N: int, K: int, x: torch.Tensor) -> torch.Tensor:
    """y[b, n] = sum_k W[n, k] x[b, k] for fp16 x [B, K]; fp32 y [B, N]."""
    x2 = x.reshape(-1, K)
    return Gemv(N, K, x2.shape[0], device=x.device)(packed, x2)


def q4_gemm(packed, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """The prefill product: y[b, n] = sum_k W[n, k] x[b, k] for fp16 x [n <= 64, K]
    on MFMA; fp32 y [n, N]."""
    _need_cuda(packed, x)
    x = x.reshape(-1, K).contiguous()
    n = x.shape[0]
    if y is None:
        y = torch.empty((n, N), dtype=torch.float32, device=x.device)
    _check("q4_gemm", lib().q4_gemm(_ptr(packed), N, K, _ptr(x), n, _ptr(y), _stream()))
    return y


# ----------------------------------------------------------- q8 int8lin ----
def q8_packed_bytes(N: int, K: int) -> int:
    return int(lib().q8_packed_bytes(N, K))


def q8_pack(w: torch.Tensor, nonfinite: torch.Tensor | None = None) -> torch.Tensor:
    """Quantise fp32/bf16 [N, K] (device) to the packed int8 layout (uint8)."""
    _need_cuda(w)
    w = w.contiguous()
    N, K = w.shape
    dt = {torch.float32: Q4_F32, torch.bfloat16: Q4_BF16}.get(w.dtype)
    if dt is None:
        raise ValueError("q8_pack takes fp32 or bf16 weights")
    nbytes = q8_packed_bytes(N, K)
    if nbytes == 0:
        raise Q4Error("q8_pack", Q4_ESHAPE)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check("q8_pack", lib().q8_pack(_ptr(w), dt, N, K, _ptr(out), nbytes, _ptr(nonfinite), _stream()))
    return out


def q8_unpack(packed: torch.Tensor, N: int, K: int) -> torch.Tensor:
    """Canonical int8 blocks [N, K/32, 34] (uint8) of a packed matrix."""
    out = torch.empty((N, K // 32, 34), dtype=torch.uint8, device=packed.device)
    _check("q8_unpack", lib().q8_unpack(_ptr(packed), N, K, _ptr(out), _stream()))
    return out


def q8_gemv(packed, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[b, n] = sum_k W[n, k] x[b, k] for int8 weights and fp16 x [B, K]; fp32 y [B, N]."""
    _need_cuda(packed, x)
    x2 = x.reshape(-1, K).contiguous()
    B = x2.shape[0]
    if y is None:
        y = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _check("q8_gemv", lib().q8_gemv(_ptr(packed), N, K, _ptr(x2), B, _ptr(y), _stream()))
    return y


# ------------------------------------------------------------- attention ----
def _fd_ws(n_seq, n_rows, Hq, D, device):
    n = int(lib().flash_decode_workspace_size(n_seq, n_rows, Hq, D))
    if n == 0:
        raise Q4Error("flash_decode_workspace_size", Q4_ESHAPE)
    return torch.empty(n, dtype=torch.uint8, device=device)


def flash_decode_full(q, k, v, pos0, scale: float = 1.0, ws=None):
    """q fp16 [n_seq, n_rows, Hq, D]; k, v fp16 [n_seq, cap, D] (or [cap, D]);
    pos0 list/int per sequence.  Returns fp32 [n_seq, n_rows, Hq, D]."""
    _need_cuda(q, k, v)
    if k.dim() == 2:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    if q.dim() == 3:
        q = q.unsqueeze(0)
    n_seq, n_rows, Hq, D = q.shape
    cap = k.shape[1]
    pos = (C.c_int32 * n_seq)(*([int(pos0)] * n_seq if isinstance(pos0, int) else [int(p) for p in pos0]))
    out = torch.empty((n_seq, n_rows, Hq, D), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else _fd_ws(n_seq, n_rows, Hq, D, q.device)
    _check("flash_decode_full", lib().flash_decode_full(
        _ptr(q.contiguous()), _ptr(k), _ptr(v), k.stride(0), cap, Hq, D, pos, n_seq, n_rows,
        float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def flash_decode_full_noalloc(q, k, v, pos0, scale: float = 1.0, out=None):
    """flash_decode_full with the library's static scratch instead of a
    workspace (no allocation inside the call; ``out`` may be given so that
    none happens here either).  Calls overlapping on one GPU race."""
    _need_cuda(q, k, v)
    if k.dim() == 2:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    if q.dim() == 3:
        q = q.unsqueeze(0)
    n_seq, n_rows, Hq, D = q.shape
    cap = k.shape[1]
    pos = (C.c_int32 * n_seq)(*([int(pos0)] * n_seq if isinstance(pos0, int) else [int(p) for p in pos0]))
    if out is None:
        out = torch.empty((n_seq, n_rows, Hq, D), dtype=torch.float32, device=q.device)
    _check("flash_decode_full_noalloc", lib().flash_decode_full_noalloc(
        _ptr(q.contiguous()), _ptr(k), _ptr(v), k.stride(0), cap, Hq, D, pos, n_seq, n_rows,
        float(scale), _ptr(out), _stream()))
    return out


def flash_decode_full_vrow(q, vrow, kw, theta: float, rot_pairs: int, pos0, scale: float = 1.0, ws=None):
    """Full layer caching one row per position: q fp16 [n_seq, n_rows, Hq, D];
    vrow fp16 [n_seq, cap, D] (or [cap, D]), the V rows; kw fp32 [D], the
    k_norm multiplier; the key of row t is RoPE_t(kw * v_t).  D in {128, 512}."""
    _need_cuda(q, vrow, kw)
    if vrow.dim() == 2:
        vrow = vrow.unsqueeze(0)
    if q.dim() == 3:
        q = q.unsqueeze(0)
    n_seq, n_rows, Hq, D = q.shape
    cap = vrow.shape[1]
    pos = (C.c_int32 * n_seq)(*([int(pos0)] * n_seq if isinstance(pos0, int) else [int(p) for p in pos0]))
    out = torch.empty((n_seq, n_rows, Hq, D), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else _fd_ws(n_seq, n_rows, Hq, D, q.device)
    kw = kw.contiguous()
    _check("flash_decode_full_vrow", lib().flash_decode_full_vrow(
        _ptr(q.contiguous()), _ptr(vrow), vrow.stride(0), cap, Hq, D, _ptr(kw), float(theta), int(rot_pairs),
        pos, n_seq, n_rows, float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def flash_decode_ring(q, k, v, W: int, pos0, scale: float = 1.0, ws=None):
    """q fp16 [n_seq, n_rows, Hq, D]; k, v fp16 [n_seq, Hkv, R, D] (or [Hkv, R, D])."""
    _need_cuda(q, k, v)
    if k.dim() == 3:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    if q.dim() == 3:
        q = q.unsqueeze(0)
    n_seq, n_rows, Hq, D = q.shape
    Hkv, R = k.shape[1], k.shape[2]
    pos = (C.c_int32 * n_seq)(*([int(pos0)] * n_seq if isinstance(pos0, int) else [int(p) for p in pos0]))
    out = torch.empty((n_seq, n_rows, Hq, D), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else _fd_ws(n_seq, n_rows, Hq, D, q.device)
    _check("flash_decode_ring", lib().flash_decode_ring(
        _ptr(q.contiguous()), _ptr(k), _ptr(v), k.stride(0), Hq, Hkv, D, R, W, pos, n_seq, n_rows,
        float(scale), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


# ----------------------------------------------------------- decode step ----
class DecodeModel:
    """Device-resident model for :meth:`step`: packed weights, fp32 norms,
    fp16 tied table and fp16 KV caches, all torch CUDA tensors kept alive
    here, plus the ctypes descriptor the library reads."""

    def __init__(self, cfg, layers, embed, final_norm, weight_format: int = 0, kv_format: int = 0):
        self.cfg = cfg
        self.weight_format = weight_format   # 0: q4_0 packs, 1: int8 packs
        self.kv_format = kv_format           # 0: full layers cache K and V, 1: only the V row
        self.layers = layers          # list of dicts of device tensors
        self.embed = embed
        self.final_norm = final_norm
        arr = (Layer * len(layers))()
        for i, L in enumerate(layers):
            arr[i] = Layer(int(L["is_full"]), int(L["v_norm"]),
                           L["wq"].data_ptr(), L["wk"].data_ptr(),
                           L["wv"].data_ptr() if L.get("wv") is not None else None,
                           L["wo"].data_ptr(), L["wg"].data_ptr(), L["wu"].data_ptr(), L["wd"].data_ptr(),
                           L["attn_norm"].data_ptr(), L["q_norm"].data_ptr(), L["k_norm"].data_ptr(),
                           L["post_attn_norm"].data_ptr(), L["pre_ff_norm"].data_ptr(),
                           L["post_ff_norm"].data_ptr(), float(L["layer_scalar"]),
                           L["k_cache"].data_ptr() if L.get("k_cache") is not None else None,
                           L["v_cache"].data_ptr())
        self._arr = arr
        c = cfg
        self.desc = Model(c.hidden, c.n_heads, c.inter, c.vocab, len(layers),
                          c.sl_kv_heads, c.sl_head_dim, c.full_head_dim,
                          c.window, c.ring, c.full_cap, c.sl_rot_pairs, c.full_rot_pairs,
                          c.sl_theta, c.full_theta, c.sl_scale, c.full_scale, c.eps, c.softcap,
                          embed.data_ptr(), final_norm.data_ptr(), arr, int(weight_format), int(kv_format))
        self._ws = {}
        self._argmax = {}

    def workspace(self, n: int):
        if n not in self._ws:
            nb = int(lib().decode_step_workspace_size(C.byref(self.desc), n))
            if nb == 0:
                raise Q4Error("decode_step_workspace_size", Q4_ESHAPE)
            self._ws[n] = torch.zeros(nb, dtype=torch.uint8, device=self.embed.device)
        return self._ws[n]

    def step(self, tokens, pos0: int, logits: torch.Tensor | None = None,
             argmax: torch.Tensor | None = None, graph: bool = True, want_logits: bool = True):
        """One decode step of len(tokens) rows at positions pos0 ..; returns
        (logits [n, vocab] or None, argmax [n]).  Without an ``argmax`` the
        model's own buffer for n rows is used and returned: the next step of
        the same width overwrites it (clone it to keep it).  Fresh ``logits``
        are allocated unless given."""
        toks = [int(t) for t in tokens]
        n = len(toks)
        dev = self.embed.device
        if logits is None and want_logits:
            logits = torch.empty((n, self.cfg.vocab), dtype=torch.float32, device=dev)
        if argmax is None:
            if n not in self._argmax:
                self._argmax[n] = torch.zeros(n, dtype=torch.int32, device=dev)
            argmax = self._argmax[n]
        ws = self.workspace(n)
        tk = (C.c_int32 * n)(*toks)
        fn = lib().decode_step if graph else lib().decode_step_eager
        _check("decode_step", fn(C.byref(self.desc), tk, n, int(pos0), _ptr(logits), _ptr(argmax),
                                 _ptr(ws), ws.numel(), _stream()))
        return logits, argmax


def _prefill(self, tokens, pos0: int, logits: torch.Tensor | None = None, argmax: torch.Tensor | None = None,
             want_logits: bool = True, want_hidden: bool = False):
    """One prefill chunk of len(tokens) <= 64 rows at positions pos0 ..:
    returns (logits of the last row [vocab] or None, argmax [1], residual
    stream of every row [n, hidden] or None)."""
    toks = [int(t) for t in tokens]
    n = len(toks)
    dev = self.embed.device
    if logits is None and want_logits:
        logits = torch.empty(self.cfg.vocab, dtype=torch.float32, device=dev)
    if argmax is None:
        argmax = torch.empty(1, dtype=torch.int32, device=dev)
    h = torch.empty((n, self.cfg.hidden), dtype=torch.float32, device=dev) if want_hidden else None
    if getattr(self, "_chunk_ws", None) is None:
        nb = int(lib().prefill_chunk_workspace_size(C.byref(self.desc)))
        if nb == 0:
            raise Q4Error("prefill_chunk_workspace_size", Q4_ESHAPE)
        self._chunk_ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    ws = self._chunk_ws
    tk = (C.c_int32 * n)(*toks)
    _check("prefill_chunk", lib().prefill_chunk(C.byref(self.desc), tk, n, int(pos0), _ptr(logits), _ptr(argmax),
                                                _ptr(h), _ptr(ws), ws.numel(), _stream()))
    return logits, argmax, h


DecodeModel.prefill = _prefill


def _hidden(self, n: int) -> torch.Tensor:
    ws = self.workspace(n)
    out = torch.empty((n, self.cfg.hidden), dtype=torch.float32, device=self.embed.device)
    _check("decode_step_hidden", lib().decode_step_hidden(C.byref(self.desc), _ptr(ws), ws.numel(), n,
                                                          _ptr(out), _stream()))
    return out


DecodeModel.hidden = _hidden

STAGE_H_OUT, STAGE_H_MID, STAGE_X_ATTN, STAGE_QKV, STAGE_Q16, STAGE_O16, STAGE_X_MLP, STAGE_A16, STAGE_X_HEAD = range(9)
_STAGE_DTYPE = {STAGE_H_OUT: torch.float32, STAGE_H_MID: torch.float32, STAGE_QKV: torch.float32}


def _stage(self, n: int, stage: int) -> torch.Tensor:
    """A stage of the last layer of the most recent step of width n
    (decode_step_stage): [n, ...] fp32 or fp16 as the header lists."""
    ws = self.workspace(n)
    nb = int(lib().decode_step_stage_bytes(C.byref(self.desc), n, stage))
    if nb == 0:
        raise Q4Error("decode_step_stage_bytes", Q4_EINVAL)
    dt = _STAGE_DTYPE.get(stage, torch.float16)
    out = torch.empty(nb // (4 if dt == torch.float32 else 2), dtype=dt, device=self.embed.device)
    _check("decode_step_stage", lib().decode_step_stage(C.byref(self.desc), _ptr(ws), ws.numel(), n, stage,
                                                        _ptr(out), nb, _stream()))
    return out.view(n, -1)


DecodeModel.stage = _stage


def _step_gemvs(self, n: int = 1):
    """decode_step_gemvs: the step's q/k/v, output and down products only
    (measurement of that kernel in its step launch configuration)."""
    ws = self.workspace(n)
    _check("decode_step_gemvs", lib().decode_step_gemvs(C.byref(self.desc), n, _ptr(ws), ws.numel(), _stream()))


DecodeModel.step_gemvs = _step_gemvs


def graph_count() -> int:
    """Captured decode-step graphs the library holds."""
    return int(lib().q4dec_graph_count())


def release():
    _check("q4dec_release", lib().q4dec_release())


# ------------------------------------------------------ speculative verify ----
def spec_accept(block, argmax) -> list[int]:
    """q4_spec_accept on host lists: the tokens a verify block emits."""
    n = len(block)
    if len(argmax) != n:
        raise ValueError("block and argmax need the same length")
    b = (C.c_int32 * n)(*[int(t) for t in block])
    a = (C.c_int32 * n)(*[int(t) for t in argmax])
    e = (C.c_int32 * n)()
    ne = C.c_int(0)
    _check("q4_spec_accept", lib().q4_spec_accept(b, a, n, e, C.byref(ne)))
    return [int(e[i]) for i in range(ne.value)]


def speculative_greedy(model: DecodeModel, token0: int, pos0: int, n_new: int, drafter, width: int = 4):
    """Greedy decoding with single-pass speculative verify blocks of `width`
    rows: each block feeds the last emitted token and width - 1 drafts
    (drafter(pos, token, k) -> k proposed tokens for positions pos+1..pos+k)
    to decode_step at `pos`, and q4_spec_accept picks the emitted tokens.
    Returns (the first n_new emitted tokens, the number of blocks run)."""
    dev = model.embed.device
    am = torch.empty(width, dtype=torch.int32, device=dev)
    out: list[int] = []
    tok, pos, blocks = int(token0), int(pos0), 0
    while len(out) < n_new:
        drafts = [int(t) for t in drafter(pos, tok, width - 1)]
        if len(drafts) != width - 1:
            raise ValueError("the drafter must propose width - 1 tokens")
        block = [tok] + drafts
        model.step(block, pos, argmax=am, want_logits=False)
        emitted = spec_accept(block, am.cpu().tolist())
        out.extend(emitted)
        pos += len(emitted)
        tok = emitted[-1]
        blocks += 1
    return out[:n_new], blocks


# ------------------------------------------------------------ measurement ----
def stream_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """q4_stream_read over a contiguous device tensor; returns the uint32
    sink (its XOR is the XOR of every 32-bit word of src)."""
    _need_cuda(src)
    if not src.is_contiguous():
        raise ValueError("stream_read needs a contiguous tensor")
    if sink is None:
        sink = torch.empty(int(lib().q4_stream_read_sink_words()), dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check("q4_stream_read", lib().q4_stream_read(_ptr(src), nbytes, _ptr(sink), _stream()))
    return sink


def build_decode_model(cfg, seed: int, ctx: int, device="cuda", pack_check=None, gen_device=None,
                       weights: str = "q4", kv: str = "pair"):
    """Draws the synthetic model of ``synth`` on the GPU, packs every matrix
    with q4_pack (``weights="q4"``) or q8_pack (``"q8"``) and prefills the
    caches for a decode at position ``ctx``.  ``kv="vrow"`` keeps only the V
    row of the full layers (no K cache is allocated for them).
    ``pack_check(name, l, w_fp32_device, packed)`` is called per matrix when
    given (the tests use it to compare against the oracle)."""
    if weights not in ("q4", "q8"):
        raise ValueError("weights is 'q4' or 'q8'")
    if kv not in ("pair", "vrow"):
        raise ValueError("kv is 'pair' or 'vrow'")
    pack = q4_pack if weights == "q4" else q8_pack
    from . import synth
    gd = gen_device or device
    layers = []
    for l in range(cfg.n_layers):
        if cfg.n_layers > 8 and l % 8 == 0:
            print(f"  building layer {l}/{cfg.n_layers}", file=sys.stderr, flush=True)
        lp = synth.layer_params(cfg, l, seed, device=gd)
        L = {"is_full": cfg.is_full(l), "v_norm": cfg.is_full(l) or cfg.sl_v_norm,
             "layer_scalar": lp.layer_scalar}
        for name, w in lp.mats.items():
            wd = w.to(device)
            L[name] = pack(wd)
            if pack_check is not None:
                pack_check(name, l, wd, L[name])
            del wd
        lp.mats.clear()
        for name, t in lp.norms.items():
            L[name] = t.to(device).contiguous()
        k, v = synth.layer_cache(cfg, l, seed, ctx, device=gd)
        if kv == "vrow" and L["is_full"]:
            L["k_cache"], L["v_cache"] = None, v.to(device).contiguous()
        else:
            L["k_cache"], L["v_cache"] = k.to(device).contiguous(), v.to(device).contiguous()
        del k, v
        layers.append(L)
    embed = synth.embed_table(cfg, seed, device=gd).to(device).contiguous()
    fnorm = synth.final_norm(cfg, seed, device=gd).to(device).contiguous()
    return DecodeModel(cfg, layers, embed, fnorm, weight_format=0 if weights == "q4" else 1,
                       kv_format=0 if kv == "pair" else 1)
