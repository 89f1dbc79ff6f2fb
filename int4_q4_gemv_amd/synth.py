"""Seeded synthetic inputs shared by the tests, ``smoke()`` and ``bench.py``.

This module only draws random numbers and lays them out; it holds none of the
decode step's arithmetic (no quantisation, no matrix products, no attention).
Both the HIP path and the CPU oracle receive exactly these arrays.

Recipes (distributions follow the workloads the pages describe; sizes follow
the five workload configurations: toy 2-layer step, isolated GEMV at 12B
shapes, full-attention flash decode, sliding-ring flash decode, 48-layer step):
  * linear weights ~ N(0, 0.02^2), fp32, quantised later by each side;
  * fp16 activations / queries / keys / values ~ N(0, 1);
  * tied fp16 vocab table ~ N(0, 0.02^2);
  * norm multipliers ~ N(1, 0.1^2); layer_scalar 1.0 unless stated;
  * full-layer V rows: the key row divided by its root-mean-square (the
    "V = RMSNorm without scale of K" workload); a preparation of the input
    array, not a step the kernels under test perform.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


def gen(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float, g: torch.Generator, dtype=torch.float32, mean: float = 0.0,
           device: str = "cpu") -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def f16_bits(t: torch.Tensor) -> np.ndarray:
    """fp16 tensor -> numpy uint16 bit pattern (host)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def unit_rms_rows(k16: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """Full-layer V rows for the isolated attention workload (see header)."""
    k = k16.float()
    return (k / torch.sqrt((k * k).mean(-1, keepdim=True) + eps)).to(torch.float16)


# ------------------------------------------------------------------ model ----
@dataclass(frozen=True)
class ModelConfig:
    hidden: int = 3840
    n_heads: int = 16
    inter: int = 15360
    vocab: int = 262144
    n_layers: int = 48
    full_every: int = 6          # full attention at l % full_every == full_every - 1
    sl_kv_heads: int = 8
    sl_head_dim: int = 256
    full_head_dim: int = 512
    window: int = 1024
    ring: int = 2048
    full_cap: int = 32768 + 8
    sl_theta: float = 1.0e4
    full_theta: float = 1.0e6
    sl_rot_frac_den: int = 1     # sliding: every pair rotates
    full_rot_frac_den: int = 4   # full: first quarter of the pairs rotate (64 of 256)
    sl_scale: float = 1.0
    full_scale: float = 1.0
    eps: float = 1e-6
    softcap: float = 30.0
    sl_v_norm: bool = False
    layer_scalar: float = 1.0

    def is_full(self, l: int) -> bool:
        return (l % self.full_every) == self.full_every - 1

    @property
    def sl_rot_pairs(self) -> int:
        return (self.sl_head_dim // 2) // self.sl_rot_frac_den

    @property
    def full_rot_pairs(self) -> int:
        return (self.full_head_dim // 2) // self.full_rot_frac_den

    def layer_shapes(self, l: int):
        """(name, N, K) of every q4 matrix of layer l."""
        H, Hq = self.hidden, self.n_heads
        if self.is_full(l):
            D, Hkv = self.full_head_dim, 1
            mats = [("wq", Hq * D, H), ("wk", Hkv * D, H)]
        else:
            D, Hkv = self.sl_head_dim, self.sl_kv_heads
            mats = [("wq", Hq * D, H), ("wk", Hkv * D, H), ("wv", Hkv * D, H)]
        mats += [("wo", H, Hq * D), ("wg", self.inter, H), ("wu", self.inter, H),
                 ("wd", H, self.inter)]
        return mats


# Toy 2-layer step: hidden 256, 4 query heads; layer 0 sliding (2 KV heads x 64,
# window 64, ring 128), layer 1 full (1 KV head x 128), MLP 1024, vocab 4096.
TOY = ModelConfig(hidden=256, n_heads=4, inter=1024, vocab=4096, n_layers=2, full_every=2,
                  sl_kv_heads=2, sl_head_dim=64, full_head_dim=128, window=64, ring=128,
                  full_cap=256)

# 48-layer step at 12B shapes (40 sliding + 8 full, full at 5, 11, ..., 47).
FULL48 = ModelConfig()


@dataclass
class LayerTensors:
    """Un-quantised parameters of one layer (host or device torch tensors)."""
    mats: dict            # name -> fp32 [N, K]
    norms: dict           # name -> fp32 [dim]
    layer_scalar: float


def layer_params(cfg: ModelConfig, l: int, seed: int, device: str = "cpu",
                 with_mats: bool = True) -> LayerTensors:
    """Draws layer l's parameters from a generator seeded by (seed, l)."""
    g = gen(seed * 1000 + l + 1, device)
    mats = {}
    for name, N, K in cfg.layer_shapes(l):
        w = normal((N, K), 0.02, g, device=device)
        if with_mats:
            mats[name] = w
    D = cfg.full_head_dim if cfg.is_full(l) else cfg.sl_head_dim
    norms = {
        "attn_norm": normal((cfg.hidden,), 0.1, g, mean=1.0, device=device),
        "q_norm": normal((D,), 0.1, g, mean=1.0, device=device),
        "k_norm": normal((D,), 0.1, g, mean=1.0, device=device),
        "post_attn_norm": normal((cfg.hidden,), 0.1, g, mean=1.0, device=device),
        "pre_ff_norm": normal((cfg.hidden,), 0.1, g, mean=1.0, device=device),
        "post_ff_norm": normal((cfg.hidden,), 0.1, g, mean=1.0, device=device),
    }
    return LayerTensors(mats, norms, cfg.layer_scalar)


def embed_table(cfg: ModelConfig, seed: int, device: str = "cpu") -> torch.Tensor:
    g = gen(seed * 1000 + 999, device)
    return normal((cfg.vocab, cfg.hidden), 0.02, g, dtype=torch.float16, device=device)


def final_norm(cfg: ModelConfig, seed: int, device: str = "cpu") -> torch.Tensor:
    g = gen(seed * 1000 + 998, device)
    return normal((cfg.hidden,), 0.1, g, mean=1.0, device=device)


def layer_cache(cfg: ModelConfig, l: int, seed: int, ctx: int, device: str = "cpu"):
    """Prefilled fp16 caches for a decode at position ``ctx``.

    Full layers: rows 0..ctx-1 hold K ~ N(0,1) and V = K / rms(K); the rest of
    the capacity is zero.  Sliding layers: every ring slot j holds keys and
    values ~ N(0,1) for the newest position p < ctx with p mod R == j."""
    g = gen(seed * 1000 + 500 + l, device)
    if cfg.is_full(l):
        D = cfg.full_head_dim
        k = torch.zeros(cfg.full_cap, D, dtype=torch.float16, device=device)
        v = torch.zeros_like(k)
        if ctx > 0:
            kk = normal((ctx, D), 1.0, g, dtype=torch.float16, device=device)
            k[:ctx] = kk
            v[:ctx] = unit_rms_rows(kk)
    else:
        D, Hkv, R = cfg.sl_head_dim, cfg.sl_kv_heads, cfg.ring
        k = normal((Hkv, R, D), 1.0, g, dtype=torch.float16, device=device)
        v = normal((Hkv, R, D), 1.0, g, dtype=torch.float16, device=device)
        if ctx < R:   # never-written slots are zero
            k[:, ctx:] = 0
            v[:, ctx:] = 0
    return k, v


def tokens(cfg: ModelConfig, n: int, seed: int) -> np.ndarray:
    g = gen(seed * 1000 + 997)
    return torch.randint(0, cfg.vocab, (n,), generator=g).numpy().astype(np.int32)


# --------------------------------------------------------- kernel inputs ----
def gemv_inputs(N: int, K: int, B: int, seed_w: int = 1, seed_x: int = 2, device: str = "cpu"):
    w = normal((N, K), 0.02, gen(seed_w, device), device=device)
    x = normal((B, K), 1.0, gen(seed_x, device), dtype=torch.float16, device=device)
    return w, x


def full_attn_inputs(ctx: int, cap: int, n_rows: int = 1, Hq: int = 16, D: int = 512,
                     seed: int = 3, device: str = "cpu"):
    """Query [n, Hq, D] and K/V [cap, D]; rows ctx..cap-1 are zero.  The
    verify rows decode positions ctx-n_rows .. ctx-1."""
    g = gen(seed, device)
    q = normal((n_rows, Hq, D), 1.0, g, dtype=torch.float16, device=device)
    k = torch.zeros(cap, D, dtype=torch.float16, device=device)
    kk = normal((ctx, D), 1.0, g, dtype=torch.float16, device=device)
    k[:ctx] = kk
    v = torch.zeros_like(k)
    v[:ctx] = unit_rms_rows(kk)
    return q, k, v


POISON = 60000.0


def ring_inputs(q_pos: int, n_rows: int = 1, n_rejected: int = 4, Hq: int = 16, Hkv: int = 8,
                D: int = 256, R: int = 2048, seed: int = 4, device: str = "cpu"):
    """Query rows at positions q_pos..q_pos+n_rows-1 over a ring holding
    N(0,1) keys/values; the ``n_rejected`` slots after the last row hold
    rejected speculative rows filled with +-POISON (never to be admitted)."""
    g = gen(seed, device)
    q = normal((n_rows, Hq, D), 1.0, g, dtype=torch.float16, device=device)
    k = normal((Hkv, R, D), 1.0, g, dtype=torch.float16, device=device)
    v = normal((Hkv, R, D), 1.0, g, dtype=torch.float16, device=device)
    last = q_pos + n_rows - 1
    for i in range(1, n_rejected + 1):
        s = (last + i) % R
        sign = torch.where(normal((Hkv, D), 1.0, g, device=device) >= 0, 1.0, -1.0)
        k[:, s, :] = (sign * POISON).to(torch.float16)
        v[:, s, :] = (-sign * POISON).to(torch.float16)
    return q, k, v


__all__ = [n for n in dir() if not n.startswith("_")]
