"""Algorithmic byte model of the decode step (what the method must move).

Per unit:
  * int4 q4_0 weight: 18 bytes per 32 weights (16 bytes of codes + one fp16
    scale) = 0.5625 B/weight (gemma4-12b card intro: per-block-32 q4_0);
  * fp16 vocab-table element: 2 B (Gemma-4-12B-CoreAI card, tiered-v3: fp16
    vocab path, tied head [262144, 3840]);
  * full-attention position: K and V rows of head_dim fp16 values, 2*2*D B
    (2,048 B at D = 512; Gemma-4-12B-CoreAI card, per-tier cost: a global pair
    [8,1,1,C,512] is 16,384 B per token over 8 layers), or 2*D B when the
    layer caches only the V row and forms the key from it;
  * sliding-window position: 2*2*D B per KV head, W positions per KV head.
Activations, norm vectors and split-K partials are not counted (they are
kilobytes and stay in L2/MALL).
"""
from __future__ import annotations

from .synth import ModelConfig


def q4_matrix_bytes(N: int, K: int) -> int:
    assert K % 32 == 0
    return N * (K // 32) * 18


def layer_weight_bytes(cfg: ModelConfig, l: int) -> int:
    return sum(q4_matrix_bytes(N, K) for _, N, K in cfg.layer_shapes(l))


def weight_bytes(cfg: ModelConfig) -> int:
    return sum(layer_weight_bytes(cfg, l) for l in range(cfg.n_layers))


def head_bytes(cfg: ModelConfig) -> int:
    return cfg.vocab * cfg.hidden * 2


def full_pos_bytes(cfg: ModelConfig, kv_format: int = 0) -> int:
    """Bytes per full-attention position: the K and V rows, or only the V
    row when the layer caches one row per position (kv_format 1)."""
    return (2 if kv_format == 0 else 1) * 2 * cfg.full_head_dim


def ring_call_bytes(cfg: ModelConfig, q_pos: int) -> int:
    """K+V bytes one sliding layer reads for a query at position q_pos."""
    admitted = min(cfg.window, q_pos + 1)
    return cfg.sl_kv_heads * admitted * 2 * 2 * cfg.sl_head_dim


def n_full(cfg: ModelConfig) -> int:
    return sum(1 for l in range(cfg.n_layers) if cfg.is_full(l))


def step_bytes(cfg: ModelConfig, pos: int, n_rows: int = 1, kv_format: int = 0) -> int:
    """Algorithmic bytes of one decode step whose last row sits at ``pos``.

    Weights, head and KV are streamed once for all rows of a verify block."""
    nf = n_full(cfg)
    ns = cfg.n_layers - nf
    return (weight_bytes(cfg) + head_bytes(cfg) + nf * (pos + 1) * full_pos_bytes(cfg, kv_format)
            + ns * ring_call_bytes(cfg, pos))


# ---- cache sizes in the pages' own layouts (used to pin the arithmetic) ----
def cache_bytes(*dims: int, elem: int = 2, pair: bool = True) -> int:
    n = elem
    for d in dims:
        n *= d
    return n * (2 if pair else 1)


def chunk_bytes(cfg: ModelConfig, pos0: int, n: int) -> int:
    """Algorithmic bytes of a prefill chunk of n rows at positions pos0 ..
    pos0 + n - 1: the weights and the head once (the head for the last row),
    and every cached position the rows attend read once for the whole chunk
    (the rows share their K/V tiles): on a full layer positions 0 .. pos0+n-1,
    on a sliding layer the union of the rows' windows."""
    nf = n_full(cfg)
    ns = cfg.n_layers - nf
    last = pos0 + n - 1
    ring_pos = min(cfg.window + n - 1, last + 1)
    return (weight_bytes(cfg) + head_bytes(cfg) + nf * (last + 1) * full_pos_bytes(cfg)
            + ns * cfg.sl_kv_heads * ring_pos * 2 * 2 * cfg.sl_head_dim)
