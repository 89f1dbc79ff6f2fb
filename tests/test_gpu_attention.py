"""GPU parity: flash_decode_full and flash_decode_ring against the oracle.

Full: gemma4-12b card, "The fix" (one KV head, 16 query heads, head_dim 512,
scale 1).  Ring: Gemma-4-12B-CoreAI card, "v5/ -- ring extent R = 2W"
(implied-position rule, rejected verify rows never admitted)."""
import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import assert_close, f16bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("ctx,n_rows", [(1, 1), (31, 1), (200, 2), (333, 4), (4100, 1)])
def test_full_small_vs_oracle(orc, D, ctx, n_rows):
    print(f"full D={D} ctx={ctx} rows={n_rows}", flush=True)
    cap = ctx + 40
    q, k, v = synth.full_attn_inputs(ctx, cap, n_rows, Hq=16, D=D, seed=ctx + D)
    pos0 = ctx - n_rows
    out = q4.flash_decode_full(q.to(DEV), k.to(DEV), v.to(DEV), pos0, 1.0)
    ref = orc.flash_full(f16bits(q), f16bits(k), f16bits(v), pos0, 1.0)
    assert_close(out[0], ref, what=f"full D={D} ctx={ctx}")


def test_full_scale_and_heads(orc):
    q, k, v = synth.full_attn_inputs(700, 800, 1, Hq=8, D=128, seed=5)
    out = q4.flash_decode_full(q.to(DEV), k.to(DEV), v.to(DEV), 699, 0.0625)
    ref = orc.flash_full(f16bits(q), f16bits(k), f16bits(v), 699, 0.0625)
    assert_close(out[0], ref, what="full scale 1/16, 8 heads")


def test_full_capacity_independence():
    """Padded capacity is never read: identical bits at two capacities."""
    q, k, v = synth.full_attn_inputs(3000, 3000, 1, seed=6)
    big_k = torch.cat([k, torch.full((5000, 512), float("nan"), dtype=torch.float16)])
    big_v = torch.cat([v, torch.full((5000, 512), float("nan"), dtype=torch.float16)])
    a = q4.flash_decode_full(q.to(DEV), k.to(DEV), v.to(DEV), 2999, 1.0)
    b = q4.flash_decode_full(q.to(DEV), big_k.to(DEV), big_v.to(DEV), 2999, 1.0)
    assert torch.equal(a, b)


@pytest.mark.parametrize("ctx", [32768, 131072])
def test_full_config_sizes_vs_oracle(orc, ctx):
    """The full-attention workload at 32K and 131K context, every output."""
    print(f"full config ctx={ctx}", flush=True)
    q, k, v = synth.full_attn_inputs(ctx, ctx + 4, 1, seed=3)
    out = q4.flash_decode_full(q.to(DEV), k.to(DEV), v.to(DEV), ctx - 1, 1.0)
    ref = orc.flash_full(f16bits(q), f16bits(k), f16bits(v), ctx - 1, 1.0)
    assert_close(out[0], ref, what=f"full ctx={ctx}")


def test_full_multi_sequence(orc):
    n_seq, cap, D = 3, 600, 256
    qs, ks, vs = [], [], []
    for s in range(n_seq):
        q, k, v = synth.full_attn_inputs(500 + 30 * s, cap, 2, Hq=16, D=D, seed=40 + s)
        qs.append(q); ks.append(k); vs.append(v)
    pos = [498, 528, 558]
    out = q4.flash_decode_full(torch.stack(qs).to(DEV), torch.stack(ks).to(DEV), torch.stack(vs).to(DEV), pos, 1.0)
    for s in range(n_seq):
        ref = orc.flash_full(f16bits(qs[s]), f16bits(ks[s]), f16bits(vs[s]), pos[s], 1.0)
        assert_close(out[s], ref, what=f"full seq {s}")


# ------------------------------------------------------------------ ring ----
RING_POSITIONS = [0, 10, 1022, 1023, 1024, 2046, 2047, 2048, 3070, 100000, 100350]


@pytest.mark.parametrize("P", RING_POSITIONS)
def test_ring_positions_vs_oracle(orc, P):
    print(f"ring P={P}", flush=True)
    q, k, v = synth.ring_inputs(P, n_rows=1, n_rejected=4)
    out = q4.flash_decode_ring(q.to(DEV), k.to(DEV), v.to(DEV), 1024, P, 1.0)
    ref = orc.flash_ring(f16bits(q), f16bits(k), f16bits(v), 1024, P, 1.0)
    assert_close(out[0], ref, what=f"ring P={P}")


def test_ring_poisoned_workload_admitted_set_exact():
    """Uniform keys and V = slot id: the output is the exact mean of the
    admitted slot ids, so the admitted set itself is checked bit for bit."""
    P, R, W = 100000, 2048, 1024
    q, k, v = synth.ring_inputs(P, n_rows=1, n_rejected=4)
    k = torch.zeros_like(k)
    ids = torch.arange(R, dtype=torch.float32)[None, :, None].expand(8, R, 256).to(torch.float16)
    v = ids.clone()
    for i in range(1, 5):
        v[:, (P + i) % R] = synth.POISON
    out = q4.flash_decode_ring(q.to(DEV), k.to(DEV), v.contiguous().to(DEV), W, P, 1.0)[0].cpu()
    expect = float(np.mean(np.arange(673, 1697)))
    assert torch.all(out == expect)


@pytest.mark.parametrize("n_rows", [2, 4])
def test_ring_verify_rows(orc, n_rows):
    P = 100000
    q, k, v = synth.ring_inputs(P, n_rows=n_rows, n_rejected=2)
    out = q4.flash_decode_ring(q.to(DEV), k.to(DEV), v.to(DEV), 1024, P, 1.0)
    ref = orc.flash_ring(f16bits(q), f16bits(k), f16bits(v), 1024, P, 1.0)
    assert_close(out[0], ref, what=f"ring rows={n_rows}")


@pytest.mark.parametrize("P", [2045, 2046, 2047, 4094, 100350])
def test_ring_verify_rows_across_the_ring_end(orc, P):
    """4 rows whose slots wrap from R-1 to 0 (P mod 2048 in 2045 .. 2047)."""
    print(f"ring rows across the end P={P}", flush=True)
    q, k, v = synth.ring_inputs(P, n_rows=4, n_rejected=0)
    out = q4.flash_decode_ring(q.to(DEV), k.to(DEV), v.to(DEV), 1024, P, 1.0)
    ref = orc.flash_ring(f16bits(q), f16bits(k), f16bits(v), 1024, P, 1.0)
    assert_close(out[0], ref, what=f"ring 4 rows at P={P}")


def test_ring_small_window_shapes(orc):
    # toy sliding layer: 4 heads over 2 KV heads, D 64, W 64, R 128
    q, k, v = synth.ring_inputs(200, n_rows=3, n_rejected=0, Hq=4, Hkv=2, D=64, R=128, seed=8)
    out = q4.flash_decode_ring(q.to(DEV), k.to(DEV), v.to(DEV), 64, 200, 1.0)
    ref = orc.flash_ring(f16bits(q), f16bits(k), f16bits(v), 64, 200, 1.0)
    assert_close(out[0], ref, what="toy ring")


def test_ring_forty_sequences(orc):
    n_seq = 40
    qs, ks, vs = [], [], []
    for s in range(n_seq):
        q, k, v = synth.ring_inputs(100000 + s, seed=100 + s)
        qs.append(q); ks.append(k); vs.append(v)
    out = q4.flash_decode_ring(torch.stack(qs).to(DEV), torch.stack(ks).to(DEV), torch.stack(vs).to(DEV),
                               1024, [100000 + s for s in range(n_seq)], 1.0)
    for s in (0, 17, 39):
        ref = orc.flash_ring(f16bits(qs[s]), f16bits(ks[s]), f16bits(vs[s]), 1024, 100000 + s, 1.0)
        assert_close(out[s], ref, what=f"ring seq {s}")
