"""GPU parity: q4_pack (bit-exact against the oracle's packing, via the
canonical export) and q4_gemv (bit-exact on exact probes, within tolerance on
random inputs) at small ragged sizes and at the 12B shapes."""
import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import assert_close, f16bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pack_both(orc, w_cpu):
    packed = q4.q4_pack(w_cpu.to(DEV))
    N, K = w_cpu.shape
    gpu_blocks = q4.q4_unpack(packed, N, K).cpu().numpy()
    ref_blocks = orc.q4_pack(w_cpu.numpy())
    return packed, gpu_blocks, ref_blocks


@pytest.mark.parametrize("N,K", [(64, 32), (1, 64), (100, 96), (130, 256), (257, 3840), (64, 15360)])
def test_pack_bit_exact(orc, N, K):
    print(f"pack N={N} K={K}", flush=True)
    w = synth.normal((N, K), 0.02, synth.gen(N * 7 + K))
    packed, gb, rb = _pack_both(orc, w)
    assert packed.numel() == q4.packed_bytes(N, K)
    assert np.array_equal(gb, rb)


def test_pack_special_blocks(orc):
    rng = np.random.default_rng(0)
    w = rng.normal(0, 0.02, (64, 256)).astype(np.float32)
    w[0, :32] = 0.0                                  # zero block
    w[1, :32] = np.arange(-8, 24) * 0.25 * (np.arange(32) < 16)   # grid values
    w[2, 32:64] = 0.0; w[2, 40] = 2.0 ** -17         # subnormal scale
    w[3, :32] = 0.375; w[3, 0] = -2.0                # ties
    w[4, 64:96] *= 1e-30                             # underflowing scale
    w[5, :32] = 1e4                                  # large
    wt = torch.from_numpy(w)
    packed, gb, rb = _pack_both(orc, wt)
    assert np.array_equal(gb, rb)


def test_pack_bf16_matches_fp32_of_same_values(orc):
    w = synth.normal((128, 512), 0.02, synth.gen(9)).to(torch.bfloat16)
    pb = q4.q4_pack(w.to(DEV))
    rb = orc.q4_pack(w.float().numpy())
    assert np.array_equal(q4.q4_unpack(pb, 128, 512).cpu().numpy(), rb)


def test_pack_counts_nonfinite_blocks():
    w = torch.zeros(64, 64, device=DEV)
    w[3, 5] = float("nan")
    w[7, 40] = float("inf")
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = q4.q4_pack(w, nonfinite=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 2
    blk = q4.q4_unpack(packed, 64, 64).cpu().numpy()
    assert blk[3, 0, 0] == 0 and blk[3, 0, 1] == 0 and (blk[3, 0, 2:] == 0x88).all()


def test_pack_degenerate_blocks_match_oracle(orc):
    # non-finite weights and scales that overflow fp16 give the zero block on
    # both sides, and the GPU counts each such block once
    rng = np.random.default_rng(1)
    w = rng.normal(0, 0.02, (48, 256)).astype(np.float32)
    w[0, 3] = np.inf
    w[1, 40] = -np.inf
    w[2, 70] = np.nan
    w[3, 96:128] = 1e6                               # absmax/8 far past 65504
    w[4, 128:160] = 8 * 65520.0 / 3; w[4, 130] = -8 * 65520.0   # rounds to inf
    w[5, :32] = 0.0; w[5, 5] = -8 * 65504.0          # the largest finite scale: kept
    w[6, 224:256] = np.nan                           # a whole block
    w[7, 0] = np.nan; w[7, 1] = np.inf               # two in one block: counted once
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = q4.q4_pack(torch.from_numpy(w).to(DEV), nonfinite=cnt)
    gb = q4.q4_unpack(packed, 48, 256).cpu().numpy()
    rb = orc.q4_pack(w)
    assert np.array_equal(gb, rb)
    assert int(cnt.item()) == 7
    zero = np.array([0, 0] + [0x88] * 16, dtype=np.uint8)
    for n, b in [(0, 0), (1, 1), (2, 2), (3, 3), (4, 4), (6, 7), (7, 0)]:
        assert np.array_equal(rb[n, b], zero), (n, b)
    assert rb[5, 0, 0] == 0xFF and rb[5, 0, 1] == 0x7B


def _grid_weights(N, K, seed, unit=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(N, K))
    for n in range(N):
        for b in range(K // 32):
            q[n, b * 32 + rng.integers(0, 32)] = -8
    d = np.ones((N, K // 32)) if unit else np.float16(np.exp2(rng.uniform(-9, -3, (N, K // 32)))).astype(np.float64)
    w = (q.reshape(N, -1, 32) * d[:, :, None]).reshape(N, K).astype(np.float32)
    return q, d, w


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(64, 64), (200, 512), (130, 4096), (33, 96), (17, 16384)])
def test_gemv_one_hot_bit_exact(orc, N, K, B):
    print(f"gemv one-hot N={N} K={K} B={B}", flush=True)
    q, d, w = _grid_weights(N, K, N + K)
    packed = q4.q4_pack(torch.from_numpy(w).to(DEV))
    ks = [0, 1, 31, 32, K // 2 + 3, K - 1, 17, 100 % K]
    for i in range(0, len(ks), B):
        sel = ks[i:i + B]
        x = torch.zeros(len(sel), K, dtype=torch.float16)
        for r, k in enumerate(sel):
            x[r, k] = 1.0
        y = q4.q4_gemv(packed, N, K, x.to(DEV)).cpu().numpy()
        for r, k in enumerate(sel):
            assert np.array_equal(y[r], (q[:, k] * d[:, k // 32]).astype(np.float32)), (k, r)


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_gemv_integer_probe_bit_exact(orc, B):
    N, K = 190, 1024
    q, d, w = _grid_weights(N, K, 5, unit=True)
    packed = q4.q4_pack(torch.from_numpy(w).to(DEV))
    xi = np.random.default_rng(B).integers(-2, 3, size=(B, K))
    y = q4.q4_gemv(packed, N, K, torch.from_numpy(xi.astype(np.float16)).to(DEV)).cpu().numpy()
    assert np.array_equal(y, (xi @ q.T).astype(np.float32))
    blocks = orc.q4_pack(w)
    ref = orc.q4_gemv(blocks, N, K, xi.astype(np.float16).view(np.uint16))
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(64, 32), (100, 96), (333, 256), (1000, 3840), (77, 15360), (3840, 4096)])
def test_gemv_random_vs_oracle(orc, N, K, B):
    print(f"gemv random N={N} K={K} B={B}", flush=True)
    w, x = synth.gemv_inputs(N, K, B, seed_w=N, seed_x=K)
    packed = q4.q4_pack(w.to(DEV))
    y = q4.q4_gemv(packed, N, K, x.to(DEV))
    ref = orc.q4_gemv(orc.q4_pack(w.numpy()), N, K, f16bits(x))
    assert_close(y, ref, what=f"q4_gemv N={N} K={K} B={B}")


@pytest.mark.parametrize("B", [1, 4])
def test_gemv_deterministic(B):
    N, K = 3840, 15360
    w, x = synth.gemv_inputs(N, K, B, seed_w=1, seed_x=2, device=DEV)
    packed = q4.q4_pack(w)
    y1 = q4.q4_gemv(packed, N, K, x).clone()
    y2 = q4.q4_gemv(packed, N, K, x).clone()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(15360, 3840), (3840, 15360)])
def test_gemv_12b_shapes_sampled_rows(orc, N, K, B):
    """Full 12B shapes in the benchmark's launch configuration; the oracle
    computes a sample of 256 rows one by one."""
    print(f"gemv 12B N={N} K={K} B={B}", flush=True)
    w, x = synth.gemv_inputs(N, K, B, seed_w=1, seed_x=2)
    packed = q4.q4_pack(w.to(DEV))
    y = q4.q4_gemv(packed, N, K, x.to(DEV)).cpu()
    rows = np.sort(np.random.default_rng(3).choice(N, 256, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 63, 64, N - 1]]))
    ref = orc.q4_gemv(orc.q4_pack(w[rows].numpy()), len(rows), K, f16bits(x))
    assert_close(y[:, rows], ref, what=f"12B q4_gemv N={N} K={K} B={B}")
