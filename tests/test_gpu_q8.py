"""GPU parity of the int8 ("int8lin") weights: q8_pack bit-exact against the
oracle's packing through the canonical export, and q8_gemv bit-exact on
exact probes and within tolerance on random inputs, at small ragged sizes and
at the 12B shapes."""
import numpy as np
import pytest
import torch

import int4_q4_gemv_amd as q4
from int4_q4_gemv_amd import synth
from helpers import assert_close, f16bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("N,K", [(64, 32), (1, 64), (100, 96), (130, 256), (257, 3840), (64, 15360)])
def test_q8_pack_bit_exact(orc, N, K):
    print(f"q8 pack N={N} K={K}", flush=True)
    w = synth.normal((N, K), 0.02, synth.gen(N * 11 + K))
    packed = q4.q8_pack(w.to(DEV))
    assert packed.numel() == q4.q8_packed_bytes(N, K)
    gb = q4.q8_unpack(packed, N, K).cpu().numpy()
    assert np.array_equal(gb, orc.q8_pack(w.numpy()))


def test_q8_pack_special_blocks(orc):
    rng = np.random.default_rng(1)
    w = rng.normal(0, 0.02, (48, 256)).astype(np.float32)
    w[0, :32] = 0.0                                              # zero block
    w[1, :32] = np.arange(-16, 16) * 2.0 ** -7; w[1, 0] = -127 * 2.0 ** -7   # grid values
    w[2, 32:64] = 0.0; w[2, 40] = 2.0 ** -17                     # subnormal scale
    w[3, :32] = 2.5 * 2.0 ** -6; w[3, 0] = -127 * 2.0 ** -6      # ties
    w[4, 64:96] *= 1e-30                                         # underflowing scale
    w[5, :32] = 3e6                                              # large, finite scale
    w[6, 32:64] = 1e7                                            # scale overflows fp16
    packed = q4.q8_pack(torch.from_numpy(w).to(DEV))
    gb = q4.q8_unpack(packed, 48, 256).cpu().numpy()
    assert np.array_equal(gb, orc.q8_pack(w))


def test_q8_pack_bf16_matches_fp32_of_same_values(orc):
    w = synth.normal((128, 512), 0.02, synth.gen(19)).to(torch.bfloat16)
    pb = q4.q8_pack(w.to(DEV))
    assert np.array_equal(q4.q8_unpack(pb, 128, 512).cpu().numpy(), orc.q8_pack(w.float().numpy()))


def test_q8_pack_counts_nonfinite_blocks():
    w = torch.zeros(64, 64, device=DEV)
    w[3, 5] = float("nan")
    w[7, 40] = float("inf")
    w[9, 2] = 1e10                                               # absmax/127 overflows fp16
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = q4.q8_pack(w, nonfinite=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 3
    blk = q4.q8_unpack(packed, 64, 64).cpu().numpy()
    for r, b in ((3, 0), (7, 1), (9, 0)):
        assert (blk[r, b] == 0).all()


def _grid_weights(N, K, seed, unit=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(N, K))
    for n in range(N):
        for b in range(K // 32):
            q[n, b * 32 + rng.integers(0, 32)] = 127
    d = np.ones((N, K // 32)) if unit else np.float16(np.exp2(rng.uniform(-12, -6, (N, K // 32)))).astype(np.float64)
    w = (q.reshape(N, -1, 32) * d[:, :, None]).reshape(N, K).astype(np.float32)
    return q, d, w


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(64, 64), (200, 512), (130, 4096), (33, 96), (17, 16384)])
def test_q8_gemv_one_hot_bit_exact(N, K, B):
    print(f"q8 gemv one-hot N={N} K={K} B={B}", flush=True)
    q, d, w = _grid_weights(N, K, N + K)
    packed = q4.q8_pack(torch.from_numpy(w).to(DEV))
    ks = [0, 1, 31, 32, K // 2 + 3, K - 1, 17, 100 % K]
    for i in range(0, len(ks), B):
        sel = ks[i:i + B]
        x = torch.zeros(len(sel), K, dtype=torch.float16)
        for r, k in enumerate(sel):
            x[r, k] = 1.0
        y = q4.q8_gemv(packed, N, K, x.to(DEV)).cpu().numpy()
        for r, k in enumerate(sel):
            assert np.array_equal(y[r], (q[:, k] * d[:, k // 32]).astype(np.float32)), (k, r)


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_q8_gemv_integer_probe_bit_exact(orc, B):
    N, K = 190, 1024
    q, d, w = _grid_weights(N, K, 5, unit=True)
    packed = q4.q8_pack(torch.from_numpy(w).to(DEV))
    xi = np.random.default_rng(B).integers(-2, 3, size=(B, K))
    y = q4.q8_gemv(packed, N, K, torch.from_numpy(xi.astype(np.float16)).to(DEV)).cpu().numpy()
    assert np.array_equal(y, (xi @ q.T).astype(np.float32))
    ref = orc.q8_gemv(orc.q8_pack(w), N, K, xi.astype(np.float16).view(np.uint16))
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(64, 32), (100, 96), (333, 256), (1000, 3840), (77, 15360), (3840, 4096)])
def test_q8_gemv_random_vs_oracle(orc, N, K, B):
    print(f"q8 gemv random N={N} K={K} B={B}", flush=True)
    w, x = synth.gemv_inputs(N, K, B, seed_w=N + 1, seed_x=K + 1)
    packed = q4.q8_pack(w.to(DEV))
    y = q4.q8_gemv(packed, N, K, x.to(DEV))
    ref = orc.q8_gemv(orc.q8_pack(w.numpy()), N, K, f16bits(x))
    assert_close(y, ref, what=f"q8_gemv N={N} K={K} B={B}")


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("N,K", [(15360, 3840), (3840, 15360)])
def test_q8_gemv_12b_shapes_sampled_rows(orc, N, K, B):
    """Full 12B shapes in the benchmark's launch configuration; the oracle
    computes a sample of 256 rows one by one."""
    print(f"q8 gemv 12B N={N} K={K} B={B}", flush=True)
    w, x = synth.gemv_inputs(N, K, B, seed_w=1, seed_x=2)
    packed = q4.q8_pack(w.to(DEV))
    y = q4.q8_gemv(packed, N, K, x.to(DEV)).cpu()
    rows = np.sort(np.random.default_rng(3).choice(N, 256, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 63, 64, N - 1]]))
    ref = orc.q8_gemv(orc.q8_pack(w[rows].numpy()), len(rows), K, f16bits(x))
    assert_close(y[:, rows], ref, what=f"12B q8_gemv N={N} K={K} B={B}")
    y2 = q4.q8_gemv(packed, N, K, x.to(DEV)).cpu()
    assert torch.equal(y, y2)
