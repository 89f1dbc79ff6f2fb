"""Pins of the oracle's q8 ("int8lin") packing and int8 matrix-vector product.

The pages name the int8lin ship (gemma4-12b card, intro and Throughput table:
the verified-clean variant beside int4linsym) without its block format; the
reading is the int4 rule on the int8 grid: per block of 32, d = fp16(absmax /
127), q = clamp(round_half_away(w / d), -127, 127).  The pins are hand-worked
blocks, closed forms and brute force against codes the test itself chose.
"""
import numpy as np


def f16bits(x):
    return int(np.float16(x).view(np.uint16))


def pack1(orc, w):
    blk = orc.q8_pack(np.asarray(w, dtype=np.float32).reshape(1, 32))
    b = blk[0, 0]
    scale_bits = int(b[0]) | (int(b[1]) << 8)
    return scale_bits, [int(v) for v in b[2:].view(np.int8)]


def test_zero_block(orc):
    s, q = pack1(orc, np.zeros(32))
    assert s == 0 and q == [0] * 32


def test_exact_grid_block(orc):
    # d = 2^-7 exactly: absmax 127 d gives that scale, and every w = d k maps to k
    k = np.array([127, -127, 0, 1, -1, 2, -2, 63, -64, 100, -100, 126, -126, 5, 50, -50,
                  7, 17, 27, 37, 47, 57, 67, 77, 87, 97, 107, 117, -3, -33, -77, -120])
    s, q = pack1(orc, k * 2.0 ** -7)
    assert s == f16bits(2.0 ** -7)
    assert q == list(k)


def test_symmetric_ends(orc):
    # +absmax and -absmax both land on the grid ends
    w = np.zeros(32)
    w[3], w[9] = 3.0, -3.0
    s, q = pack1(orc, w)
    assert q[3] == 127 and q[9] == -127
    assert s == f16bits(np.float32(3.0) / np.float32(127.0))


def test_ties_round_half_away(orc):
    d = 2.0 ** -6
    w = np.zeros(32)
    w[0] = 127 * d                                   # fixes d
    w[1:6] = np.array([0.5, 1.5, 2.5, 10.5, 125.5]) * d
    w[6:11] = -np.array([0.5, 1.5, 2.5, 10.5, 125.5]) * d
    s, q = pack1(orc, w)
    assert s == f16bits(d)
    assert q[1:6] == [1, 2, 3, 11, 126]
    assert q[6:11] == [-1, -2, -3, -11, -126]


def test_subnormal_scale(orc):
    d = 2.0 ** -20                                   # fp16 subnormal
    k = np.arange(-16, 16)
    k[0] = -127
    s, q = pack1(orc, k * d)
    assert s == f16bits(d) and (s & 0x7C00) == 0
    assert q == list(k)


def test_nonfinite_block_is_zero(orc):
    w = np.linspace(-1, 1, 32)
    w[5] = np.inf
    s, q = pack1(orc, w)
    assert s == 0 and q == [0] * 32
    w[5] = np.nan
    s, q = pack1(orc, w)
    assert s == 0 and q == [0] * 32


def test_error_bound_and_byte_order(orc):
    rng = np.random.default_rng(3)
    N, K = 37, 256
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    blk = orc.q8_pack(w)
    d = blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8)
    d = d.view(np.float16).astype(np.float64)
    q = blk[:, :, 2:].view(np.int8).astype(np.float64)       # element i in byte 2 + i
    w_hat = (q * d[:, :, None]).reshape(N, K)
    assert np.array_equal(w_hat, orc.q8_dequant(blk, N, K))
    err = np.abs(w.astype(np.float64) - w_hat).reshape(N, K // 32, 32)
    assert np.all(err <= d[:, :, None] / 2 * (1 + 1e-6))
    assert np.abs(q).max() == 127


def test_gemv_one_hot_columns(orc):
    rng = np.random.default_rng(4)
    N, K = 24, 96
    blk = orc.q8_pack(rng.normal(0, 1, (N, K)).astype(np.float32))
    w_hat = orc.q8_dequant(blk, N, K)
    for k in (0, 31, 32, 95):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1.0
        y = orc.q8_gemv(blk, N, K, x.view(np.uint16))
        assert np.array_equal(y[0], w_hat[:, k])


def test_gemv_integer_probe_exact(orc):
    # d = 1 (absmax 127) and integer codes and inputs: the product is an exact integer sum
    rng = np.random.default_rng(5)
    N, K, B = 16, 128, 3
    k = rng.integers(-127, 128, (N, K))
    k[:, ::32] = 127
    x = rng.integers(-8, 9, (B, K)).astype(np.float16)
    y = orc.q8_gemv(orc.q8_pack(k.astype(np.float32)), N, K, x.view(np.uint16))
    assert np.array_equal(y, x.astype(np.float64) @ k.T.astype(np.float64))


def test_gemv_brute_force(orc):
    rng = np.random.default_rng(6)
    N, K, B = 19, 160, 4
    blk = orc.q8_pack(rng.normal(0, 0.05, (N, K)).astype(np.float32))
    x = rng.normal(0, 1, (B, K)).astype(np.float16)
    ref = np.zeros((B, N))
    for b in range(B):
        for n in range(N):
            acc = 0.0
            for kk in range(K):
                blkn = blk[n, kk // 32]
                d = float(np.frombuffer(bytes(blkn[:2]), dtype=np.float16)[0])
                acc += d * float(np.int8(blkn[2 + kk % 32])) * float(x[b, kk])
            ref[b, n] = acc
    y = orc.q8_gemv(blk, N, K, x.view(np.uint16))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
