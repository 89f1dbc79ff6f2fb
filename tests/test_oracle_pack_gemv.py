"""Pins of the oracle's q4_0 packing and int4 matrix-vector product.

The pages define q4_0 only in words (gemma4-12b card intro: per-block-32
absmax symmetric int4; gemma-4-E4B-CoreAI card, Provenance: symmetric with
clipping, the q4_0 grid), so the pins are hand-worked blocks, closed forms
and brute force against codes the test itself chose.
"""
import numpy as np
import pytest


def f16bits(x):
    return int(np.float16(x).view(np.uint16))


def canon_bytes(codes):
    """Expected canonical code bytes: byte j = (q_j + 8) | (q_{j+16} + 8) << 4."""
    c = np.asarray(codes, dtype=np.int64) + 8
    return [int(c[j] | (c[j + 16] << 4)) for j in range(16)]


def pack1(orc, w):
    blk = orc.q4_pack(np.asarray(w, dtype=np.float32).reshape(1, 32))
    b = blk[0, 0]
    scale_bits = int(b[0]) | (int(b[1]) << 8)
    return scale_bits, [int(v) for v in b[2:]]


# -------------------------------------------------------------- fp16 ----
def test_f16_rounding_matches_numpy(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-5, 5000),      # normals + subnormals
        rng.normal(0, 3e4, 2000), [65504, 65519.99, 65520, 1e6, -1e6, 0.0, -0.0],
        # exact ties between fp16 neighbours (ties to even)
        (np.arange(1024, 1100) + 0.5), (np.arange(1, 200) * 2.0 ** -24 + 2.0 ** -25),
    ])
    got = orc.f64_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    back = orc.f16_to_f64(ref[:3000])
    assert np.array_equal(back, ref[:3000].view(np.float16).astype(np.float64))


# -------------------------------------------------------------- pack ----
def test_zero_block(orc):
    s, codes = pack1(orc, np.zeros(32))
    assert s == 0 and codes == [0x88] * 16


def test_exact_grid_block_all_codes(orc):
    # values k * 0.25 for k = -8..7 (twice): absmax 2.0 -> d = 0.25, codes = k
    q = np.concatenate([np.arange(-8, 8), np.arange(7, -9, -1)])
    s, codes = pack1(orc, q * 0.25)
    assert s == f16bits(0.25)
    assert codes == canon_bytes(q)


def test_positive_absmax_clips_to_7(orc):
    w = np.zeros(32); w[3] = 2.0; w[20] = 0.25; w[31] = -1.0
    s, codes = pack1(orc, w)
    q = np.zeros(32, dtype=int); q[3] = 7; q[20] = 1; q[31] = -4
    assert s == f16bits(0.25) and codes == canon_bytes(q)


def test_ties_round_half_away(orc):
    # -2.0 fixes d = 0.25; w/d = +-1.5, +-0.5, 2.5, -7.5 round away from zero
    w = np.zeros(32)
    w[0] = -2.0
    vals = {1: 0.375, 2: -0.375, 3: 0.125, 4: -0.125, 17: 0.625, 30: -1.875}
    for i, v in vals.items():
        w[i] = v
    s, codes = pack1(orc, w)
    q = np.zeros(32, dtype=int)
    q[0] = -8
    q[1], q[2], q[3], q[4], q[17], q[30] = 2, -2, 1, -1, 3, -8
    assert s == f16bits(0.25) and codes == canon_bytes(q)


def test_subnormal_scale(orc):
    w = np.zeros(32)
    w[5] = -(2.0 ** -17)          # absmax/8 = 2^-20: an fp16 subnormal (16 * 2^-24)
    w[6] = 3 * 2.0 ** -20
    s, codes = pack1(orc, w)
    q = np.zeros(32, dtype=int); q[5] = -8; q[6] = 3
    assert s == 0x0010 and codes == canon_bytes(q)


def test_codes_use_the_stored_fp16_scale(orc):
    # absmax/8 = 0.1250125 rounds to the fp16 scale 0.125; 0.81254/0.125 = 6.5003
    # rounds to 7, while the unrounded scale would give 6.4997 -> 6.
    w = np.zeros(32)
    w[0] = 1.0001
    w[9] = 0.81254
    s, codes = pack1(orc, w)
    q = np.zeros(32, dtype=int); q[0] = 7; q[9] = 7
    assert s == f16bits(0.125) and codes == canon_bytes(q)


@pytest.mark.parametrize("bad", [float("inf"), float("-inf"), float("nan")])
def test_nonfinite_weight_gives_zero_block(orc, bad):
    # a block holding a non-finite weight has no q4_0 encoding: the zero block
    # (scale 0, every code 0), whatever its other weights
    w = np.linspace(-0.05, 0.05, 32)
    w[11] = bad
    s, codes = pack1(orc, w)
    assert s == 0 and codes == [0x88] * 16


def test_overflowing_scale_gives_zero_block(orc):
    # absmax/8 must be representable in fp16: 8 * 65504 keeps the largest
    # finite scale; 8 * 65520 rounds (ties to even) to inf, and 1e6 is far past
    w = np.zeros(32)
    w[0] = -8 * 65504.0
    w[1] = 4 * 65504.0
    s, codes = pack1(orc, w)
    q = np.zeros(32, dtype=int); q[0] = -8; q[1] = 4
    assert s == 0x7BFF and codes == canon_bytes(q)
    for amax in (8 * 65520.0, 1e6):
        w = np.full(32, amax / 3)
        w[7] = -amax
        s, codes = pack1(orc, w)
        assert s == 0 and codes == [0x88] * 16


def test_degenerate_block_leaves_its_neighbours(orc):
    # only the block that holds the bad value is zeroed
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (3, 128)).astype(np.float32)
    ref = orc.q4_pack(w.copy())
    w[1, 40] = np.nan
    w[2, 100] = 1e6
    blk = orc.q4_pack(w)
    zero = np.array([0, 0] + [0x88] * 16, dtype=np.uint8)
    assert np.array_equal(blk[1, 1], zero) and np.array_equal(blk[2, 3], zero)
    keep = np.ones((3, 4), bool); keep[1, 1] = False; keep[2, 3] = False
    assert np.array_equal(blk[keep], ref[keep])


def _grid_matrix(N, K, seed, unit_scale=False):
    """Codes in [-8,7] with one -8 per block (so the block's absmax is 8d and
    packing must reproduce the codes exactly), fp16 scales."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(N, K))
    nb = K // 32
    for n in range(N):
        for b in range(nb):
            q[n, b * 32 + rng.integers(0, 32)] = -8
    if unit_scale:
        d = np.ones((N, nb))
    else:
        d = np.float16(np.exp2(rng.uniform(-9, -3, size=(N, nb)))).astype(np.float64)
    w = (q.reshape(N, nb, 32) * d[:, :, None]).reshape(N, K)
    return q, d, w.astype(np.float32)


def test_pack_reproduces_grid_values(orc):
    N, K = 37, 96
    q, d, w = _grid_matrix(N, K, 11)
    blk = orc.q4_pack(w)
    scale_bits = blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8)
    assert np.array_equal(scale_bits, np.float16(d).view(np.uint16))
    for n in range(N):
        for b in range(K // 32):
            assert [int(v) for v in blk[n, b, 2:]] == canon_bytes(q[n, b * 32:(b + 1) * 32])


def test_quantisation_error_bound(orc):
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(64, 256)).astype(np.float32)
    blk = orc.q4_pack(w)
    wh = orc.q4_dequant(blk, 64, 256)
    d = np.float16(np.abs(w.reshape(64, 8, 32)).max(-1) / 8).astype(np.float64)
    err = np.abs(w.astype(np.float64) - wh).reshape(64, 8, 32)
    clipped = (wh.reshape(64, 8, 32) == 7 * d[:, :, None]) & (w.reshape(64, 8, 32) > 7.5 * d[:, :, None])
    assert np.all(err[~clipped] <= (0.5 + 1e-5) * np.broadcast_to(d[:, :, None], err.shape)[~clipped])
    # the stored scale can sit 2^-11 below absmax/8, so a clipped +absmax errs by up to d(1 + 8*2^-11)
    assert np.all(err[clipped] <= (1.0 + 2.0 ** -8 + 1e-6) * np.broadcast_to(d[:, :, None], err.shape)[clipped])
    codes = np.round(wh.reshape(64, 8, 32) / np.where(d == 0, 1, d)[:, :, None])
    assert codes.min() >= -8 and codes.max() <= 7


# -------------------------------------------------------------- GEMV ----
def test_gemv_one_hot_gives_columns(orc):
    N, K = 20, 128
    q, d, w = _grid_matrix(N, K, 3)
    blk = orc.q4_pack(w)
    for k in (0, 1, 15, 16, 31, 32, 77, 127):
        x = np.zeros((1, K), dtype=np.float16); x[0, k] = 1.0
        y = orc.q4_gemv(blk, N, K, x.view(np.uint16))
        assert np.array_equal(y[0], q[:, k] * d[:, k // 32])


def test_gemv_integer_probe_exact(orc):
    N, K, B = 33, 160, 3
    q, d, w = _grid_matrix(N, K, 4, unit_scale=True)
    blk = orc.q4_pack(w)
    rng = np.random.default_rng(9)
    xi = rng.integers(-2, 3, size=(B, K))
    y = orc.q4_gemv(blk, N, K, xi.astype(np.float16).view(np.uint16))
    assert np.array_equal(y, (xi @ q.T).astype(np.float64))


def test_gemv_random_brute_force(orc):
    N, K, B = 50, 224, 4
    q, d, w = _grid_matrix(N, K, 6)
    blk = orc.q4_pack(w)
    rng = np.random.default_rng(10)
    x = rng.normal(0, 1, size=(B, K)).astype(np.float16)
    y = orc.q4_gemv(blk, N, K, x.view(np.uint16))
    what = (q.reshape(N, -1, 32) * d[:, :, None]).reshape(N, K)
    ref = x.astype(np.float64) @ what.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_f16_gemv_brute_force(orc):
    rng = np.random.default_rng(12)
    W = rng.normal(0, 0.02, size=(70, 96)).astype(np.float16)
    x = rng.normal(0, 1, size=(2, 96)).astype(np.float16)
    y = orc.f16_gemv(W.view(np.uint16), x.view(np.uint16))
    assert np.allclose(y, x.astype(np.float64) @ W.astype(np.float64).T, rtol=1e-12, atol=1e-14)
