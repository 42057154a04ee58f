"""Pins for the q4_K oracle (CPU only).

The 144-byte block ("r18: Load-time B pre-expansion — staging becomes a bulk copy (W_exp's debut,
REVERTED)", sec. 1-3) is checked against what does not come from the decoder itself:
  * an independent encoder (test side) that packs chosen 6-bit (sc, m) pairs and 4-bit codes into
    blocks, whose decode must return exactly what was packed;
  * hand-built blocks with dequantized values worked out by hand;
  * brute force: integer dots and sums against numpy, the f64 output against a plain matmul of
    (da * xq) with the dequantized weights; an exact case on the integer grid.
"""
import numpy as np
import pytest

import synthetic


def encode_scales(sc, mn):
    """Pack eight 6-bit scales and mins into 12 bytes: bytes 0..3 carry sc[0..3] in their low 6
    bits and the top 2 bits of sc[4..7]; bytes 4..7 the same for m; bytes 8..11 carry the low 4
    bits of sc[4..7] (low nibble) and of m[4..7] (high nibble)."""
    s = np.zeros(12, np.uint8)
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (mn[j] & 63) | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    return s


def encode_codes(q):
    """256 codes (0..15) -> 128 bytes: byte 32g + l holds element 64g + l (low nibble) and
    element 64g + 32 + l (high nibble)."""
    q = np.asarray(q, np.uint8).reshape(4, 2, 32)
    return (q[:, 0, :] | (q[:, 1, :] << 4)).reshape(128).astype(np.uint8)


def make_block(d_bits, dmin_bits, sc, mn, q):
    b = np.zeros(144, np.uint8)
    b[0:2] = (d_bits & 255, d_bits >> 8)
    b[2:4] = (dmin_bits & 255, dmin_bits >> 8)
    b[4:16] = encode_scales(sc, mn)
    b[16:144] = encode_codes(q)
    return b


def test_scale_pairs_roundtrip(oracle_mod):
    rng = np.random.default_rng(11)
    for _ in range(200):
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        s = encode_scales(sc, mn)
        for j in range(8):
            assert oracle_mod.q4_scale_min(s, j) == (sc[j], mn[j])


def test_scale_pairs_hand_built(oracle_mod):
    s = np.zeros(12, np.uint8)
    s[0] = 0b11_000101    # sc[0] = 5, top bits 3 -> sc[4] bits 4..5
    s[8] = 0b0110_1001    # sc[4] low nibble 9, m[4] low nibble 6
    s[4] = 0b01_100000    # m[0] = 32, top bits 1 -> m[4] bits 4..5
    assert oracle_mod.q4_scale_min(s, 0) == (5, 32)
    assert oracle_mod.q4_scale_min(s, 4) == (9 | (3 << 4), 6 | (1 << 4))
    for j in (1, 2, 3, 5, 6, 7):
        assert oracle_mod.q4_scale_min(s, j) == (0, 0)


def test_codes_roundtrip_and_placement(oracle_mod):
    rng = np.random.default_rng(12)
    q = rng.integers(0, 16, 256)
    blk = make_block(0x3C00, 0, [1] * 8, [0] * 8, q)
    got = np.array([oracle_mod.q4_code(blk, e) for e in range(256)])
    np.testing.assert_array_equal(got, q)
    # one byte in group 2 at l = 7: element 135 low nibble, element 167 high nibble
    blk = np.zeros(144, np.uint8)
    blk[16 + 64 + 7] = 0xA3
    got = np.array([oracle_mod.q4_code(blk, e) for e in range(256)])
    assert got[135] == 3 and got[167] == 10 and np.count_nonzero(got) == 2


def test_dequant_hand_values(oracle_mod):
    # d = 1.0, dmin = 0.5; sub-block 0: sc 2, m 3; sub-block 5: sc 40, m 17
    sc = [2, 0, 0, 0, 0, 40, 0, 0]
    mn = [3, 0, 0, 0, 0, 17, 0, 0]
    q = np.zeros(256, np.int64)
    q[0], q[31], q[160], q[191] = 15, 7, 1, 12
    blk = make_block(0x3C00, 0x3800, sc, mn, q)
    w = oracle_mod.q4_dequant(blk, 1, 256)[0]
    assert w[0] == 2 * 15 - 1.5 and w[31] == 2 * 7 - 1.5 and w[1] == -1.5
    assert w[160] == 40 * 1 - 8.5 and w[191] == 40 * 12 - 8.5 and w[170] == -8.5
    assert w[64] == 0.0  # sub-block 2: sc = m = 0
    codes, scd, mnd, d, dmin = oracle_mod.q4_decode(blk, 1, 256)
    np.testing.assert_array_equal(codes[0], q)
    np.testing.assert_array_equal(scd[0], sc)
    np.testing.assert_array_equal(mnd[0], mn)
    assert d[0, 0] == 1.0 and dmin[0, 0] == 0.5


@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (5, 7, 512), (6, 9, 768)])
def test_dots_and_sums_brute_force(oracle_mod, n, m, k):
    raw = synthetic.weights_q4k(m, k, seed=n + m + k)
    xq, _ = oracle_mod.quantize(synthetic.activations(n, k, seed=n * 3, kind="outlier"))
    codes, *_ = oracle_mod.q4_decode(raw, m, k)
    want = np.einsum("nci,mci->nmc", xq.reshape(n, k // 32, 32).astype(np.int64),
                     codes.reshape(m, k // 32, 32).astype(np.int64))
    np.testing.assert_array_equal(oracle_mod.q4_chunkdots(xq, raw, m), want)
    np.testing.assert_array_equal(oracle_mod.q4_chunksums(xq),
                                  xq.reshape(n, k // 32, 32).astype(np.int64).sum(axis=2))


def test_dots_extreme(oracle_mod):
    blk = make_block(0x3C00, 0, [1] * 8, [0] * 8, [15] * 256)
    xq = np.full((1, 256), -127, np.int8)
    np.testing.assert_array_equal(oracle_mod.q4_chunkdots(xq, blk, 1), np.full((1, 1, 8), -32 * 127 * 15))
    np.testing.assert_array_equal(oracle_mod.q4_chunksums(xq), np.full((1, 8), -32 * 127))


@pytest.mark.parametrize("n,m,k", [(3, 5, 256), (6, 9, 512), (4, 8, 1024)])
def test_output_brute_force(oracle_mod, n, m, k):
    raw = synthetic.weights_q4k(m, k, seed=7 + k)
    x = synthetic.activations(n, k, seed=3 + n, kind="outlier")
    xq, da = oracle_mod.quantize(x)
    w = oracle_mod.q4_dequant(raw, m, k)
    xdq = xq.astype(np.float64) * np.repeat(da.astype(np.float64), 32, axis=1)
    want = xdq @ w.T
    y, t = oracle_mod.q4_gemm(xq, da, raw, m)
    assert (np.abs(y - want) <= 1e-12 * t).all()
    assert (np.abs(y) <= t * (1 + 1e-12)).all()


def test_output_exact_on_int_grid(oracle_mod):
    # integer activations with amax 127 per chunk (da = 1), d = 1, dmin = 2: y = X . W^T exactly
    n, m, k = 3, 4, 512
    rng = np.random.default_rng(5)
    blocks = []
    for _ in range(m * (k // 256)):
        blocks.append(make_block(0x3C00, 0x4000, rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                 rng.integers(0, 16, 256)))
    raw = np.stack(blocks).reshape(m, k // 256, 144)
    x = rng.integers(-127, 128, size=(n, k)).astype(np.float32)
    x[:, ::32] = 127
    xq, da = oracle_mod.quantize(x)
    assert (da == 1).all() and (xq == x).all()
    w = oracle_mod.q4_dequant(raw, m, k)
    y, _ = oracle_mod.q4_gemm(xq, da, raw, m)
    np.testing.assert_array_equal(y, x.astype(np.float64) @ w.T)
