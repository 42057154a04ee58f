"""Pins for the oracle's activation quantization (CPU only).

The pages name only a scale per token block for the activations ("r38 — q6_K BT-style raw-byte
mma kernel (LANDED)", sec. 2.2).  The reading adopted (symmetric absmax per 32-k chunk,
da = amax/127 in f32, q = round-half-away(x/da) clamped to +-127, zero chunk -> da = 0, q = 0) is
pinned here by special cases with known answers and by closed-form invariants of that reading.
"""
import numpy as np


def test_special_chunk_ties_go_away_from_zero(oracle_mod):
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [127, -127, 2.5, -2.5, 0.5, -0.5, 1.5, 126.5]
    xq, da = oracle_mod.quantize(x)
    assert da[0, 0] == 1.0
    np.testing.assert_array_equal(xq[0, :8], [127, -127, 3, -3, 1, -1, 2, 127])
    assert (xq[0, 8:] == 0).all()


def test_zero_chunk(oracle_mod):
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 3.0
    xq, da = oracle_mod.quantize(x)
    assert da[0, 0] == 0 and da[0, 1] == 0 and da[1, 0] == 0
    assert (xq[0] == 0).all() and (xq[1, :32] == 0).all()
    assert da[1, 1] == np.float32(3.0) / np.float32(127.0)
    assert (xq[1, 32:] == 127).all()


def test_scale_two(oracle_mod):
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [254, 1, -1, 3]
    xq, da = oracle_mod.quantize(x)
    assert da[0, 0] == 2.0
    np.testing.assert_array_equal(xq[0, :4], [127, 1, -1, 2])  # 0.5 -> 1, -0.5 -> -1, 1.5 -> 2


def test_chunks_are_independent_and_aligned(oracle_mod):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    xq, da = oracle_mod.quantize(x)
    for c in range(8):
        xq1, da1 = oracle_mod.quantize(np.ascontiguousarray(x[:, 32 * c:32 * c + 32]))
        np.testing.assert_array_equal(xq1, xq[:, 32 * c:32 * c + 32])
        np.testing.assert_array_equal(da1[:, 0], da[:, c])


def test_invariants_random(oracle_mod):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 1024)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(np.float32)
    x[:, 40] *= 20
    xq, da = oracle_mod.quantize(x)
    xc = x.reshape(64, 32, 32).astype(np.float64)
    q = xq.reshape(64, 32, 32).astype(np.float64)
    amax = np.abs(xc).max(axis=2)
    assert (np.abs(q) <= 127).all()
    assert np.array_equal(da, (amax.astype(np.float32) / np.float32(127)))
    # the element of largest magnitude maps to +-127
    idx = np.abs(xc).argmax(axis=2)
    top = np.take_along_axis(q, idx[..., None], 2)[..., 0]
    topx = np.take_along_axis(xc, idx[..., None], 2)[..., 0]
    np.testing.assert_array_equal(top, 127 * np.sign(topx))
    # sign agreement and the rounding bound |x - da*q| <= da/2 (plus one f32 rounding of x/da)
    assert ((np.sign(q) == np.sign(xc)) | (q == 0)).all()
    err = np.abs(xc - da[..., None].astype(np.float64) * q)
    assert (err <= da[..., None] * (0.5 + 127 * 2.0**-23)).all()


def test_roundtrip_exact_grid(oracle_mod):
    # integers with amax 127 in every chunk quantize to themselves with da = 1
    rng = np.random.default_rng(2)
    x = rng.integers(-127, 128, (4, 128)).astype(np.float32)
    x[:, ::32] = 127
    xq, da = oracle_mod.quantize(x)
    assert (da == 1).all()
    np.testing.assert_array_equal(xq, x.astype(np.int8))


def test_tile_views_agree_with_whole_buffer_views():
    # test-side helpers only: the per-tile views read the same bytes as the whole-buffer ones
    from layouts import untile_da, untile_da_tile, untile_xq, untile_xq_tile
    rng = np.random.default_rng(7)
    n, k = 200, 512
    np_ = 256
    xq = rng.integers(0, 256, np_ * k, dtype=np.uint8)
    da = rng.standard_normal(np_ * (k // 32)).astype(np.float32)
    whole_q, whole_d = untile_xq(xq, n, k), untile_da(da, n, k)
    for t in (0, 3, 7):
        np.testing.assert_array_equal(untile_xq_tile(xq, t, k), whole_q[32 * t: 32 * t + 32])
        np.testing.assert_array_equal(untile_da_tile(da, t, k), whole_d[32 * t: 32 * t + 32])
