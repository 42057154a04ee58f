"""Pins for the oracle's per-sub-block dots and output (CPU only).

  * brute force: the per-16-element dots against numpy's integer einsum, and the f64 output
    against a plain f64 matmul of (da * xq) with the dequantized weights -- the q6_K rescale
    without a dmin term ("r38 — q6_K BT-style raw-byte mma kernel", sec. 2.2) is exactly that
    product in exact arithmetic;
  * an exact special case: activations already on the int8 grid (da = 1) and power-of-two d
    make the output equal X @ W^T exactly in f64;
  * the closed-form quantization error bound against the unquantized product;
  * zero activations give y = 0 and T = 0.
"""
import numpy as np
import pytest

import synthetic


def dequant_np(raw, m, k, oracle_mod):
    return oracle_mod.dequant(raw, m, k)


@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (5, 7, 512), (8, 16, 768)])
def test_subdots_brute_force(oracle_mod, n, m, k):
    raw = synthetic.weights(m, k, seed=n * 100 + m)
    x = synthetic.activations(n, k, seed=n + m)
    xq, _ = oracle_mod.quantize(x)
    wc, _, _ = oracle_mod.decode(raw, m, k)
    want = np.einsum("nsi,msi->nms", xq.reshape(n, k // 16, 16).astype(np.int64),
                     wc.reshape(m, k // 16, 16).astype(np.int64))
    got = oracle_mod.subdots(xq, raw, m)
    np.testing.assert_array_equal(got, want)
    assert np.abs(got).max() <= 16 * 127 * 32


def test_subdots_extreme_magnitude(oracle_mod):
    # the largest |D|: all codes 0 (value -32) against xq = 127
    raw = np.zeros((1, 1, 210), np.uint8)
    xq = np.full((1, 256), 127, np.int8)
    np.testing.assert_array_equal(oracle_mod.subdots(xq, raw, 1), np.full((1, 1, 16), -65024))


@pytest.mark.parametrize("n,m,k", [(3, 5, 256), (6, 9, 512), (4, 8, 1024)])
def test_output_brute_force(oracle_mod, n, m, k):
    raw = synthetic.weights(m, k, seed=7 + k, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=3 + n, kind="outlier")
    xq, da = oracle_mod.quantize(x)
    w = dequant_np(raw, m, k, oracle_mod)
    xdq = xq.astype(np.float64) * np.repeat(da.astype(np.float64), 32, axis=1)
    want = xdq @ w.T
    y, t = oracle_mod.gemm(xq, da, raw, m)
    assert (np.abs(y - want) <= 1e-12 * t).all()
    # T is the sum of term magnitudes, so it bounds |y| and is bounded by the f64 |x||w| product
    assert (np.abs(y) <= t * (1 + 1e-12)).all()
    assert (t <= (np.abs(xdq) @ np.abs(w).T) * (1 + 1e-12)).all()


def test_output_exact_on_int_grid(oracle_mod):
    n, m, k = 4, 6, 512
    raw = synthetic.weights(m, k, seed=99, sc_lo=-128, sc_hi=127)
    raw = raw.reshape(m, k // 256, 210)
    raw[:, :, 208] = 0x00
    raw[:, :, 209] = 0x20  # d = 2^-7 everywhere
    rng = np.random.default_rng(4)
    x = rng.integers(-127, 128, (n, k)).astype(np.float32)
    x[:, ::32] = -127  # amax 127 in every chunk -> da = 1, xq = x
    xq, da = oracle_mod.quantize(x)
    assert (da == 1).all()
    w = oracle_mod.dequant(raw, m, k)
    y, _ = oracle_mod.gemm(xq, da, raw, m)
    np.testing.assert_array_equal(y, x.astype(np.float64) @ w.T)


def test_quantization_error_bound(oracle_mod):
    n, m, k = 6, 10, 512
    raw = synthetic.weights(m, k, seed=12)
    x = synthetic.activations(n, k, seed=12, kind="swiglu")
    xq, da = oracle_mod.quantize(x)
    w = oracle_mod.dequant(raw, m, k)
    y, _ = oracle_mod.gemm(xq, da, raw, m)
    exact = x.astype(np.float64) @ w.T
    bound = (np.repeat(da.astype(np.float64), 32, axis=1) * (0.5 + 2.0**-20)) @ np.abs(w).T
    assert (np.abs(y - exact) <= bound).all()


def test_zero_activations(oracle_mod):
    raw = synthetic.weights(3, 256, seed=1)
    xq, da = oracle_mod.quantize(np.zeros((2, 256), np.float32))
    y, t = oracle_mod.gemm(xq, da, raw, 3)
    assert (y == 0).all() and (t == 0).all()


def test_row_and_token_subsets_commute(oracle_mod):
    # the output for a subset of tokens / rows is the subset of the full output (used to sample
    # large workloads): y[rows][:, cols] from sliced inputs equals slicing the full y
    n, m, k = 7, 9, 512
    raw = synthetic.weights(m, k, seed=21).reshape(m, -1)
    x = synthetic.activations(n, k, seed=21)
    xq, da = oracle_mod.quantize(x)
    y, t = oracle_mod.gemm(xq, da, raw, m)
    rows, cols = np.array([0, 3, 6]), np.array([1, 2, 8])
    ys, ts = oracle_mod.gemm(xq[rows], da[rows], np.ascontiguousarray(raw[cols]), len(cols))
    np.testing.assert_array_equal(ys, y[rows][:, cols])
    np.testing.assert_array_equal(ts, t[rows][:, cols])


# ------------------------------------------------------------------------------------------------
# Per-chunk numerators with the sub-block scales applied (the integer part of a 32-k chunk's
# contribution: y = sum_c da[c] * d[c/8] * E[c]).
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,m,k", [(1, 1, 256), (5, 7, 512), (6, 9, 1024)])
def test_chunkdots_from_subdots_and_scales(oracle_mod, n, m, k):
    # E[c] = sc[2c] * D[2c] + sc[2c+1] * D[2c+1], from the pinned sub-block dots and the decoded
    # int8 scales (a different route: the scale is applied after the 16-element dot)
    raw = synthetic.weights(m, k, seed=31 + k, sc_lo=-128, sc_hi=127)
    xq, _ = oracle_mod.quantize(synthetic.activations(n, k, seed=5 + n, kind="outlier"))
    _, sc, _ = oracle_mod.decode(raw, m, k)
    dots = oracle_mod.subdots(xq, raw, m).astype(np.int64)          # [n][m][k/16]
    want = (dots * sc.astype(np.int64)[None, :, :]).reshape(n, m, k // 32, 2).sum(axis=3)
    np.testing.assert_array_equal(oracle_mod.chunkdots(xq, raw, m), want)


def test_chunkdots_brute_force_from_dequant(oracle_mod):
    # sc * (q - 32) = w / d exactly (d * sc * (q - 32) needs at most 24 significant bits), so the
    # numerators are the int64 dot of xq with w / d over each 32-element chunk
    n, m, k = 4, 6, 512
    raw = synthetic.weights(m, k, seed=77, sc_lo=-128, sc_hi=127)
    xq, _ = oracle_mod.quantize(synthetic.activations(n, k, seed=8))
    _, _, d = oracle_mod.decode(raw, m, k)
    assert (d != 0).all()
    w = oracle_mod.dequant(raw, m, k)
    ws = w / np.repeat(d.astype(np.float64), 256, axis=1)
    assert (ws == np.round(ws)).all()
    want = np.einsum("nci,mci->nmc", xq.reshape(n, k // 32, 32).astype(np.int64),
                     ws.astype(np.int64).reshape(m, k // 32, 32))
    np.testing.assert_array_equal(oracle_mod.chunkdots(xq, raw, m), want)


def test_chunkdots_reassemble_output(oracle_mod):
    # sum_c da[c] * d[c/8] * E[c] reproduces the reference output
    n, m, k = 5, 8, 768
    raw = synthetic.weights(m, k, seed=12, sc_lo=-128, sc_hi=127)
    xq, da = oracle_mod.quantize(synthetic.activations(n, k, seed=13, kind="swiglu"))
    _, _, d = oracle_mod.decode(raw, m, k)
    e = oracle_mod.chunkdots(xq, raw, m).astype(np.float64)
    got = np.einsum("nc,mc,nmc->nm", da.astype(np.float64),
                    np.repeat(d.astype(np.float64), 8, axis=1), e)
    y, t = oracle_mod.gemm(xq, da, raw, m)
    assert (np.abs(got - y) <= 1e-12 * t).all()


def test_chunkdots_extreme_magnitude(oracle_mod):
    # the largest |E|: sc = -128 on every sub-block, all codes 0 (value -32), xq = 127
    raw = np.zeros((1, 1, 210), np.uint8)
    raw[0, 0, 192:208] = np.uint8(0x80)
    xq = np.full((1, 256), 127, np.int8)
    np.testing.assert_array_equal(oracle_mod.chunkdots(xq, raw, 1),
                                  np.full((1, 1, 8), 32 * 127 * 4096))
    assert 32 * 127 * 4096 < 2 ** 24
