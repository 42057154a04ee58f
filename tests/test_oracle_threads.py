"""The oracle's row-parallel functions give the same bytes for every thread count (CPU only).

Rows of the output (tokens for the quantization) are independent and each thread runs the same
loops over its own contiguous range, so 1, 3 and 8 threads must agree bit for bit -- including
uneven splits (rows not divisible by the thread count) and more threads than rows.
"""
import numpy as np
import pytest

import synthetic


@pytest.mark.parametrize("threads", [3, 8, 64])
def test_q6k_threaded_equals_single(oracle_mod, threads):
    n, m, k = 37, 29, 768
    raw = synthetic.weights(m, k, seed=11, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=12, kind="outlier")
    xq1, da1 = oracle_mod.quantize(x, threads=1)
    xqt, dat = oracle_mod.quantize(x, threads=threads)
    np.testing.assert_array_equal(xqt, xq1)
    np.testing.assert_array_equal(dat.view(np.uint32), da1.view(np.uint32))
    y1, t1 = oracle_mod.gemm(xq1, da1, raw, m, threads=1)
    yt, tt = oracle_mod.gemm(xq1, da1, raw, m, threads=threads)
    np.testing.assert_array_equal(yt.view(np.uint64), y1.view(np.uint64))
    np.testing.assert_array_equal(tt.view(np.uint64), t1.view(np.uint64))
    np.testing.assert_array_equal(oracle_mod.subdots(xq1, raw, m, threads=threads),
                                  oracle_mod.subdots(xq1, raw, m, threads=1))
    np.testing.assert_array_equal(oracle_mod.chunkdots(xq1, raw, m, threads=threads),
                                  oracle_mod.chunkdots(xq1, raw, m, threads=1))


@pytest.mark.parametrize("threads", [5, 16])
def test_q4k_threaded_equals_single(oracle_mod, threads):
    n, m, k = 21, 19, 512
    raw = synthetic.weights_q4k(m, k, seed=13)
    x = synthetic.activations(n, k, seed=14)
    xq, da = oracle_mod.quantize(x)
    y1, t1 = oracle_mod.q4_gemm(xq, da, raw, m, threads=1)
    yt, tt = oracle_mod.q4_gemm(xq, da, raw, m, threads=threads)
    np.testing.assert_array_equal(yt.view(np.uint64), y1.view(np.uint64))
    np.testing.assert_array_equal(tt.view(np.uint64), t1.view(np.uint64))
    np.testing.assert_array_equal(oracle_mod.q4_chunkdots(xq, raw, m, threads=threads),
                                  oracle_mod.q4_chunkdots(xq, raw, m, threads=1))


def test_default_threads_positive(oracle_mod):
    assert oracle_mod.default_threads() >= 1
