"""GPU parity of the q4_K variant (include/q4k.h) against the q4_K oracle.

  * load-time planes: codes byte-exact, (d*sc, -dmin*m) pairs exact ("r18: Load-time B
    pre-expansion — staging becomes a bulk copy (W_exp's debut, REVERTED)", sec. 2);
  * das = da * S bit-exact (one correctly rounded f32 product of exact factors);
  * the per-chunk integer dots bit-exact, exported by the GEMM kernel source;
  * outputs within 1e-3 * sum|terms| for every element at small sizes and for sampled tokens
    at the ffn_down shape.
"""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import round_up, untile_da, untile_q4k

pytestmark = pytest.mark.gpu


def prep_weights(raw, m, k):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    wr = torch.from_numpy(np.ascontiguousarray(raw).reshape(-1)).to(gpu_util.DEV)
    w = torch.full((q6k.q4k_weight_bytes(m, k),), 0x5A, dtype=torch.uint8, device=gpu_util.DEV)
    q6k.q4k_expand_weights(wr, m, k, w)
    return w


def prep_acts(x):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, k = x.shape
    xq, da = gpu_util.quantize(x)
    das = torch.full_like(da, float("nan"))
    q6k.q4k_act_sums(xq, da, n, k, das)
    return xq, da, das


def run_gemm(xq, da, das, n, w, m, k, ldy=None):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    ldy = m if ldy is None else ldy
    y = torch.full((n, ldy), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q4k_gemm(xq, da, das, n, w, m, k, y, ldy=ldy)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("m,k", [(64, 256), (40, 512), (129, 1024), (1, 256)])
def test_expand(m, k):
    print(f"q4k expand m={m} k={k}", flush=True)
    raw = synthetic.weights_q4k(m, k, seed=m + k)
    w = prep_weights(raw, m, k).cpu().numpy()
    codes, pairs = untile_q4k(w, m, k)
    c_ref, sc, mn, d, dmin = oracle.q4_decode(raw, m, k)
    np.testing.assert_array_equal(codes[:m], c_ref)
    want = np.stack([np.repeat(d, 8, axis=1) * sc, -(np.repeat(dmin, 8, axis=1) * mn)], axis=2)
    np.testing.assert_array_equal(pairs[:m].view(np.uint32), want.astype(np.float32).view(np.uint32))
    assert (codes[m:] == 0).all() and (pairs[m:] == 0).all()
    assert w.size == round_up(m, 128) * k * 5 // 4


@pytest.mark.parametrize("n,k", [(64, 512), (65, 256), (200, 1024)])
def test_act_sums(n, k):
    x = synthetic.activations(n, k, seed=n, kind="outlier")
    xq, da, das = prep_acts(x)
    got = untile_da(das.cpu().numpy(), n, k)
    xq_ref, da_ref = oracle.quantize(x)
    s = oracle.q4_chunksums(xq_ref).astype(np.float32)
    want = (da_ref * s).astype(np.float32)  # one f32 product: both factors exact in f32
    np.testing.assert_array_equal(got[:n].view(np.uint32), want.view(np.uint32))
    assert (got[n:] == 0).all()


@pytest.mark.parametrize("n,k", [(64, 512), (65, 256), (200, 1024), (1, 256)])
def test_fused_prepass_equals_quantize_then_sums(n, k):
    """q4k_quantize_act writes the xq and da of q6k_quantize_act and the das of q4k_act_sums, bit
    for bit (the same codes, scales and one f32 product per (token, chunk)), and das matches the
    oracle's da * S."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    print(f"q4k fused prepass n={n} k={k}", flush=True)
    x = synthetic.activations(n, k, seed=n + 3, kind="outlier")
    xq, da, das = prep_acts(x)
    xb, db = q6k.q6k_act_bytes(n, k)
    xq2 = torch.full((xb,), 0x5A, dtype=torch.uint8, device=gpu_util.DEV)
    da2 = torch.full((db // 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    das2 = torch.full_like(da2, float("nan"))
    q6k.q4k_quantize_act(torch.from_numpy(x).to(gpu_util.DEV), xq2, da2, das2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq2.cpu().numpy(), xq.cpu().numpy())
    np.testing.assert_array_equal(da2.cpu().numpy().view(np.uint32), da.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(das2.cpu().numpy().view(np.uint32), das.cpu().numpy().view(np.uint32))
    xq_ref, da_ref = oracle.quantize(x)
    want = (da_ref * oracle.q4_chunksums(xq_ref).astype(np.float32)).astype(np.float32)
    got = untile_da(das2.cpu().numpy(), n, k)
    np.testing.assert_array_equal(got[:n].view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("n,m,k", [(64, 256, 512), (65, 40, 512), (1, 1, 256), (129, 130, 768)])
def test_dots_bit_exact(n, m, k):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    print(f"q4k dots n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights_q4k(m, k, seed=n * m + k)
    x = synthetic.activations(n, k, seed=n + 2, kind="outlier")
    xq, _, _ = prep_acts(x)
    w = prep_weights(raw, m, k)
    dots = torch.full((n, m, k // 32), -7, dtype=torch.int32, device=gpu_util.DEV)
    q6k.q4k_gemm_dots(xq, n, w, m, k, dots)
    torch.cuda.synchronize()
    xq_ref, _ = oracle.quantize(x)
    np.testing.assert_array_equal(dots.cpu().numpy(), oracle.q4_chunkdots(xq_ref, raw, m))


@pytest.mark.parametrize("n,m,k,kind,ldy", [(64, 256, 512, "normal", None),
                                            (65, 40, 512, "outlier", 48),
                                            (1, 1, 256, "normal", None),
                                            (129, 130, 768, "swiglu", None),
                                            (200, 384, 2048, "outlier", None)])
def test_gemm_every_output(n, m, k, kind, ldy):
    print(f"q4k gemm n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights_q4k(m, k, seed=k + 3 * m)
    x = synthetic.activations(n, k, seed=n + 11, kind=kind)
    xq, da, das = prep_acts(x)
    w = prep_weights(raw, m, k)
    y = run_gemm(xq, da, das, n, w, m, k, ldy)
    if ldy is not None:
        assert np.isnan(y[:, m:]).all()
        y = y[:, :m]
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.q4_gemm(xq_ref, da_ref, raw, m)
    err = np.abs(y.astype(np.float64) - y_ref)
    assert (err <= 1e-3 * t_ref).all(), float((err / np.maximum(t_ref, 1e-300)).max())


def test_gemm_full_size_sampled_and_liveness():
    import q6_int8_prefill_amd as q6k
    n, m, k = 3314, 4096, 11008
    print("q4k full size", flush=True)
    raw = synthetic.weights_q4k(m, k, seed=4)
    import gpu_util
    x = gpu_util.cached_workload("ffn_down_n3314")[1]
    xq, da, das = prep_acts(x)
    w = prep_weights(raw, m, k)
    before = q6k.q4k_launches()
    y = run_gemm(xq, da, das, n, w, m, k)
    assert q6k.q4k_launches() == before + 1
    rows = np.array(sorted(set(np.random.default_rng(2).choice(n, 13, replace=False).tolist())
                           | {0, n - 1}))
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.q4_gemm(xq_ref, da_ref, raw, m)
    err = np.abs(y[rows].astype(np.float64) - y_ref)
    assert (err <= 1e-3 * t_ref).all(), float((err / np.maximum(t_ref, 1e-300)).max())
    assert np.isfinite(y).all()


def test_split_k_pieces():
    """128 output tiles on a 768-slot device are all split along k, here 10 super-blocks over 6
    pieces of unequal length: the integer dots stay bit-exact and the outputs within tolerance,
    checked on a sample of tokens."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, m, k = 1024, 1024, 2560
    print(f"q4k split-k pieces n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights_q4k(m, k, seed=77)
    x = synthetic.activations(n, k, seed=78, kind="outlier")
    xq, da, das = prep_acts(x)
    w = prep_weights(raw, m, k)
    rows = np.array(sorted(set(np.random.default_rng(3).choice(n, 9, replace=False).tolist())
                           | {0, n - 1, n // 2}))
    xq_ref, da_ref = oracle.quantize(x[rows])
    dots = torch.full((n, m, k // 32), -7, dtype=torch.int32, device=gpu_util.DEV)
    q6k.q4k_gemm_dots(xq, n, w, m, k, dots)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dots.cpu().numpy()[rows], oracle.q4_chunkdots(xq_ref, raw, m))
    del dots
    y = run_gemm(xq, da, das, n, w, m, k)
    y_ref, t_ref = oracle.q4_gemm(xq_ref, da_ref, raw, m)
    err = np.abs(y[rows].astype(np.float64) - y_ref)
    assert (err <= 1e-3 * t_ref).all(), float((err / np.maximum(t_ref, 1e-300)).max())
    assert np.isfinite(y).all()


def test_partly_split_grid():
    """1088 output tiles on a 768-slot device: 768 computed whole, the other 320 split along k,
    their pieces reduced from workspace slabs; every output finite (y starts as NaN), sampled
    tokens against the oracle."""
    import q6_int8_prefill_amd as q6k
    n, m, k = 2176, 4096, 2048
    print("q4k partly split grid", flush=True)
    assert q6k.q4k_gemm_workspace(n, m, k) > 0
    raw = synthetic.weights_q4k(m, k, seed=61)
    x = synthetic.activations(n, k, seed=62, kind="outlier")
    xq, da, das = prep_acts(x)
    w = prep_weights(raw, m, k)
    y = run_gemm(xq, da, das, n, w, m, k)
    assert np.isfinite(y).all()
    rows = np.array(sorted(set(np.random.default_rng(5).choice(n, 13, replace=False).tolist())
                           | {0, n - 1}))
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.q4_gemm(xq_ref, da_ref, raw, m)
    err = np.abs(y[rows].astype(np.float64) - y_ref)
    assert (err <= 1e-3 * t_ref).all(), float((err / np.maximum(t_ref, 1e-300)).max())
