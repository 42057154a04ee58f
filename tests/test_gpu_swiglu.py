"""GPU parity of the fused SwiGLU -> int8 producer (q6k_swiglu_quantize_act) against the oracle.

  * h = up * silu(gate) as the producer forms it in f32 (exported by q6k_swiglu_f32 from the same
    device function) agrees with the oracle's f64 product to a few f32 ulp;
  * the codes and da are bit-exact with the oracle's quantization of that f32 h (the decision is
    taken in the same precision on both sides), and byte-identical to q6k_quantize_act on it;
  * a GEMM fed by the fused producer meets the output tolerance against the oracle.
"""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import untile_da, untile_xq

pytestmark = pytest.mark.gpu


def gpu_h(gate, up):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    g = torch.from_numpy(gate).to(gpu_util.DEV)
    u = torch.from_numpy(up).to(gpu_util.DEV)
    h = torch.full(gate.shape, float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q6k_swiglu_f32(g, u, h)
    torch.cuda.synchronize()
    return h.cpu().numpy()


def fused(gate, up, ld=None):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, k = gate.shape
    ld = k if ld is None else ld
    gp = np.zeros((n, ld), np.float32)
    up_ = np.zeros((n, ld), np.float32)
    gp[:, :k] = gate
    up_[:, :k] = up
    g = torch.from_numpy(gp).to(gpu_util.DEV)[:, :k]
    u = torch.from_numpy(up_).to(gpu_util.DEV)[:, :k]
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.full((xb,), 0xA5, dtype=torch.uint8, device=gpu_util.DEV)
    da = torch.full((db // 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q6k_swiglu_quantize_act(g, u, xq, da, n=n, k=k)
    return xq, da


def ulp_f32(v):
    v = np.abs(v.astype(np.float32))
    return np.spacing(np.maximum(v, np.float32(np.finfo(np.float32).tiny)))


def check(gate, up, ld=None):
    n, k = gate.shape
    h = gpu_h(gate, up)
    h64 = oracle.swiglu(gate, up)
    err = np.abs(h.astype(np.float64) - h64)
    # a few ulp; below ~1e-30 * |up| (silu of gates under about -70, where e^-g nears the f32
    # range) the f32 product may flush towards zero
    assert (err <= 4 * ulp_f32(h64) + 1e-30 * np.abs(up)).all(), float((err / ulp_f32(h64)).max())
    xq, da = fused(gate, up, ld)
    xq_ref, da_ref = oracle.quantize(h)
    got_q = untile_xq(xq.cpu().numpy(), n, k)
    got_d = untile_da(da.cpu().numpy(), n, k)
    np.testing.assert_array_equal(got_q[:n], xq_ref)
    np.testing.assert_array_equal(got_d[:n].view(np.uint32), da_ref.view(np.uint32))
    assert (got_q[n:] == 0).all() and (got_d[n:] == 0).all()
    return xq, da, h


@pytest.mark.parametrize("n,k,ld", [(64, 512, None), (65, 256, 260), (1, 256, None), (200, 1024, None)])
def test_fused_small(n, k, ld):
    print(f"swiglu n={n} k={k} ld={ld}", flush=True)
    gate, up = synthetic.swiglu_inputs(n, k, seed=n + k)
    check(gate, up, ld)


def test_fused_extremes():
    # very negative gates (e^-g overflows: signed zeros), very positive gates (silu(g) = g),
    # zero rows, a single nonzero per chunk
    n, k = 40, 512
    gate = np.zeros((n, k), np.float32)
    up = np.ones((n, k), np.float32)
    gate[0] = -100.0
    gate[1] = 100.0
    gate[2] = np.linspace(-90, 90, k, dtype=np.float32)
    up[3] = 0.0
    gate[4, ::32] = 3.0
    up[5] = -np.float32(1e30)
    gate[5] = 5.0
    check(gate, up)


def test_fused_matches_unfused_prepass():
    import torch
    import gpu_util
    n, k = 96, 768
    gate, up = synthetic.swiglu_inputs(n, k, seed=9)
    xq, da, h = check(gate, up)
    xq2, da2 = gpu_util.quantize(h)
    assert torch.equal(xq, xq2) and torch.equal(da.view(torch.int32), da2.view(torch.int32))


def test_fused_full_size_then_gemm():
    """ffn_down shape: codes of sampled tokens bit-exact, then the layout-2 GEMM on the fused
    producer's output within tolerance of the oracle."""
    import gpu_util
    n, m, k = 3314, 4096, 11008
    raw = gpu_util.cached_workload("ffn_down_n3314")[0]
    gate, up = synthetic.swiglu_inputs(n, k, seed=4)
    print("swiglu full size", flush=True)
    xq, da = fused(gate, up)
    rows = np.array(sorted(set(np.random.default_rng(1).choice(n, 13, replace=False).tolist())
                           | {0, n - 1}))
    h_rows = gpu_h(gate[rows], up[rows])
    xq_ref, da_ref = oracle.quantize(h_rows)
    got_q = untile_xq(xq.cpu().numpy(), n, k)[rows]
    got_d = untile_da(da.cpu().numpy(), n, k)[rows]
    np.testing.assert_array_equal(got_q, xq_ref)
    np.testing.assert_array_equal(got_d.view(np.uint32), da_ref.view(np.uint32))
    w = gpu_util.expand(raw, m, k, 2)
    y = gpu_util.gemm(xq, da, n, w, 2, m, k)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[rows], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"
