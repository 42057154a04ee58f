"""Every configuration under parity with the oracle, every output, in the launch configuration
the benchmark times.

For each workload (Tiny 64x256x512; attn_v 4096x4096 at N=512 and at N=3314 with outlier
channels; ffn_down 4096x11008 at N=3314; one GPU's 8-way share of ffn_down, 3314x512x11008) the
oracle quantizes X and forms the reference output once; then

  * the prepass codes and scales are compared bit for bit (every token and chunk);
  * every output of every layout (0, 1, 2) must satisfy |y - y_ref| <= 1e-3 * sum|terms|;
  * the integer dots are compared bit for bit on two windows of the full-size launch: the first
    full 64-token x 128-row output tile, and the tile holding token n-1 against the last 128
    rows (the per-sub-block dots of the two KSPLIT halves on layouts 0 and 1, "r38 — q6_K
    BT-style raw-byte mma kernel (LANDED)", sec. 2.4; the per-chunk numerators sc*D summed
    over both halves on layout 2).

The 32-layer sweep draws its inputs on the device exactly as the benchmark does; layers 0 and 31
are copied to the host in full and every output of both GEMMs is checked on all three layouts,
the other 30 layers on sampled tokens (all rows), each on one layout in turn.
"""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import untile_da, untile_xq

pytestmark = pytest.mark.gpu
CONFIGS = ["tiny", "attn_v_n512", "attn_v_n3314", "ffn_down_n3314", "ffn_down_shard8"]


def windows(n, m):
    """(tok0, ntok, row0, nrow): the first 64 x 128 output tile, and the tile holding token n-1
    against the last 128 rows (both clipped to the problem)."""
    last = (n - 1) // 64 * 64
    return [(0, min(64, n), 0, min(128, m)),
            (last, n - last, max(0, m - 128), min(128, m))]


def check_dots(xq, da, n, w, layout, m, k, raw, xq_ref):
    import gpu_util
    for tok0, ntok, row0, nrow in windows(n, m):
        rows = gpu_util.raw_rows(raw, m, k, row0, nrow)
        if layout == 2:
            got = gpu_util.chunkdots(xq, da, n, w, 2, m, k, tok0, ntok, row0, nrow)
            want = oracle.chunkdots(xq_ref[tok0:tok0 + ntok], rows, nrow)
        else:
            got = gpu_util.subdots(xq, da, n, w, layout, m, k, tok0, ntok, row0, nrow)
            want = oracle.subdots(xq_ref[tok0:tok0 + ntok], rows, nrow)
        np.testing.assert_array_equal(got, want, err_msg=f"window {(tok0, ntok, row0, nrow)}")


def check_every_output(raw, x, n, m, k, layouts, label, dots=True):
    import gpu_util
    print(f"{label}: oracle (n={n} m={m} k={k}, {oracle.default_threads()} threads)", flush=True)
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    xq, da = gpu_util.quantize(x)
    np.testing.assert_array_equal(untile_xq(xq.cpu().numpy(), n, k)[:n], xq_ref)
    np.testing.assert_array_equal(untile_da(da.cpu().numpy(), n, k)[:n].view(np.uint32),
                                  da_ref.view(np.uint32))
    for layout in layouts:
        print(f"{label}: layout {layout}", flush=True)
        w = gpu_util.expand(raw, m, k, layout)
        y = gpu_util.gemm(xq, da, n, w, layout, m, k)
        assert np.isfinite(y).all()
        ok, worst = gpu_util.within_tolerance(y, y_ref, t_ref)
        print(f"{label}: layout {layout} worst |err|/T = {worst:.3e}", flush=True)
        assert ok, f"layout {layout}: worst |err|/T = {worst}"
        if dots:
            check_dots(xq, da, n, w, layout, m, k, raw, xq_ref)
        del w, y


@pytest.mark.parametrize("name", CONFIGS)
def test_config_every_output(name):
    import gpu_util
    raw, x, n, m, k = gpu_util.cached_workload(name)
    check_every_output(raw, x, n, m, k, (0, 1, 2), name)


def test_tiny_seed_one_is_the_configuration():
    # the Tiny configuration is 64 tokens x 256 rows x k = 512 drawn with seed 1
    spec = synthetic.WORKLOADS["tiny"]
    assert (spec["n"], spec["m"], spec["k"], spec["seed"]) == (64, 256, 512, 1)


def sweep_host_copy(layer, kind):
    import gpu_util
    raw_d, x_d, n, m, k = synthetic.sweep_inputs_torch(layer, kind, gpu_util.DEV)
    raw = raw_d.cpu().numpy().reshape(m, k // 256, 210)
    x = x_d.cpu().numpy()
    return raw, x, n, m, k


@pytest.mark.parametrize("layer", [0, 31])
@pytest.mark.parametrize("kind", ["attn_v", "ffn_down"])
def test_sweep_layer_every_output(layer, kind):
    raw, x, n, m, k = sweep_host_copy(layer, kind)
    check_every_output(raw, x, n, m, k, (0, 1, 2), f"sweep layer {layer} {kind}", dots=False)


def test_sweep_other_layers_sampled():
    """Layers 1..30 of the sweep, both GEMMs, layout l % 3 for layer l: every row for a seeded
    sample of 64 tokens per GEMM (first, last and 62 random ones)."""
    import gpu_util
    for layer in range(1, synthetic.SWEEP_LAYERS - 1):
        layout = layer % 3
        for kind in ("attn_v", "ffn_down"):
            raw_d, x_d, n, m, k = synthetic.sweep_inputs_torch(layer, kind, gpu_util.DEV)
            print(f"sweep layer {layer} {kind} layout {layout}", flush=True)
            xq, da = gpu_util.quantize_device(x_d)
            w = gpu_util.expand_device(raw_d, m, k, layout)
            y = gpu_util.gemm(xq, da, n, w, layout, m, k)
            rng = np.random.default_rng(layer * 2 + (kind == "ffn_down"))
            rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 62, replace=False)]))
            xs = x_d[rows].cpu().numpy()
            raw = raw_d.cpu().numpy()
            xq_ref, da_ref = oracle.quantize(xs)
            y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
            ok, worst = gpu_util.within_tolerance(y[rows], y_ref, t_ref)
            assert ok, f"layer {layer} {kind} layout {layout}: worst |err|/T = {worst}"
            assert np.isfinite(y).all()
            # the sampled tokens' codes and scales are the prepass's, bit for bit
            np.testing.assert_array_equal(untile_xq(xq.cpu().numpy(), n, k)[rows], xq_ref)
            np.testing.assert_array_equal(untile_da(da.cpu().numpy(), n, k)[rows].view(np.uint32),
                                          da_ref.view(np.uint32))
            del raw_d, x_d, xq, da, w, y
