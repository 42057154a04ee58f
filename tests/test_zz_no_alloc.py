"""q6k_gemm_noalloc (the split-k workspace in the library's static device array) against q6k_gemm
with a caller workspace, through the C ABI: bit for bit on three calls in a row, each smaller
than the one before -- 2200 x 4096 x 2048 (whole rounds, then a split tail that layout 2 claims
through the counter after the slabs), 512 x 4096 x 4096 (every tile split, on layouts 0/1 into
768 pieces: the whole array), and a small problem that must not see the earlier calls' slabs."""
import ctypes

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [2, 1, 0])
def test_noalloc_equals_workspace_call(layout):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    from q6_int8_prefill_amd import _lib
    L = _lib._lib
    for n, m, k in ((2200, 4096, 2048), (512, 4096, 4096), (200, 384, 2048)):
        print(f"noalloc layout={layout} n={n} m={m} k={k}", flush=True)
        need = q6k.q6k_gemm_workspace(n, m, k, layout)
        assert 0 < need <= 768 * 32768 + 256
        raw = synthetic.weights(m, k, seed=n + k + layout, sc_lo=-128, sc_hi=127)
        x = synthetic.activations(n, k, seed=n + 3, kind="outlier")
        xq, da = gpu_util.quantize(x)
        w = gpu_util.expand(raw, m, k, layout)
        ref = gpu_util.gemm(xq, da, n, w, layout, m, k)          # q6k_gemm, caller workspace
        y = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
        st = L.q6k_gemm_noalloc(xq.data_ptr(), xq.numel(), da.data_ptr(), da.numel() * 4, n,
                                w.data_ptr(), w.numel(), layout, m, k, y.data_ptr(),
                                y.numel() * 4, m, torch.cuda.current_stream().cuda_stream)
        assert st == 0, q6k.q6k_strerror(st)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
