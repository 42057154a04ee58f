"""The hot path recorded in a HIP graph (torch.cuda.graph) and replayed: the prepass and the GEMM
(every layout) with its split-k last round (pieces into workspace slabs, then the reducing
kernel) launch only kernels on the caller's stream (no memset nodes), so a captured step replays
to the eager results.  Each replay follows eager work of the program's own that clobbers every
output and the workspace, and is checked: codes, scales and outputs bit for bit against the eager
run, codes and scales against the oracle, and outputs against the oracle within the output
tolerance."""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import untile_da, untile_xq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [2, 1, 0])
@pytest.mark.parametrize("n,m,k", [(2176, 4096, 2048), (2200, 4096, 2048), (200, 384, 2048)])
def test_captured_step_replays(n, m, k, layout):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    print(f"graph replay layout={layout} n={n} m={m} k={k}", flush=True)
    dev = gpu_util.DEV
    raw = synthetic.weights(m, k, seed=n + 5, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=n + 6, kind="outlier")
    w = gpu_util.expand(raw, m, k, layout)
    xg = torch.from_numpy(x).to(dev)
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.zeros(xb, dtype=torch.uint8, device=dev)
    da = torch.zeros(db // 4, dtype=torch.float32, device=dev)
    y = torch.zeros((n, m), dtype=torch.float32, device=dev)
    need = q6k.q6k_gemm_workspace(n, m, k, layout)
    assert need > 0  # a split-k last round
    ws = torch.zeros(need // 4, dtype=torch.float32, device=dev)

    def step():
        q6k.q6k_quantize_act(xg, xq, da)
        q6k.q6k_gemm(xq, da, n, w, layout, m, k, y, workspace=ws)

    # eager reference of the same calls
    step()
    torch.cuda.synchronize()
    xq_e, da_e, y_e = xq.clone(), da.clone(), y.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    xq_ref, da_ref = oracle.quantize(x)
    rows = np.array(sorted(set(np.random.default_rng(n).choice(n, min(n, 12), replace=False).tolist())
                           | {0, n - 1}))
    y_ref, t_ref = oracle.gemm(xq_ref[rows], da_ref[rows], raw, m)
    for rep in range(3):
        # the program's own eager work between replays: clobber every output buffer
        xq.fill_(0xA5)
        da.fill_(float("nan"))
        y.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xq, xq_e), rep
        assert torch.equal(da.view(torch.int32), da_e.view(torch.int32)), rep
        assert torch.equal(y.view(torch.int32), y_e.view(torch.int32)), rep
        got = y.cpu().numpy()
        ok, worst = gpu_util.within_tolerance(got[rows], y_ref, t_ref)
        assert ok, f"replay {rep}: worst |err|/T = {worst}"
    np.testing.assert_array_equal(untile_xq(xq.cpu().numpy(), n, k)[:n], xq_ref)
    np.testing.assert_array_equal(untile_da(da.cpu().numpy(), n, k)[:n].view(np.uint32),
                                  da_ref.view(np.uint32))


def test_captured_q4k_step_replays():
    """The q4_K step (its one-pass prepass, then the GEMM with a split-k last round) captured and
    replayed after eager clobbering, as above; here the binding allocates the GEMM's workspace
    inside the capture (from the graph's memory pool)."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, m, k = 200, 384, 2048
    print(f"graph replay q4k n={n} m={m} k={k}", flush=True)
    dev = gpu_util.DEV
    raw = synthetic.weights_q4k(m, k, seed=41)
    x = synthetic.activations(n, k, seed=42, kind="outlier")
    w = torch.empty(q6k.q4k_weight_bytes(m, k), dtype=torch.uint8, device=dev)
    q6k.q4k_expand_weights(torch.from_numpy(np.ascontiguousarray(raw).reshape(-1)).to(dev), m, k, w)
    xg = torch.from_numpy(x).to(dev)
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.zeros(xb, dtype=torch.uint8, device=dev)
    da = torch.zeros(db // 4, dtype=torch.float32, device=dev)
    das = torch.zeros(db // 4, dtype=torch.float32, device=dev)
    y = torch.zeros((n, m), dtype=torch.float32, device=dev)

    def step():
        q6k.q4k_quantize_act(xg, xq, da, das)
        q6k.q4k_gemm(xq, da, das, n, w, m, k, y)

    step()
    torch.cuda.synchronize()
    xq_e, da_e, das_e, y_e = xq.clone(), da.clone(), das.clone(), y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.q4_gemm(xq_ref, da_ref, raw, m)
    for rep in range(3):
        xq.fill_(0xA5)
        da.fill_(float("nan"))
        das.fill_(float("nan"))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xq, xq_e), rep
        assert torch.equal(da.view(torch.int32), da_e.view(torch.int32)), rep
        assert torch.equal(das.view(torch.int32), das_e.view(torch.int32)), rep
        assert torch.equal(y.view(torch.int32), y_e.view(torch.int32)), rep
        got = y.cpu().numpy()
        ok, worst = gpu_util.within_tolerance(got, y_ref, t_ref)
        assert ok, f"replay {rep}: worst |err|/T = {worst}"
