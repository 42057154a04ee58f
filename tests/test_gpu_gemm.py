"""GPU parity of q6k_gemm / q6k_gemm_subdots / q6k_gemm_chunkdots against the oracle.

  * per-sub-block int32 dots (layouts 0 and 1): bit-exact (the KSPLIT=2 halves of "r38 — q6_K
    BT-style raw-byte mma kernel (LANDED)", sec. 2.4), exported by the same kernel source;
  * per-chunk numerators sc*D summed over both halves (layout 2): bit-exact, exported by the same
    kernel source after its float reconstruction of the two digit products;
  * outputs: |y - y_ref| <= 1e-3 * sum|terms| per element, for every element at sizes the
    oracle runs in seconds and on sampled tokens (all rows) at the full workload sizes, in the
    launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu
LAYOUTS = [0, 1, 2]
SPLIT_LAYOUTS = [0, 1]  # layouts whose kernel keeps the two 16-k halves apart


def prepare(x, raw, m, layout):
    import gpu_util
    n, k = x.shape
    xq, da = gpu_util.quantize(x)
    w = gpu_util.expand(raw, m, k, layout)
    return xq, da, w


@pytest.mark.parametrize("layout", SPLIT_LAYOUTS)
@pytest.mark.parametrize("n,m,k", [(64, 256, 512), (65, 40, 512), (1, 1, 256), (129, 130, 768),
                                   (33, 200, 1024)])
def test_subdots_bit_exact(layout, n, m, k):
    import gpu_util
    print(f"subdots layout={layout} n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights(m, k, seed=n + m + k, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=n * m, kind="outlier")
    xq, da, w = prepare(x, raw, m, layout)
    got = gpu_util.subdots(xq, da, n, w, layout, m, k)
    xq_ref, _ = oracle.quantize(x)
    np.testing.assert_array_equal(got, oracle.subdots(xq_ref, raw, m))


def test_subdots_extreme_magnitude():
    # D = 16 * 127 * (-32) = -65024, the largest |D|: all codes 0 against xq = 127
    import gpu_util
    n, m, k = 32, 32, 256
    raw = np.zeros((m, 1, 210), np.uint8)
    raw[:, 0, 208:210] = (0x00, 0x3C)
    x = np.full((n, k), 5.0, np.float32)
    for layout in SPLIT_LAYOUTS:
        xq, da, w = prepare(x, raw, m, layout)
        got = gpu_util.subdots(xq, da, n, w, layout, m, k)
        assert (got == -65024).all()
        y = gpu_util.gemm(xq, da, n, w, layout, m, k)
        xq_ref, da_ref = oracle.quantize(x)
        y_ref, _ = oracle.gemm(xq_ref, da_ref, raw, m)
        np.testing.assert_array_equal(y, y_ref.astype(np.float32))


@pytest.mark.parametrize("n,m,k", [(64, 256, 512), (65, 40, 512), (1, 1, 256), (129, 130, 768),
                                   (33, 200, 1024), (160, 384, 2048)])
def test_chunkdots_bit_exact(n, m, k):
    import gpu_util
    print(f"chunkdots layout=2 n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights(m, k, seed=n + m + k, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=n * m, kind="outlier")
    xq, da, w = prepare(x, raw, m, 2)
    got = gpu_util.chunkdots(xq, da, n, w, 2, m, k)
    xq_ref, _ = oracle.quantize(x)
    np.testing.assert_array_equal(got, oracle.chunkdots(xq_ref, raw, m))


@pytest.mark.parametrize("sc_byte,code_byte,want", [(0x80, 0x00, 32 * 127 * 4096),
                                                    (0x7F, 0x00, -32 * 127 * 127 * 32),
                                                    (0x80, 0xFF, None)])
def test_chunkdots_extreme_magnitude(sc_byte, code_byte, want):
    # |E| up to 32 * 127 * 4096 (sc = -128, all codes 0, xq = 127): the digit products and their
    # float reconstruction must stay exact at the ends of the range
    import gpu_util
    n, m, k = 32, 32, 256
    raw = np.zeros((m, 1, 210), np.uint8)
    raw[:, 0, :192] = code_byte
    raw[:, 0, 192:208] = sc_byte
    raw[:, 0, 208:210] = (0x00, 0x3C)
    x = np.full((n, k), 5.0, np.float32)
    x[1::2] *= -1
    xq, da, w = prepare(x, raw, m, 2)
    got = gpu_util.chunkdots(xq, da, n, w, 2, m, k)
    xq_ref, da_ref = oracle.quantize(x)
    ref = oracle.chunkdots(xq_ref, raw, m)
    np.testing.assert_array_equal(got, ref)
    if want is not None:
        assert (np.abs(ref) == abs(want)).all()
    y = gpu_util.gemm(xq, da, n, w, 2, m, k)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y, y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n,m,k,kind,wide", [(64, 256, 512, "normal", False),
                                             (65, 40, 512, "outlier", True),
                                             (1, 1, 256, "normal", True),
                                             (129, 130, 768, "swiglu", True),
                                             (200, 384, 2048, "outlier", False)])
def test_gemm_small_every_output(layout, n, m, k, kind, wide):
    import gpu_util
    print(f"gemm layout={layout} n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights(m, k, seed=k + 3 * m, sc_lo=-128 if wide else -32,
                            sc_hi=127 if wide else 31)
    x = synthetic.activations(n, k, seed=n + 11, kind=kind)
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y, y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_sparse_and_zero_inputs(layout):
    # degenerate inputs: a single nonzero activation per token, an all-zero token, zero d
    import gpu_util
    n, m, k = 40, 72, 512
    raw = synthetic.weights(m, k, seed=77, sc_lo=-128, sc_hi=127)
    raw.reshape(m, 2, 210)[5, 1, 208:210] = 0  # d = 0 for one super-block
    x = np.zeros((n, k), np.float32)
    for t in range(n - 1):
        x[t, (37 * t) % k] = (t - 20) * 0.37 + 0.01
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y, y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"
    assert (y[n - 1] == 0).all()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_leading_dimension_untouched_tail(layout):
    import gpu_util
    n, m, k, ldy = 70, 50, 512, 64
    raw = synthetic.weights(m, k, seed=5)
    x = synthetic.activations(n, k, seed=5)
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k, ldy=ldy)
    assert np.isnan(y[:, m:]).all()
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[:, :m], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"


def test_liveness_counters_tick_per_layout():
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, m, k = 32, 32, 256
    raw = synthetic.weights(m, k, seed=1)
    x = synthetic.activations(n, k, seed=1)
    for layout in LAYOUTS:
        xq, da, w = prepare(x, raw, m, layout)
        before = q6k.q6k_stats()
        gpu_util.gemm(xq, da, n, w, layout, m, k)
        after = q6k.q6k_stats()
        for other in LAYOUTS:
            assert after[other] == before[other] + (1 if other == layout else 0)


def sampled_tokens(n, count, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(n, size=count - 3, replace=False).tolist()) | {0, n - 1, n // 2}
    return np.array(sorted(idx))


@pytest.mark.parametrize("name", ["attn_v_n512", "attn_v_n3314", "ffn_down_n3314", "ffn_down_shard8"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_full_size_sampled(name, layout):
    """Full workload shape, the benchmark's launch configuration; every row of W checked for a
    sample of tokens (first, middle, last and random ones)."""
    import gpu_util
    raw, x, n, m, k = gpu_util.cached_workload(name)
    print(f"full-size gemm {name} layout={layout}", flush=True)
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    rows = sampled_tokens(n, 24, seed=n + layout)
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[rows], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"
    assert np.isfinite(y).all()


@pytest.mark.parametrize("name", ["attn_v_n3314", "ffn_down_n3314"])
def test_folded_rounding_no_worse_than_split(name):
    """Layout 2 combines the two 16-k halves of a chunk before any float rounding, but only after
    each half's own int8 scale has been applied exactly in integers.  The pages warn that fusing
    the halves before their scales breaks the 1e-3 gate ("r38 — q6_K BT-style raw-byte mma kernel",
    sec. 3.3, item 2); this checks that the folded form's error against the f64 reference stays
    within the two-halves form's on the same inputs (measured: 3-5 times smaller)."""
    import gpu_util
    raw, x, n, m, k = gpu_util.cached_workload(name)
    rows = sampled_tokens(n, 16, seed=7)
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    worst = {}
    for layout in (1, 2):
        xq, da, w = prepare(x, raw, m, layout)
        y = gpu_util.gemm(xq, da, n, w, layout, m, k)[rows].astype(np.float64)
        worst[layout] = float((np.abs(y - y_ref) / np.maximum(t_ref, 1e-300)).max())
    print(f"{name}: worst |err|/T layout 1 {worst[1]:.3e}, layout 2 {worst[2]:.3e}", flush=True)
    assert worst[2] <= 2 * worst[1]
    assert worst[2] < 1e-6


def test_empty_problems_launch_nothing():
    # n = 0 or m = 0 is a no-op that leaves the output untouched, for every layout
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    k = 256
    raw = synthetic.weights(8, k, seed=1)
    x = synthetic.activations(8, k, seed=1)
    for layout in LAYOUTS:
        xq, da, w = prepare(x, raw, 8, layout)
        before = q6k.q6k_stats()
        y = torch.full((8, 8), 3.0, dtype=torch.float32, device=gpu_util.DEV)
        q6k.q6k_gemm(xq, da, 0, w, layout, 8, k, y, ldy=8)
        q6k.q6k_gemm(xq, da, 8, w, layout, 0, k, y, ldy=8)
        torch.cuda.synchronize()
        assert (y == 3.0).all().item()
        assert q6k.q6k_stats() == before


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_long_k(layout):
    # 64 super-blocks per row (on layout 2 these few tiles are split along k into many pieces)
    import gpu_util
    n, m, k = 33, 40, 16384
    print(f"long k layout={layout}", flush=True)
    raw = synthetic.weights(m, k, seed=21, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=22, kind="outlier")
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    xq_ref, da_ref = oracle.quantize(x)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y, y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_zero_scales_give_zero(layout):
    # d = 0 on every super-block: every term is zero, so y must be exactly 0 (T = 0)
    import gpu_util
    n, m, k = 40, 72, 512
    raw = synthetic.weights(m, k, seed=31)
    raw.reshape(m, k // 256, 210)[:, :, 208:210] = 0
    x = synthetic.activations(n, k, seed=31)
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    assert (y == 0).all()


@pytest.mark.parametrize("n,m,k", [(1024, 1024, 2560), (256, 256, 25600)])
def test_folded_split_k_pieces(n, m, k):
    """Layout 2 deals its 64-token x 128-row output tiles out in rounds of one per workgroup slot
    and splits the tiles of a partial last round along k into pieces of whole super-blocks, whose
    partial sums go to workspace slabs that a second kernel adds into y in piece order.  On a
    256-CU device these shapes give
    pieces of unequal length (10 super-blocks over 4 pieces; 100 over 64).  The integer numerators
    must stay bit-exact and the outputs within tolerance, checked on a sample of tokens."""
    import gpu_util
    print(f"split-k pieces n={n} m={m} k={k}", flush=True)
    raw = synthetic.weights(m, k, seed=k + m, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=n + 5, kind="outlier")
    xq, da, w = prepare(x, raw, m, 2)
    rows = sampled_tokens(n, 12, seed=k)
    xq_ref, da_ref = oracle.quantize(x[rows])
    dots = gpu_util.chunkdots(xq, da, n, w, 2, m, k)[rows]
    np.testing.assert_array_equal(dots, oracle.chunkdots(xq_ref, raw, m))
    del dots
    y = gpu_util.gemm(xq, da, n, w, 2, m, k)
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[rows], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"
    assert np.isfinite(y).all()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ldy", [4094, 4097, 4100])
def test_gemm_whole_tiles_ragged_rows(layout, ldy):
    """Enough tiles (1664) that most are computed whole, with m not a multiple of 4 and leading
    dimensions that do (4100) and do not (4094, 4097) allow 16-byte stores: every store path of
    the epilogues (vector, scalar, partial last row group) and of the split pieces' reduction,
    with the columns past m untouched."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, m, k = 3314, 4094, 2048
    print(f"whole tiles layout={layout} ldy={ldy}", flush=True)
    assert q6k.q6k_gemm_workspace(n, m, k, layout) > 0  # the last round is split
    raw = synthetic.weights(m, k, seed=ldy, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=ldy + 1, kind="outlier")
    xq, da, w = prepare(x, raw, m, layout)
    y = torch.full((n, ldy), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q6k_gemm(xq, da, n, w, layout, m, k, y, ldy=ldy)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.isnan(y[:, m:]).all()
    rows = sampled_tokens(n, 16, seed=ldy)
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[rows, :m], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"
    assert np.isfinite(y[:, :m]).all()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemm_partly_split_grid(layout):
    """2176 x 4096 outputs: 1088 tiles of 64 x 128 (544 of 128 x 128), more than one round of
    workgroup slots with a short last round, so some tiles are computed whole and the rest are
    split along k into workspace slabs that a second kernel adds up; the reduction must hit
    exactly the split tiles of the GEMM's own tile order (y starts as NaN: every output is checked
    finite, sampled tokens against the oracle)."""
    import gpu_util
    import q6_int8_prefill_amd as q6k
    n, m, k = 2176, 4096, 2048
    print(f"partly split grid layout={layout}", flush=True)
    assert q6k.q6k_gemm_workspace(n, m, k, layout) > 0
    raw = synthetic.weights(m, k, seed=55, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=56, kind="outlier")
    xq, da, w = prepare(x, raw, m, layout)
    y = gpu_util.gemm(xq, da, n, w, layout, m, k)
    assert np.isfinite(y).all()
    rows = sampled_tokens(n, 24, seed=57)
    xq_ref, da_ref = oracle.quantize(x[rows])
    y_ref, t_ref = oracle.gemm(xq_ref, da_ref, raw, m)
    ok, worst = gpu_util.within_tolerance(y[rows], y_ref, t_ref)
    assert ok, f"worst |err|/T = {worst}"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_repeatability_whole_and_split_tiles(layout):
    """Every output is bit-for-bit repeatable: tiles computed whole by construction, tiles split
    along k because their pieces' slabs are added in piece order by one thread per output.  The
    second problem is all split tiles (a workspace is needed); the first, 6 x CUs tiles of 64 x
    128, fills whole rounds of 2 and of 3 workgroups per CU (3072 tokens on 256 CUs)."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for n, m, k, split in ((12 * cus, 4096, 512, False), (200, 384, 2048, True)):
        print(f"repeatability layout={layout} n={n} m={m} k={k}", flush=True)
        assert (q6k.q6k_gemm_workspace(n, m, k, layout) > 0) == split
        raw = synthetic.weights(m, k, seed=n + 9, sc_lo=-128, sc_hi=127)
        x = synthetic.activations(n, k, seed=n + 10, kind="outlier")
        xq, da = gpu_util.quantize(x)
        w = gpu_util.expand(raw, m, k, layout)
        runs = [gpu_util.gemm(xq, da, n, w, layout, m, k) for _ in range(3)]
        assert np.isfinite(runs[0]).all()
        for r in runs[1:]:
            np.testing.assert_array_equal(r.view(np.uint32), runs[0].view(np.uint32))


def test_workspace_rules_and_size():
    """Through the C ABI: the workspace q6k_gemm_workspace reports is one 32 KiB slab per piece of
    a split tile (at most one per workgroup slot); a call that needs one rejects a missing,
    misaligned or short workspace before launching anything, and a caller's workspace full of NaN
    gives the same y, bit for bit, as one the binding allocates.  The same for q4k_gemm."""
    import ctypes
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    from q6_int8_prefill_amd import _lib
    L = _lib._lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n, m, k = 200, 384, 2048
    print(f"workspace rules n={n} m={m} k={k}", flush=True)
    for layout, slots in ((2, 2 * cus), (1, 3 * cus), (0, 3 * cus)):
        tiles = (-(-n // 128) * 128 // 64) * (-(-m // 128))   # 64 x 128 output tiles
        pieces = min(slots // tiles, k // 256)                  # every tile split, whole super-blocks
        assert q6k.q6k_gemm_workspace(n, m, k, layout) == tiles * pieces * 32768, layout
    assert q6k.q4k_gemm_workspace(n, m, k) == q6k.q6k_gemm_workspace(n, m, k, 1)
    assert q6k.q6k_gemm_workspace(12 * cus, 4096, 512, 2) == 0  # whole rounds only
    raw = synthetic.weights(m, k, seed=71, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=72, kind="outlier")
    xq, da = gpu_util.quantize(x)
    for layout in (2, 1):
        need = q6k.q6k_gemm_workspace(n, m, k, layout)
        w = gpu_util.expand(raw, m, k, layout)
        y = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
        ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)

        def call(p, nb):
            return L.q6k_gemm(xq.data_ptr(), xq.numel(), da.data_ptr(), da.numel() * 4, n,
                              w.data_ptr(), w.numel(), layout, m, k, y.data_ptr(), y.numel() * 4,
                              m, p, nb, torch.cuda.current_stream().cuda_stream)
        assert call(None, 0) == -1
        assert call(ws.data_ptr() + 4, need) == -3
        assert call(ws.data_ptr(), need - 1) == -4
        torch.cuda.synchronize()
        assert torch.isnan(y).all()                            # nothing ran
        assert call(ws.data_ptr(), need) == 0
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        ref = gpu_util.gemm(xq, da, n, w, layout, m, k)
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    # q4k_gemm: the same rules
    raw4 = synthetic.weights_q4k(m, k, seed=73)
    w4 = torch.empty(q6k.q4k_weight_bytes(m, k), dtype=torch.uint8, device=gpu_util.DEV)
    q6k.q4k_expand_weights(torch.from_numpy(np.ascontiguousarray(raw4).reshape(-1)).to(
        gpu_util.DEV), m, k, w4)
    das = torch.empty_like(da)
    q6k.q4k_act_sums(xq, da, n, k, das)
    need = q6k.q4k_gemm_workspace(n, m, k)
    y = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    ws = torch.full((need // 4 + 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)

    def call4(p, nb):
        return L.q4k_gemm(xq.data_ptr(), xq.numel(), da.data_ptr(), da.numel() * 4,
                          das.data_ptr(), das.numel() * 4, n, w4.data_ptr(), w4.numel(), m, k,
                          y.data_ptr(), y.numel() * 4, m, p, nb,
                          torch.cuda.current_stream().cuda_stream)
    assert call4(None, 0) == -1
    assert call4(ws.data_ptr() + 4, need) == -3
    assert call4(ws.data_ptr(), need - 1) == -4
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
    assert call4(ws.data_ptr(), need) == 0
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    y2 = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q4k_gemm(xq, da, das, n, w4, m, k, y2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.view(np.uint32), y2.cpu().numpy().view(np.uint32))


def test_claimed_tail_workspace_size_and_garbage_counter():
    """Layout 2 behind whole rounds hands its graded tail pieces out through a claim counter after
    the slabs: q6k_gemm_workspace reports the slabs plus 256 bytes, and a caller workspace full of
    garbage (NaN, so the counter's word too), then the same workspace again, give y bit for bit
    equal to a binding-allocated one -- the launch sets the counter itself."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    from q6_int8_prefill_amd import _lib
    L = _lib._lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slots = 2 * cus
    gx = 2 * ((9 * slots) // (8 * 32))          # about 2.25 rounds of 32 row quads
    n, m, k = gx * 64 - 104, 4096, 2048         # 2200 x 4096 x 2048 on 256 CUs
    print(f"claimed tail n={n} m={m} k={k}", flush=True)
    tiles = (-(-n // 128) * 2) * (m // 128)
    rem = tiles % slots
    assert tiles >= 2 * slots and rem
    pieces = min(slots // rem, k // 256)
    need = q6k.q6k_gemm_workspace(n, m, k, 2)
    assert need == rem * pieces * 32768 + 256
    raw = synthetic.weights(m, k, seed=81)
    x = synthetic.activations(n, k, seed=82)
    xq, da = gpu_util.quantize(x)
    w = gpu_util.expand(raw, m, k, 2)
    ref = gpu_util.gemm(xq, da, n, w, 2, m, k)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    for rep in range(2):
        y = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
        st = L.q6k_gemm(xq.data_ptr(), xq.numel(), da.data_ptr(), da.numel() * 4, n,
                        w.data_ptr(), w.numel(), 2, m, k, y.data_ptr(), y.numel() * 4, m,
                        ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_claimed_tails_on_two_streams():
    """Two layout-2 GEMMs with claimed tails in flight at once on two streams (default priority),
    each with its own workspace, give their one-at-a-time results bit for bit, three times over:
    each launch's claims come from its own workspace's counter."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gx = 2 * ((9 * 2 * cus) // (8 * 32))
    n, m, k = gx * 64 - 104, 4096, 2048
    print(f"two streams n={n} m={m} k={k}", flush=True)
    runs = []
    for seed in (91, 93):
        raw = synthetic.weights(m, k, seed=seed)
        xq, da = gpu_util.quantize(synthetic.activations(n, k, seed=seed + 1))
        w = gpu_util.expand(raw, m, k, 2)
        ws = torch.empty(q6k.q6k_gemm_workspace(n, m, k, 2), dtype=torch.uint8,
                         device=gpu_util.DEV)
        assert ws.numel() % 32768 == 256                    # the tail is claimed
        runs.append((xq, da, w, ws, gpu_util.gemm(xq, da, n, w, 2, m, k)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        ys = []
        for (xq, da, w, ws, _), st in zip(runs, streams):
            y = torch.full((n, m), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
            ys.append(y)
            with torch.cuda.stream(st):
                q6k.q6k_gemm(xq, da, n, w, 2, m, k, y, workspace=ws)
        torch.cuda.synchronize()
        for y, (_, _, _, _, ref) in zip(ys, runs):
            np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_packed_layout_equals_expanded_bit_for_bit():
    """Layout 0 stages 4 (q - 32) and d*sc, so its MFMAs yield 4 D, every rescale product and
    accumulator is exactly 4 times layout 1's (scaling by a power of two commutes with rounding),
    and its store multiplies by 1/4: on whole tiles (no split along k) the two layouts must agree
    bit for bit.  768 tiles of 64 x 128 fill the grid of 3 workgroups per CU without a split on
    any device of 256 to 511 CUs."""
    import gpu_util
    n, m, k = 2048, 3072, 512
    raw = synthetic.weights(m, k, seed=71, sc_lo=-128, sc_hi=127)
    x = synthetic.activations(n, k, seed=72, kind="outlier")
    xq, da = gpu_util.quantize(x)
    y0 = gpu_util.gemm(xq, da, n, gpu_util.expand(raw, m, k, 0), 0, m, k)
    y1 = gpu_util.gemm(xq, da, n, gpu_util.expand(raw, m, k, 1), 1, m, k)
    np.testing.assert_array_equal(y0.view(np.uint32), y1.view(np.uint32))
