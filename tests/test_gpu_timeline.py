"""The workgroup-timeline build (libq6k_timeline.so) on the GPU: its GEMMs give the product
library's outputs bit for bit, and its records show the work split the host planned -- every
output tile exactly once, either whole over all of k or as split-k pieces whose super-block
ranges partition k, one record per workgroup of the grid, workgroup b on XCD (b + c) mod 8 for
one c per launch (the placement the XCD-aware tile order relies on: the workgroups with one value
of b mod 8 share an XCD; c carries over from the previous launch's round robin), and plausible
times and clocks."""
import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

N, M, K = 2200, 4096, 2048  # 36 x 32 tiles: one or two whole rounds and a split remainder


def _check_records(d, n, m, k, has_pieces):
    # 64-token x 128-row tiles over the tokens padded to 128 and the rows padded to 128
    gx, gy, nsb = 2 * -(-n // 128), -(-m // 128), k // 256
    nwg = len(d["wg"])
    assert list(d["wg"]) == list(range(nwg))          # every workgroup of the grid wrote one
    c = (d["xcd"][0] - d["wg"][0]) % 8
    assert ((d["wg"] + c) % 8 == d["xcd"]).all()
    assert (d["end"] > d["start"]).all() and (d["cycles"] > 0).all()
    ghz = d["cycles"] / ((d["end"] - d["start"]) * 1e3)
    assert ((ghz > 0.5) & (ghz < 3.0)).all(), (ghz.min(), ghz.max())
    cover = {}
    for i in range(nwg):
        key = (int(d["bx"][i]), int(d["by"][i]))
        assert 0 <= key[0] < gx and 0 <= key[1] < gy
        cover.setdefault(key, []).append((int(d["s0"][i]), int(d["s1"][i]), bool(d["split"][i])))
    assert len(cover) == gx * gy
    pieces = 0
    for key, parts in cover.items():
        parts.sort()
        if len(parts) == 1 and not parts[0][2]:
            assert parts[0][:2] == (0, nsb), key
            continue
        assert all(p[2] for p in parts), key                  # a split tile has only pieces
        assert parts[0][0] == 0 and parts[-1][1] == nsb, key
        assert all(a[1] == b[0] and a[0] < a[1] for a, b in zip(parts, parts[1:])), key
        pieces += len(parts)
    assert (pieces > 0) == has_pieces


@pytest.mark.parametrize("layout", [2, 1, 0, "q4k"])
def test_timeline_build_matches_product_and_records_the_split(layout):
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    from q6_int8_prefill_amd import timeline as tl
    print(f"timeline layout={layout} n={N} m={M} k={K}", flush=True)
    dev = gpu_util.DEV
    x = synthetic.activations(N, K, seed=41)
    y0 = torch.full((N, M), float("nan"), dtype=torch.float32, device=dev)
    y1 = torch.full((N, M), float("nan"), dtype=torch.float32, device=dev)
    if layout == "q4k":
        raw = synthetic.weights_q4k(M, K, seed=42)
        xb, db = q6k.q6k_act_bytes(N, K)
        xq = torch.empty(xb, dtype=torch.uint8, device=dev)
        da = torch.empty(db // 4, dtype=torch.float32, device=dev)
        das = torch.empty_like(da)
        q6k.q4k_quantize_act(torch.from_numpy(x).to(dev), xq, da, das)
        w = torch.empty(q6k.q4k_weight_bytes(M, K), dtype=torch.uint8, device=dev)
        q6k.q4k_expand_weights(torch.from_numpy(raw.reshape(-1)).to(dev), M, K, w)
        ws = q6k.q4k_gemm_workspace(N, M, K)

        def run(y):
            q6k.q4k_gemm(xq, da, das, N, w, M, K, y)
    else:
        raw = synthetic.weights(M, K, seed=42)
        xq, da = gpu_util.quantize(x)
        w = gpu_util.expand(raw, M, K, layout)
        ws = q6k.q6k_gemm_workspace(N, M, K, layout)

        def run(y):
            q6k.q6k_gemm(xq, da, N, w, layout, M, K, y)
    run(y0)                                   # the product library
    torch.cuda.synchronize()
    rec = tl.Recorder()
    try:
        rec.clear()
        run(y1)                               # the same call through the timeline build
        torch.cuda.synchronize()
        records = rec.read()
    finally:
        rec.close()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    d = tl.decode(records)
    _check_records(d, N, M, K, ws > 0)
    s = tl.summarize(d)
    assert s["whole_tiles"] + s["pieces"] == len(d["wg"])
    if layout == 2:
        # behind whole rounds the tail is graded and claimed in start order: the pieces that start
        # at k = 0 (the largest) start, on average, before those that end at k (the smallest)
        nsb = K // 256
        pc = d["split"]
        size = d["s1"][pc] - d["s0"][pc]
        assert size.max() > size.min()
        first, last = d["start"][pc][d["s0"][pc] == 0], d["start"][pc][d["s1"][pc] == nsb]
        assert first.mean() < last.mean(), (first.mean(), last.mean())
