"""Host-side analysis of workgroup timelines (q6_int8_prefill_amd.timeline) on hand-built records
whose answers follow by hand: record decoding, the per-XCD clock, the CU hand-over gap, the
operand-sharing lag, and the LRU model of an XCD's L2."""
import numpy as np

from q6_int8_prefill_amd import timeline as tl


def rec(start_us, end_us, cycles, xcd, cu, bx, by, s0, s1, split=False, t0=10_000_000):
    """One 8-word record as the instrumented kernels write it."""
    ticks = lambda us: t0 + int(round(us * 100))  # noqa: E731  (100 MHz)
    return [ticks(start_us), ticks(end_us), 5_000, 5_000 + cycles, (xcd << 32) | (cu << 8) | 3,
            bx | (by << 32), s0 | (s1 << 32), 1 if split else 0]


def records(rows, capacity=16):
    out = np.zeros((capacity, tl.WORDS), dtype=np.uint64)
    for i, r in rows:
        out[i] = np.array(r, dtype=np.uint64)
    return out


def test_decode_fields_and_unwritten_slots():
    r = records([(0, rec(0.0, 10.0, 20_000, 0, 0x21, 5, 7, 0, 4)),
                 (3, rec(1.5, 4.0, 6_000, 3, 0x40, 2, 1, 1, 3, split=True))])
    d = tl.decode(r)
    assert list(d["wg"]) == [0, 3]                       # slots 1, 2 and 4.. were not written
    assert np.allclose(d["start"], [0.0, 1.5]) and np.allclose(d["end"], [10.0, 4.0])
    assert list(d["cycles"]) == [20_000, 6_000]
    assert list(d["xcd"]) == [0, 3] and list(d["cu"]) == [0x21, 0x40]
    assert list(d["bx"]) == [5, 2] and list(d["by"]) == [7, 1]
    assert list(d["s0"]) == [0, 1] and list(d["s1"]) == [4, 3]
    assert list(d["split"]) == [False, True]


def test_summarize_clock_handover_and_share_lag():
    rows = [
        (0, rec(0.0, 10.0, 20_000, 0, 1, 0, 0, 0, 4)),    # XCD 0, CU 1: 2.0 GHz
        (1, rec(11.0, 21.0, 20_000, 0, 1, 1, 1, 0, 4)),   # next workgroup on CU 1, 1 us later
        (2, rec(2.0, 12.0, 20_000, 0, 2, 1, 0, 0, 4)),    # shares row tile 0, starts 2 us late
        (3, rec(0.0, 10.0, 15_000, 1, 1, 2, 2, 0, 4)),    # XCD 1: 1.5 GHz
        (4, rec(10.0, 12.5, 5_000, 1, 1, 2, 3, 0, 1, split=True)),
    ]
    s = tl.summarize(tl.decode(records(rows)))
    assert (s["workgroups"], s["whole_tiles"], s["pieces"]) == (5, 4, 1)
    assert s["span_us"] == 21.0
    assert s["us_per_superblock"] == {"whole": 2.5, "pieces": 2.5}
    x0, x1 = s["xcd"]
    assert x0["clock_ghz"] == 2.0 and x1["clock_ghz"] == 1.6   # (15000 + 5000) / 12.5 us
    assert x0["last_end_us"] == 21.0 and x1["whole_tile_us"] == 10.0
    # hand-over: workgroup 1 after workgroup 0 on CU 1 of XCD 0 (1 us), workgroup 4 right at the
    # end of workgroup 3 (0 us)
    assert s["cu_handover_us_p10_p50_p90"][1] == 0.5
    # row tile 0 on XCD 0: workgroup 2 starts 2 us = 0.8 super-blocks after workgroup 0; token
    # tile 1: workgroup 1 starts after workgroup 2 began (9 us) while it still runs
    assert s["share_lag_sb_p50_p90"]["row_tile"] == [0.8, 0.8]
    assert s["share_lag_sb_p50_p90"]["token_tile"] == [3.6, 3.6]


def test_l2_model_shared_weight_tile_fetched_once():
    # two workgroups on one XCD, same row tile, different token tiles, in lockstep over 4
    # super-blocks: the weights are fetched once, each token tile once
    rows = [(0, rec(0.0, 8.0, 1, 0, 1, 0, 0, 0, 4)), (1, rec(0.0, 8.0, 1, 0, 2, 1, 0, 0, 4))]
    m = tl.l2_model(tl.decode(records(rows)), act_block=100, wgt_block=1000, l2_bytes=1 << 20)
    assert m == {"fetch_bytes": 4 * (2 * 100 + 1000), "distinct_block_bytes": 4800}


def test_l2_model_eviction_refetches():
    # the same schedule with room for 1000 bytes: per super-block, workgroup 0's token block is
    # evicted by the weight block, which the second token block then evicts before workgroup 1
    # asks for it -- the weights cross the fabric twice
    rows = [(0, rec(0.0, 8.0, 1, 0, 1, 0, 0, 0, 4)), (1, rec(0.0, 8.0, 1, 0, 2, 1, 0, 0, 4))]
    m = tl.l2_model(tl.decode(records(rows)), act_block=100, wgt_block=1000, l2_bytes=1000)
    assert m == {"fetch_bytes": 4 * (2 * 100 + 2 * 1000), "distinct_block_bytes": 4800}


def test_l2_model_each_xcd_fetches_its_own_copy():
    rows = [(0, rec(0.0, 8.0, 1, 0, 1, 0, 0, 0, 4)), (1, rec(0.0, 8.0, 1, 1, 1, 0, 0, 0, 4))]
    m = tl.l2_model(tl.decode(records(rows)), act_block=100, wgt_block=1000, l2_bytes=1 << 20)
    assert m == {"fetch_bytes": 2 * 4 * 1100, "distinct_block_bytes": 2 * 4 * 1100}


def test_l2_model_split_piece_covers_its_own_superblocks():
    # a piece over super-blocks [2, 4) after a whole tile [0, 4) of the same operands on the same
    # XCD, with the cache large: the piece hits on every block
    rows = [(0, rec(0.0, 8.0, 1, 0, 1, 0, 0, 0, 4)),
            (1, rec(8.0, 12.0, 1, 0, 1, 0, 0, 2, 4, split=True))]
    m = tl.l2_model(tl.decode(records(rows)), act_block=100, wgt_block=1000, l2_bytes=1 << 20)
    assert m["fetch_bytes"] == 4 * 1100


def test_lockstep_brings_sharing_workgroups_together():
    # one XCD with 2 slots: the second round's two workgroups share row tile 2, but the slot of
    # the slower first-round workgroup frees 2 us (1 super-block) later.  With room for about one
    # super-block of their operands the late one refetches each weight block; in lockstep (both
    # rounds at the median 2 us per super-block) the pair shares them.
    rows = [(0, rec(0.0, 8.0, 1, 0, 1, 0, 0, 0, 4)),
            (1, rec(0.0, 10.0, 1, 0, 2, 1, 1, 0, 4)),
            (2, rec(8.0, 16.0, 1, 0, 1, 2, 2, 0, 4)),
            (3, rec(10.0, 18.0, 1, 0, 2, 3, 2, 0, 4))]
    d = tl.decode(records(rows))
    e = tl.lockstep(d)
    assert list(e["start"]) == [0.0, 0.0, 8.0, 8.0] and list(e["end"]) == [8.0, 8.0, 16.0, 16.0]
    before = tl.l2_model(d, act_block=100, wgt_block=1000, l2_bytes=1300)
    after = tl.l2_model(e, act_block=100, wgt_block=1000, l2_bytes=1300)
    assert after["distinct_block_bytes"] == before["distinct_block_bytes"] == 4 * 4 * 100 + \
        3 * 4 * 1000
    # lockstep: every block once; recorded: row tile 2's weights twice
    assert after["fetch_bytes"] == after["distinct_block_bytes"]
    assert before["fetch_bytes"] == after["fetch_bytes"] + 4 * 1000
