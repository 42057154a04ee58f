"""Workgroup timelines of the GEMM launches and their analysis.

`Recorder` switches the binding to libq6k_timeline.so (a second build of q6k.hip whose GEMM
workgroups each write one record: include/q6k_timeline.h) and reads the records back.  The
functions below are plain numpy over those records:
  * `decode` - one array per record field, times in microseconds from the launch's first start;
  * `summarize` - tile durations and the rate per super-block of k, each XCD's shader clock and
    last end, the gap between a workgroup's end and the next start on its CU, and how far apart
    in time the workgroups that share an operand tile start;
  * `l2_model` - the bytes each XCD's L2 fetches across the memory fabric if it held the most
    recently used operand blocks (one tile's slice of one 256-k super-block) up to its capacity,
    each block requested when the workgroup's progress, taken as linear in time, reaches it;
  * `lockstep` - the same launch rescheduled so that the workgroups running together on an XCD
    walk k together (what the model gives for it bounds what synchronizing them could save).
"""
import ctypes
import os
from collections import OrderedDict

import numpy as np

from . import _lib

timeline_lib_path = os.path.join(os.path.dirname(_lib.lib_path), "libq6k_timeline.so")
WORDS = 8          # uint64 per record
TICK_US = 0.01     # s_memrealtime runs at 100 MHz
L2_BYTES = 4 << 20  # one XCD's L2


class Recorder:
    """Routes the binding through libq6k_timeline.so until `close()`."""

    def __init__(self):
        if not os.path.exists(timeline_lib_path):
            raise ImportError(f"libq6k_timeline.so is not built ({timeline_lib_path}); run "
                              "__graft_entry__.build()")
        lib = _lib.use_library(timeline_lib_path)
        lib.q6k_timeline_capacity.restype = ctypes.c_int64
        lib.q6k_timeline_capacity.argtypes = []
        lib.q6k_timeline_clear.restype = ctypes.c_int
        lib.q6k_timeline_clear.argtypes = [ctypes.c_void_p]
        lib.q6k_timeline_read.restype = ctypes.c_int
        lib.q6k_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        self.lib = lib
        self.capacity = int(lib.q6k_timeline_capacity())

    def clear(self, stream=None):
        _lib._check(self.lib.q6k_timeline_clear(_lib._stream(stream)), "q6k_timeline_clear")

    def read(self):
        """Every record slot, [capacity][8] uint64 (a blocking copy: synchronize first)."""
        buf = np.zeros((self.capacity, WORDS), dtype=np.uint64)
        _lib._check(self.lib.q6k_timeline_read(buf.ctypes.data, self.capacity),
                    "q6k_timeline_read")
        return buf

    def close(self):
        _lib.use_library(_lib.lib_path)


def decode(rec):
    """Arrays over the written records (start word non-zero) of one launch."""
    rec = np.asarray(rec, dtype=np.uint64).reshape(-1, WORDS)
    wg = np.nonzero(rec[:, 0])[0]
    r = rec[wg]
    t0 = r[:, 0].min() if len(r) else 0
    lo = np.uint64(0xFFFFFFFF)
    return {
        "wg": wg,
        "start": (r[:, 0] - t0).astype(np.float64) * TICK_US,
        "end": (r[:, 1] - t0).astype(np.float64) * TICK_US,
        "cycles": (r[:, 3] - r[:, 2]).astype(np.float64),
        "xcd": (r[:, 4] >> np.uint64(32)).astype(np.int64),
        # HW_ID bits 8-15: CU, shader array and shader engine
        "cu": ((r[:, 4] >> np.uint64(8)) & np.uint64(0xFF)).astype(np.int64),
        "bx": (r[:, 5] & lo).astype(np.int64),
        "by": (r[:, 5] >> np.uint64(32)).astype(np.int64),
        "s0": (r[:, 6] & lo).astype(np.int64),
        "s1": (r[:, 6] >> np.uint64(32)).astype(np.int64),
        "split": r[:, 7] == 1,
    }


def _pct(v, qs=(10, 50, 90)):
    return [round(float(np.percentile(v, q)), 2) for q in qs] if len(v) else None


def _share_lags(d, key):
    """For every workgroup that starts while another one using the same operand tile (same XCD,
    same `key`) is running: its start minus the earliest such running user's start."""
    lags = []
    for x in np.unique(d["xcd"]):
        for v in np.unique(d[key][d["xcd"] == x]):
            sel = np.nonzero((d["xcd"] == x) & (d[key] == v))[0]
            order = sel[np.argsort(d["start"][sel])]
            for j, i in enumerate(order[1:], 1):
                earlier = order[:j]
                live = earlier[d["end"][earlier] > d["start"][i]]
                if len(live):
                    lags.append(d["start"][i] - d["start"][live].min())
    return np.array(lags)


def summarize(d):
    """Durations, per-XCD clocks and ends, CU hand-over gaps and operand-sharing lags (all in
    microseconds; `*_sb` figures in super-blocks of k at the whole tiles' median rate)."""
    dur = d["end"] - d["start"]
    nsb = (d["s1"] - d["s0"]).astype(np.float64)
    whole, piece = ~d["split"], d["split"]
    per_sb = float(np.median(dur[whole] / nsb[whole])) if whole.any() else float("nan")
    xcds = []
    for x in np.unique(d["xcd"]):
        s = d["xcd"] == x
        xcds.append({"xcd": int(x), "workgroups": int(s.sum()),
                     "clock_ghz": round(float(d["cycles"][s].sum() / dur[s].sum() / 1e3), 3),
                     "whole_tile_us": round(float(dur[s & whole].mean()), 2)
                     if (s & whole).any() else None,
                     "last_end_us": round(float(d["end"][s].max()), 2)})
    # the gap between a CU's latest earlier end and a workgroup's start (workgroups that did not
    # start with the launch)
    gaps = []
    first = d["start"].min() if len(dur) else 0.0
    for x, c in set(zip(d["xcd"].tolist(), d["cu"].tolist())):
        s = np.nonzero((d["xcd"] == x) & (d["cu"] == c))[0]
        for i in s:
            if d["start"][i] - first < 1.0:
                continue
            ends = d["end"][s][d["end"][s] <= d["start"][i] + 1e-9]
            if len(ends):
                gaps.append(d["start"][i] - ends.max())
    row_lag, tok_lag = _share_lags(d, "by"), _share_lags(d, "bx")
    return {
        "workgroups": int(len(dur)), "whole_tiles": int(whole.sum()), "pieces": int(piece.sum()),
        "span_us": round(float(d["end"].max()), 2) if len(dur) else 0.0,
        "us_per_superblock": {"whole": round(per_sb, 4),
                              "pieces": round(float(np.median(dur[piece] / nsb[piece])), 4)
                              if piece.any() else None},
        "tile_us_p10_p50_p90": {"whole": _pct(dur[whole]), "pieces": _pct(dur[piece])},
        "xcd": xcds,
        "cu_handover_us_p10_p50_p90": _pct(np.array(gaps)),
        "share_lag_sb_p50_p90": {
            "row_tile": [round(v / per_sb, 2) for v in _pct(row_lag, (50, 90))]
            if len(row_lag) else None,
            "token_tile": [round(v / per_sb, 2) for v in _pct(tok_lag, (50, 90))]
            if len(tok_lag) else None},
    }


def lockstep(d):
    """The same workgroups on the same XCDs, rescheduled so that those running together walk k
    together: each XCD's workgroups, in their recorded start order, run in rounds of the XCD's
    slot count (the workgroups that started with the launch); a round starts when the previous
    one's last workgroup ends, and every workgroup advances at the launch's median rate per
    super-block.  Returns a copy of `d` with the new start and end times."""
    e = dict(d)
    nsb = (d["s1"] - d["s0"]).astype(np.float64)
    whole = ~d["split"]
    rate = float(np.median((d["end"] - d["start"])[whole] / nsb[whole])) if whole.any() else \
        float(np.median((d["end"] - d["start"]) / nsb))
    start, end = np.zeros(len(nsb)), np.zeros(len(nsb))
    first = d["start"].min() if len(nsb) else 0.0
    for x in np.unique(d["xcd"]):
        idx = np.nonzero(d["xcd"] == x)[0]
        idx = idx[np.argsort(d["start"][idx], kind="stable")]
        slots = max(1, int((d["start"][idx] - first < 1.0).sum()))
        t = 0.0
        for r in range(0, len(idx), slots):
            grp = idx[r:r + slots]
            start[grp] = t
            end[grp] = t + rate * nsb[grp]
            t = end[grp].max()
    e["start"], e["end"] = start, end
    return e


def l2_model(d, act_block, wgt_block, l2_bytes=L2_BYTES):
    """Modelled fabric fetch of one launch: per XCD, a least-recently-used cache of `l2_bytes`
    over blocks ('a', token tile, super-block) of `act_block` bytes and ('w', row tile,
    super-block) of `wgt_block` bytes, requested in time order.  Returns the fetched bytes and
    the bytes of distinct blocks (each XCD's blocks counted once: what any order of the same
    tiles on the same XCDs must fetch at least)."""
    fetched = unique = 0
    for x in np.unique(d["xcd"]):
        ev = []
        for i in np.nonzero(d["xcd"] == x)[0]:
            s0, s1 = int(d["s0"][i]), int(d["s1"][i])
            t, span = d["start"][i], (d["end"][i] - d["start"][i]) / max(s1 - s0, 1)
            for j, s in enumerate(range(s0, s1)):
                tj = t + (j + 0.5) * span
                ev.append((tj, ("a", int(d["bx"][i]), s), act_block))
                ev.append((tj, ("w", int(d["by"][i]), s), wgt_block))
        ev.sort(key=lambda e: e[0])
        lru, size, seen = OrderedDict(), 0, set()
        for _, key, nbytes in ev:
            if key in lru:
                lru.move_to_end(key)
                continue
            fetched += nbytes
            if key not in seen:
                seen.add(key)
                unique += nbytes
            lru[key] = nbytes
            size += nbytes
            while size > l2_bytes:
                _, b = lru.popitem(last=False)
                size -= b
    return {"fetch_bytes": int(fetched), "distinct_block_bytes": int(unique)}
