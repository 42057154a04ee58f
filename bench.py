"""Benchmark of the q6_K x int8 prefill hot path on one MI355X.

One step = one pass of the hot path over one batch: the activation quantize-transpose prepass
(q6k_quantize_act) followed by the GEMM (q6k_gemm) on weights prepared once at load time
(q6k_expand_weights, outside the timed region).  Inputs are synthetic, seeded, and resident in HBM
before timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout 0|1|2] [--layouts 0,1,2]
                    [--workload NAME] [--weights q6k|q4k] [--cold] [--swiglu]
                    [--no-cpu-baseline] [--copy-probe-mib MIB] [--ceilings] [--timeline]
                    [--activations normal|outlier|swiglu|zero]

Timing protocol (all with HIP events recorded on the stream the kernels run on):
  * ms_per_step: K steps of prepass + GEMM of the headline layout (--layout) back to back, events
    only at the two ends;
  * the GEMM of every layout in --layouts, interleaved in the same window: K rounds, each round
    one block of --block back-to-back launches per layout (the starting layout rotates from round
    to round), events only around each block;  per-launch time = block time / block;
  * `value` = the headline layout's GEMM effective int8 TOPS, 2*N*M*K / its mean per-launch time
    (a launch is the GEMM kernel plus the small kernel that adds up the split tiles' workspace
    slabs, when there are any); the per-layout figures (mean, p10/p50/p90 over rounds, TOPS, fraction of the int8 peak)
    are in `layouts`;
  * the prepass time comes from a third pass of K steps with events between the two kernels.

Workloads: tiny, attn_v_n512, attn_v_n3314, ffn_down_n3314 (the default and headline case),
ffn_down_shard8 (3314 x 512 x 11008: one GPU's share of ffn_down under an 8-way split of the
output rows), and sweep32: 32 layers of (attn_v 4096x4096 + ffn_down 4096x11008) at 3314 tokens,
64 GEMMs back to back on one stream over 1.6 GB of raw weights, inputs drawn on the device (a
step and a GEMM block then cover all 64).  --cold writes a 512 MiB scrub buffer and then reads a
1 GiB one before every timed step and every GEMM block (of one launch), so weights and
activations come from HBM rather than the 256 MB Infinity Cache (the read leaves the cache
holding clean lines: evicting the write's dirty lines inside the timed span would time their
write-back instead).  --swiglu replaces the prepass by the fused producer q6k_swiglu_quantize_act
reading the two SwiGLU factors, and also times the unfused pair (q6k_swiglu_f32 writing h, then
q6k_quantize_act).  --weights q4k runs the q4_K variant on the same shapes: step =
q4k_quantize_act (codes, da and das in one pass) + q4k_gemm.  --activations replaces the
workload's activation distribution (named in `config`): 'zero' runs every launch unchanged on
all-zero operands, which shows how far the sustained clock depends on the data.

--timeline runs the GEMMs through libq6k_timeline.so (same kernels, each workgroup also writing
where and when it ran) and prints, per layout, tile durations, each XCD's shader clock and last
end, CU hand-over gaps, the start lags of workgroups sharing an operand tile, and an L2 model's
fabric fetch (for the recorded schedule, and for the same tiles with each XCD's concurrent
workgroups in lockstep) beside the committed FETCH_SIZE figure (use a few --steps: the model is
Python).

--ceilings runs the microbenchmarks of libq6k_ceilings.so instead (MFMA issue rates, vector-ALU
issue rates at 1, 2, 4 and 8 waves per SIMD, the GEMMs' tile operation without memory traffic,
HBM streaming) and prints them as one JSON line.  The default run also measures the vector-ALU
rate of the GEMMs' own instruction forms at their occupancy, which `alu_roofline` uses as its
measured peak.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
# f32 vector lane-operations per second from the unit counts: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz issues one wave64 instruction per SIMD every 4 cycles (39.3 T lane-ops/s); the
# published 157.3 TFLOP/s fp32 vector figure is twice that again (78.6 T lane-ops/s, counting an
# FMA as 2 flops), which needs two instructions per SIMD per 4 cycles
VALU_SPEC_SINGLE = 256 * 4 * 16 * 2.4e9 / 1e12
VALU_SPEC_DUAL = 2 * VALU_SPEC_SINGLE
METRIC = "q6_K GEMM effective int8 TOPS + µs/GMAC, % of MFMA peak (ffn_down, N=3314)"
KERNEL_NAMES = {0: "gemm_kernel<layout 0> (6-bit codes expanded at staging; two 16-k halves, "
                   "each with its own d*sc rescale)",
                1: "gemm_kernel<layout 1> (load-time centered int8 plane + f32 d*sc plane; two "
                   "16-k halves, each with its own d*sc rescale)",
                2: "folded_kernel (layout 2: int8 sc folded into two int8 digit planes; one "
                   "rescale per 32-k chunk)",
                "q4k": "q4k_gemm_kernel"}
# f32 vector lane-operations the method's rescale needs per output (the unit that binds it)
VALU_FORM = {0: "4 per 32-k chunk: two halves x (fma with d*sc, fma with da)",
             1: "4 per 32-k chunk: two halves x (fma with d*sc, fma with da)",
             2: "3 per 32-k chunk (digit fold: two adds; fma with da) + 1 per super-block (d)",
             "q4k": "3 per 32-k chunk: fma with d*sc, fma with da, fma with -dmin*m and da*S"}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~50 steps (~30 ms on ffn_down) bring the GPU's clock to its loaded steady state; with 5, the
    # first timed steps still run several percent slow
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layout", type=int, default=2, choices=[0, 1, 2],
                    help="headline layout: the step's GEMM and `value`")
    ap.add_argument("--layouts", default="0,1,2",
                    help="layouts whose GEMMs are timed interleaved in the same window")
    ap.add_argument("--block", type=int, default=5, help="GEMM launches per timed block")
    ap.add_argument("--workload", default="ffn_down_n3314")
    ap.add_argument("--weights", default="q6k", choices=["q6k", "q4k"],
                    help="weight format: q6_K (the headline) or the q4_K variant")
    ap.add_argument("--activations", default=None,
                    choices=["normal", "outlier", "swiglu", "zero"],
                    help="activation distribution (default: the workload's own); 'zero' runs the "
                         "same launches on all-zero operands, for the clock's data dependence")
    ap.add_argument("--cold", action="store_true")
    ap.add_argument("--swiglu", action="store_true",
                    help="feed the GEMM from the fused SwiGLU -> int8 producer (gate, up inputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the CPU-baseline sample (0: the whole workload)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ceilings", action="store_true",
                    help="run the unit microbenchmarks instead of the GEMM")
    ap.add_argument("--timeline", action="store_true",
                    help="record per-workgroup timelines of --steps GEMM launches per layout "
                         "with libq6k_timeline.so instead of timing")
    return ap.parse_args(argv)


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ------------------------------------------------------------------------------------------------
def host_cpu():
    """The host CPU's model name and the hardware threads this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"model": model, "threads_available": threads}


def cpu_baseline(raw, x, m, k, tokens, weights="q6k"):
    """The oracle (plain C, rows split over the host threads it may use) on the first `tokens`
    tokens of the same workload (all of them when tokens <= 0), all rows: quantize + reference
    GEMM, scaled to TOPS."""
    import oracle
    tokens = x.shape[0] if tokens <= 0 else min(tokens, x.shape[0])
    xs = x[:tokens]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    xq, da = oracle.quantize(xs, threads=threads)
    (oracle.q4_gemm if weights == "q4k" else oracle.gemm)(xq, da, raw, m, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * tokens * m * k / dt / 1e12, 5), "unit": "TOPS",
            "cores": threads, "kind": "oracle",
            "sample": f"{'all' if tokens == x.shape[0] else 'first'} {tokens} tokens x all {m} "
                      f"rows x k={k} (quantize + reference GEMM), {dt:.2f} s on {threads} threads",
            "host": host_cpu()}


# ------------------------------------------------------------------------------------------------
# Committed counter summary (HBM traffic per launch)
# ------------------------------------------------------------------------------------------------
def kernel_source_digest():
    """sha256 (16 hex digits) of the kernel source with comments and whitespace removed: it
    changes when the code changes, not when only its comments do."""
    import hashlib
    import re
    with open(os.path.join(ROOT, "q6_int8_prefill_amd", "csrc", "q6k.hip")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def _counter_entry(workload, layout):
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_code_sha256_16") != kernel_source_digest():
        return None, None
    return rec, rec.get("layouts", {}).get(str(layout))


def counter_fetch(workload, layout):
    """FETCH_SIZE bytes of one GEMM launch from the committed summary (scaled as its traffic
    figure is), or None."""
    rec, entry = _counter_entry(workload, layout)
    if entry is None:
        return None
    return int(entry["gemm_fetch_size_kib"] * 1024 * rec["fetch_scale"])


def counter_traffic(workload, layout):
    """HBM-side bytes of one GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None if there is none for this workload or the kernel code changed since it was taken."""
    _, entry = _counter_entry(workload, layout)
    return None if entry is None else int(entry["traffic_bytes"])


# ------------------------------------------------------------------------------------------------
# Microbenchmarks (libq6k_ceilings.so)
# ------------------------------------------------------------------------------------------------
MFMA_KINDS = {0: ("v_mfma_i32_32x32x16_i8", 2 * 32 * 32 * 16),
              1: ("v_mfma_i32_32x32x32_i8", 2 * 32 * 32 * 32),
              2: ("v_mfma_i32_16x16x64_i8", 2 * 16 * 16 * 64),
              3: ("v_mfma_f32_32x32x16_f16", 2 * 32 * 32 * 16)}
VALU_KINDS = {0: "v_fma_f32", 1: "v_fmac_f32", 2: "v_add_f32", 3: "v_mul_f32",
              4: "v_cvt_f32_i32", 5: "v_add_u32"}
TILEOP_KINDS = {0: ("folded: 2 x v_mfma_i32_32x32x32_i8 + 48 VALU", 48),
                1: ("two halves: 2 x v_mfma_i32_32x32x16_i8 + 64 VALU", 64),
                2: ("folded, MFMAs issued half a step ahead of the fold", 48),
                3: ("folded mix, MFMA accumulator input an inline zero (cost of reading C)", 48),
                4: ("f16 digits: 4 x v_mfma_f32_32x32x16_f16 chained from zero + 16 VALU", 16)}


class Probes:
    def __init__(self, torch):
        self.torch = torch
        path = os.path.join(ROOT, "q6_int8_prefill_amd", "_build", "libq6k_ceilings.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        for fn in ("q6c_mfma", "q6c_valu", "q6c_tileop"):
            getattr(L, fn).restype = i
            getattr(L, fn).argtypes = [i, i, i, p, sz, p]
        L.q6c_overlap.restype = i
        L.q6c_overlap.argtypes = [i, i, i, p, sz, p]
        L.q6c_stream.restype = i
        L.q6c_stream.argtypes = [i, p, p, sz, sz, p]
        L.q6c_probe_waves.restype = i
        L.q6c_probe_waves.argtypes = [i]
        L.q6c_wall_clock_khz.restype = i
        L.q6c_wall_clock_khz.argtypes = []
        self.L = L
        self.wall_khz = L.q6c_wall_clock_khz()

    def run(self, fn, kind, iters, w):
        """-> (elapsed s, per-wave cycles, per-wave seconds, waves)."""
        import numpy as np
        torch = self.torch
        nw = self.L.q6c_probe_waves(w)
        out = torch.zeros(nw * 4, dtype=torch.int64, device="cuda")
        stream = torch.cuda.current_stream()
        f = getattr(self.L, fn)
        for it in (max(1, iters // 20), iters):  # a short warm launch, then the timed one
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = f(kind, it, w, out.data_ptr(), out.numel() * 8, stream.cuda_stream)
            e1.record(stream)
            if st != 0:
                raise RuntimeError(f"{fn}({kind}) failed with status {st}")
            torch.cuda.synchronize()
        r = out.view(nw, 4).cpu().numpy()
        cycles = r[:, 0].astype(np.float64)
        secs = r[:, 1].astype(np.float64) / (self.wall_khz * 1e3)
        return e0.elapsed_time(e1) * 1e-3, cycles, secs, nw

    @staticmethod
    def clock_ghz(cycles, secs):
        import numpy as np
        return float(np.median(cycles / secs) / 1e9)

    # Cycle figures are per SIMD over the whole launch: the clock measured inside the waves times
    # the event-timed launch, divided by the instructions (or tiles) one SIMD ran -- all SIMDs run
    # the same share concurrently.  (A single wave's own span would overstate the rate when several
    # waves share a SIMD and start or end at different times.)
    def mfma(self, kind, w, iters=20000):
        name, ops = MFMA_KINDS[kind]
        el, cyc, secs, nw = self.run("q6c_mfma", kind, iters, w)
        n_instr = nw * iters * 4
        ghz = self.clock_ghz(cyc, secs)
        return {"instr": name, "waves_per_simd": w, "tops": round(n_instr * ops / el / 1e12, 1),
                "cycles_per_instr_per_simd": round(ghz * 1e9 * el / (n_instr / 1024), 2),
                "clock_ghz": round(ghz, 3)}

    def valu(self, kind, w, iters=8000):
        el, cyc, secs, nw = self.run("q6c_valu", kind, iters, w)
        n_instr = nw * iters * 64
        ghz = self.clock_ghz(cyc, secs)
        return {"instr": VALU_KINDS[kind], "waves_per_simd": w,
                "lane_ops_t_per_s": round(n_instr * 64 / el / 1e12, 2),
                "cycles_per_instr_per_simd": round(ghz * 1e9 * el / (n_instr / 1024), 3),
                "clock_ghz": round(ghz, 3)}

    def tileop(self, kind, w, iters=4000):
        name, nvalu = TILEOP_KINDS[kind]
        el, cyc, secs, nw = self.run("q6c_tileop", kind, iters, w)
        tiles = nw * iters * 2  # two 32x32 tiles per wave and round, one 32-k chunk each
        ghz = self.clock_ghz(cyc, secs)
        return {"op": name, "waves_per_simd": w,
                "ns_per_tile_chunk_per_simd": round(el * 1e9 * 1024 / tiles, 2),
                "cycles_per_tile_chunk_per_simd": round(ghz * 1e9 * el / (tiles / 1024), 1),
                "valu_lane_ops_t_per_s": round(tiles * nvalu * 64 / el / 1e12, 2),
                "equiv_gemm_tops": round(tiles * 2 * 32 * 32 * 32 / el / 1e12, 1),
                "clock_ghz": round(ghz, 3)}

    def overlap(self, iters=20000):
        """Whether the vector ALU issues while the matrix core runs (see q6k_ceilings.h): median
        shader cycles of the MFMA waves and of the VALU waves, each role alone and both together
        (12 waves per CU: one MFMA and two VALU waves per SIMD), and the cycles per round of one
        wave alternating MFMAs
        and independent VALU instructions against its MFMAs alone."""
        import numpy as np
        torch = self.torch
        stream = torch.cuda.current_stream()
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        out = torch.zeros(cus * 12 * 4, dtype=torch.int64, device="cuda")

        def run(kind, im, iv):
            st = self.L.q6c_overlap(kind, im, iv, out.data_ptr(), out.numel() * 8,
                                    stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"q6c_overlap({kind}) failed with status {st}")
            torch.cuda.synchronize()
            waves = 12 if kind == 0 else 4
            return out[:cus * waves * 4].view(cus, waves, 4)[:, :, 0].cpu().numpy().astype(np.float64)

        # 4 MFMAs of 32 cycles against 64 VALU from two waves at ~2.2 cycles each
        iv = int(iters * 128 / 141)
        run(0, iters // 10, iv // 10)
        m_alone = float(np.median(run(0, iters, 0)[:, :4]))
        v_alone = float(np.median(run(0, 0, iv)[:, 4:]))
        both = run(0, iters, iv)
        same = float(np.median(run(1, iters, 0)))
        return {"roles": {"mfma_waves_cycles_alone": m_alone,
                          "valu_waves_cycles_alone": v_alone,
                          "mfma_waves_cycles_together": float(np.median(both[:, :4])),
                          "valu_waves_cycles_together": float(np.median(both[:, 4:])),
                          "mfma_rounds": iters, "valu_rounds": iv,
                          "note": "4 x v_mfma_i32_32x32x32_i8 per MFMA round (one wave per "
                                  "SIMD), 64 x v_add_f32 per VALU round (two waves per SIMD); "
                                  "overlap keeps 'together' near 'alone'"},
                "same_wave": {"cycles_per_round": round(same / iters, 1),
                              "round": "4 x (1 v_mfma_i32_32x32x32_i8 + 8 independent v_add_f32)",
                              "mfma_alone_cycles_per_round": 128,
                              "valu_alone_cycles_per_round": round(32 * 4.44, 1)}}

    def hbm(self, mib=2048):
        torch = self.torch
        src = torch.ones(mib << 18, dtype=torch.int32, device="cuda")
        dst = torch.empty(mib << 17, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream()
        res = {}
        names = {0: "read", 1: "copy", 2: "read_nontemporal"}
        for mode, nbytes, moved in ((0, mib << 20, mib << 20), (2, mib << 20, mib << 20),
                                    (1, mib << 19, mib << 20)):
            best = None
            for _ in range(6):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st = self.L.q6c_stream(mode, src.data_ptr(), dst.data_ptr(), nbytes,
                                       dst.numel() * 4, stream.cuda_stream)
                e1.record(stream)
                if st != 0:
                    raise RuntimeError(f"q6c_stream({mode}) failed with status {st}")
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3
                best = t if best is None else min(best, t)
            res[names[mode]] = {
                "bytes_moved": moved, "gbs": round(moved / best / 1e9, 1)}
        return res


def alu_probe(torch):
    """The vector-ALU rate of the GEMMs' own rescale instruction forms (v_add_f32, v_fmac_f32,
    v_fma_f32) at the kernels' occupancy (2 waves per SIMD) and at 8 waves per SIMD, and the
    tile operations at 2 waves per SIMD: -> (summary, best measured lane-ops/s in T)."""
    pr = Probes(torch)
    rows = [pr.valu(kind, w) for kind in (2, 1, 0) for w in (2, 8)]
    tiles = [pr.tileop(kind, 2) for kind in (0, 1)]
    best = max(r["lane_ops_t_per_s"] for r in rows)
    return {"valu": rows, "tileop": tiles}, best


def run_ceilings(args):
    import torch
    pr = Probes(torch)

    def each(fn, *cases):
        rows = []
        for case in cases:
            try:
                rows.append(fn(*case))
            except RuntimeError as exc:  # a launch the runtime refused: report it, keep going
                rows.append({"case": list(case), "error": str(exc)})
        return rows

    out = {"mode": "ceilings", "n_gpus": 1, "wall_clock_khz": pr.wall_khz,
           "mfma": each(pr.mfma, *[(k, w) for k in (0, 1, 2, 3) for w in (1, 2)]),
           "valu": each(pr.valu, *[(k, w) for k in (0, 1, 2, 3, 4, 5) for w in (1, 2, 4, 8)]),
           "tileop": each(pr.tileop, *[(k, w) for k in (0, 1, 2, 3, 4) for w in (1, 2, 3, 4)]),
           "overlap": pr.overlap(),
           "hbm": pr.hbm(),
           "spec": {"int8_dense_tops": INT8_PEAK_TOPS, "hbm_gbs": HBM_PEAK_GBS,
                    "valu_lane_ops_t_single": round(VALU_SPEC_SINGLE, 1),
                    "valu_lane_ops_t_dual": round(VALU_SPEC_DUAL, 1)}}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------------------------
# Device buffers
# ------------------------------------------------------------------------------------------------
class Acts:
    """One batch of activations and its prepass output."""

    def __init__(self, q6k, torch, x_d, n, k, dev, up_d=None, q4=False):
        self.q6k, self.n, self.k = q6k, n, k
        self.x, self.up = x_d, up_d  # with up: x is the gate, the producer is the fused SwiGLU
        xb, db = q6k.q6k_act_bytes(n, k)
        self.xq = torch.empty(xb, dtype=torch.uint8, device=dev)
        self.da = torch.empty(db // 4, dtype=torch.float32, device=dev)
        self.das = torch.empty(db // 4, dtype=torch.float32, device=dev) if q4 else None

    def quantize(self):
        if self.up is not None:
            self.q6k.q6k_swiglu_quantize_act(self.x, self.up, self.xq, self.da)
            if self.das is not None:
                self.q6k.q4k_act_sums(self.xq, self.da, self.n, self.k, self.das)
        elif self.das is not None:
            self.q6k.q4k_quantize_act(self.x, self.xq, self.da, self.das)
        else:
            self.q6k.q6k_quantize_act(self.x, self.xq, self.da)

    def bytes(self):
        """prepass algorithmic bytes: f32 input(s) + int8 codes + f32 scales (and das)"""
        extra = self.n * (self.k // 32) * 4 * (2 if self.das is not None else 1)
        return self.n * self.k * (4 if self.up is None else 8) + self.n * self.k + extra


class Gemm:
    """Prepared weights of one matrix in one layout (or q4_K) and the GEMM launch."""

    def __init__(self, q6k, torch, acts, raw_d, m, layout, y, dev):
        self.q6k, self.acts, self.m, self.layout, self.y = q6k, acts, m, layout, y
        n, k = acts.n, acts.k
        self.n, self.k = n, k
        if layout == "q4k":
            self.w = torch.empty(q6k.q4k_weight_bytes(m, k), dtype=torch.uint8, device=dev)
            q6k.q4k_expand_weights(raw_d, m, k, self.w)
            ws = q6k.q4k_gemm_workspace(n, m, k)
        else:
            self.w = torch.empty(q6k.q6k_weight_bytes(m, k, layout), dtype=torch.uint8, device=dev)
            q6k.q6k_expand_weights(raw_d, m, k, layout, self.w)
            ws = q6k.q6k_gemm_workspace(n, m, k, layout)
        # the split-k slabs, allocated once (the timed steps allocate nothing)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)

    def launch(self):
        a = self.acts
        if self.layout == "q4k":
            self.q6k.q4k_gemm(a.xq, a.da, a.das, self.n, self.w, self.m, self.k, self.y,
                              workspace=self.ws)
        else:
            self.q6k.q6k_gemm(a.xq, a.da, self.n, self.w, self.layout, self.m, self.k, self.y,
                              workspace=self.ws)

    def ops(self):
        return 2.0 * self.n * self.m * self.k

    def bytes(self):
        """GEMM algorithmic bytes: weights as stored + int8 codes + f32 scales + f32 Y"""
        a = self.acts
        return (self.w.numel() + self.n * self.k + self.n * (self.k // 32) * 4 *
                (2 if a.das is not None else 1) + self.n * self.m * 4)

    def valu_lane_ops(self):
        if self.layout == 2:
            return float(self.n) * self.m * (3 * (self.k // 32) + self.k // 256)
        per_chunk = 3 if self.layout == "q4k" else 4
        return float(self.n) * self.m * per_chunk * (self.k // 32)


# ------------------------------------------------------------------------------------------------
# Workgroup timelines (libq6k_timeline.so)
# ------------------------------------------------------------------------------------------------
def run_timeline(args, torch, acts, gemms, layouts):
    """--timeline: after --warmup launches of each layout, --steps blocks of --block back-to-back
    launches of each (interleaved, the starting layout rotating), the last launch of every block
    recorded; per layout the summary of the recorded launch of median span and the L2 model of
    every recorded launch, beside the committed FETCH_SIZE."""
    import numpy as np

    from q6_int8_prefill_amd import timeline as tl

    acts.quantize()  # the GEMMs' int8 operand and its scales
    rec = tl.Recorder()
    try:
        for _ in range(args.warmup):
            for L in layouts:
                gemms[L].launch()
        torch.cuda.synchronize()
        runs = {L: [] for L in layouts}
        for r in range(args.steps):
            for j in range(len(layouts)):
                L = layouts[(r + j) % len(layouts)]
                rec.clear()
                # --block launches back to back, as the timed blocks run them: every workgroup
                # rewrites its record, so the records read are the last launch's
                for _ in range(args.block):
                    gemms[L].launch()
                torch.cuda.synchronize()
                runs[L].append(tl.decode(rec.read()))
    finally:
        rec.close()
    out = {"mode": "timeline", "workload": args.workload, "recorded_launches": args.steps,
           "block": args.block, "warmup": args.warmup, "layouts": {}}
    for L in layouts:
        g = gemms[L]
        # 64-token x 128-row output tiles; tokens are padded to 128 in the activation buffers
        nsb, gx, gy = g.k // 256, 2 * -(-g.n // 128), -(-g.m // 128)
        scale_words = 2 if acts.das is not None else 1
        # one 64-token tile's or one 128-row tile's bytes per super-block, as stored
        act_block = (acts.xq.numel() + acts.da.numel() * 4 * scale_words) / (gx * nsb)
        wgt_block = g.w.numel() / (gy * nsb)
        spans = [float(d["end"].max()) for d in runs[L]]
        med = runs[L][int(np.argsort(spans)[len(spans) // 2])]
        model = [tl.l2_model(d, act_block, wgt_block) for d in runs[L]]
        locked = tl.l2_model(tl.lockstep(med), act_block, wgt_block)
        out["layouts"][str(L)] = {
            "kernel": KERNEL_NAMES[L],
            "span_us": [round(v, 2) for v in spans],
            "median_launch": tl.summarize(med),
            "l2_model": {
                "l2_bytes": tl.L2_BYTES, "act_block_bytes": act_block,
                "wgt_block_bytes": wgt_block,
                "fetch_bytes_mean": int(np.mean([v["fetch_bytes"] for v in model])),
                "fetch_bytes_lockstep": locked["fetch_bytes"],
                "distinct_block_bytes": model[0]["distinct_block_bytes"]},
            "counter_fetch_bytes": counter_fetch(args.workload, L)}
    print(json.dumps(out))


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py: the GEMM runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU split is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if args.ceilings:
        run_ceilings(args)
        return
    if args.activations and (args.swiglu or args.workload == "sweep32"):
        print("bench.py: --activations sets the activations of a single-GEMM workload; the SwiGLU "
              "producer and the sweep draw their own", file=sys.stderr)
        sys.exit(2)
    if args.timeline and args.workload == "sweep32":
        print("bench.py: --timeline records one GEMM's launches; pick a single-GEMM workload",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import q6_int8_prefill_amd as q6k

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sweep = args.workload == "sweep32"
    q4 = args.weights == "q4k"
    head = "q4k" if q4 else args.layout
    if q4:
        layouts = ["q4k"]
    elif args.swiglu:
        layouts = [args.layout]
    else:
        layouts = sorted({int(v) for v in args.layouts.split(",") if v.strip()} | {args.layout})

    # ------------------------------------------------------------ inputs resident in HBM
    t0 = time.perf_counter()
    raw = x = None
    units = []  # per matrix: (acts, {layout: Gemm})
    if sweep:
        for layer in range(synthetic.SWEEP_LAYERS):
            for kind in ("attn_v", "ffn_down"):
                raw_d, x_d, sn, sm, sk = synthetic.sweep_inputs_torch(layer, kind, dev)
                acts = Acts(q6k, torch, x_d, sn, sk, dev)
                y = torch.empty((sn, sm), dtype=torch.float32, device=dev)
                units.append((acts, {L: Gemm(q6k, torch, acts, raw_d, sm, L, y, dev)
                                     for L in layouts}))
                del raw_d
    else:
        spec = synthetic.WORKLOADS[args.workload]
        n, m, k = spec["n"], spec["m"], spec["k"]
        if q4:
            raw = synthetic.weights_q4k(m, k, spec["seed"])
        else:
            raw = synthetic.weights(m, k, spec["seed"])
        up_d = None
        if args.swiglu:
            gate, up = synthetic.swiglu_inputs(n, k, spec["seed"])
            x_d, up_d = torch.from_numpy(gate).to(dev), torch.from_numpy(up).to(dev)
            x = None  # the CPU baseline quantizes x; here the input is the factor pair
        else:
            x = synthetic.activations(n, k, spec["seed"], args.activations or spec["x"])
            x_d = torch.from_numpy(x).to(dev)
        raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
        acts = Acts(q6k, torch, x_d, n, k, dev, up_d=up_d, q4=q4)
        y = torch.empty((n, m), dtype=torch.float32, device=dev)
        units.append((acts, {L: Gemm(q6k, torch, acts, raw_d, m, L, y, dev) for L in layouts}))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    if args.timeline:
        run_timeline(args, torch, units[0][0], units[0][1], layouts)
        return

    # load-time weight preparation of the first matrix in the headline layout, timed once
    a0, g0 = units[0][0], units[0][1][head]
    raw0 = (torch.from_numpy(raw.reshape(-1)).to(dev) if raw is not None
            else synthetic.weights_torch(g0.m, g0.k, 7, dev))
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_a.record(stream)
    if q4:
        q6k.q4k_expand_weights(raw0, g0.m, g0.k, g0.w)
    else:
        q6k.q6k_expand_weights(raw0, g0.m, g0.k, head, g0.w)
    e_b.record(stream)
    torch.cuda.synchronize()
    expand_us = e_a.elapsed_time(e_b) * 1e3
    del raw0

    if args.copy_probe_mib:
        # plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE readings calibrate the
        # GEMM's counter-based HBM traffic
        nel = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # 512 MiB written, then 1 GiB read, before each timed span: evicts the 256 MB Infinity Cache
    # and leaves it holding clean lines
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    scrub_rd = torch.ones(256 << 20, dtype=torch.float32, device=dev) if args.cold else None

    def cool():
        if scrub is not None:
            scrub.fill_(7)
            scrub_rd.sum()
            torch.cuda.synchronize()

    def step(evs=None):
        # evs[j] = events before the prepass, between prepass and GEMM, after the GEMM
        for j, (acts, gemms) in enumerate(units):
            if evs is not None:
                evs[j][0].record(stream)
            acts.quantize()
            if evs is not None:
                evs[j][1].record(stream)
            gemms[head].launch()
            if evs is not None:
                evs[j][2].record(stream)

    def gemm_pass(L):
        for _, gemms in units:
            gemms[L].launch()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ------------------------------------------------------------ warm-up
    for _ in range(args.warmup):
        step()
    for L in layouts:
        for _ in range(max(2, args.warmup // 10)):
            gemm_pass(L)
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed steps (no markers inside)
    if scrub is None:
        start, end = ev(), ev()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_per_step = start.elapsed_time(end) / args.steps
    else:
        step_ms, wall = [], 0.0
        for _ in range(args.steps):
            cool()
            s_ev, e_ev = ev(), ev()
            wall0 = time.perf_counter()
            s_ev.record(stream)
            step()
            e_ev.record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - wall0
            step_ms.append(s_ev.elapsed_time(e_ev))
        ms_per_step = float(np.mean(step_ms))

    # ------------------------------------------------------------ per-kernel breakdown of a step
    evs = [[[ev() for _ in range(3)] for _ in units] for _ in range(args.steps)]
    for i in range(args.steps):
        cool()
        step(evs[i])
    torch.cuda.synchronize()
    prep_us = np.array([[e[0].elapsed_time(e[1]) * 1e3 for e in st] for st in evs])
    stepgemm_us = np.array([[e[1].elapsed_time(e[2]) * 1e3 for e in st] for st in evs])
    prep_total_us = float(prep_us.sum(axis=1).mean())

    # ------------------------------------------------------------ GEMMs, layouts interleaved
    block = 1 if scrub is not None else max(1, args.block)
    per_launch = {L: [] for L in layouts}
    for r in range(args.steps):
        order = layouts[r % len(layouts):] + layouts[:r % len(layouts)]
        for L in order:
            cool()
            b0, b1 = ev(), ev()
            b0.record(stream)
            for _ in range(block):
                gemm_pass(L)
            b1.record(stream)
            if scrub is not None:
                torch.cuda.synchronize()
            per_launch[L].append((b0, b1))
    torch.cuda.synchronize()
    gemm_us = {L: np.array([b0.elapsed_time(b1) * 1e3 / block for b0, b1 in per_launch[L]])
               for L in layouts}  # per pass (one launch per matrix; 64 for the sweep)

    ops = sum(g[head].ops() for _, g in units)
    gmac = ops / 2e9
    prep_bytes = sum(a.bytes() for a, _ in units)

    # vector-ALU rate of the kernels' instruction forms, measured now on this GPU
    try:
        alu_meas, alu_best = alu_probe(torch)
    except (ImportError, RuntimeError, OSError) as exc:
        alu_meas, alu_best = {"error": str(exc)}, None

    lay_out = {}
    for L in layouts:
        us = gemm_us[L]
        mean = float(us.mean())
        tops = ops / (mean * 1e-6) / 1e12
        gb = sum(g[L].bytes() for _, g in units)
        valu = sum(g[L].valu_lane_ops() for _, g in units)
        lay_out[str(L)] = {
            "kernel": KERNEL_NAMES[L],
            "gemm_us_mean": round(mean, 2),
            "gemm_us_p10_p50_p90": [round(float(v), 2) for v in np.percentile(us, [10, 50, 90])],
            "tops": round(tops, 2), "us_per_gmac": round(mean / gmac, 4),
            "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
            "alg_bytes": int(gb), "alg_gbs": round(gb / (mean * 1e-6) / 1e9, 1),
            "weight_bytes": int(sum(g[L].w.numel() for _, g in units)),
            "valu_lane_ops_t_per_s": round(valu / (mean * 1e-6) / 1e12, 2),
            "valu_per_output": VALU_FORM[L],
        }
    hd = lay_out[str(head)]
    value = hd["tops"]
    gemm_head_us = hd["gemm_us_mean"]
    valu_head = sum(g[head].valu_lane_ops() for _, g in units)

    if sweep:
        config = {"workload": "sweep32", "layers": synthetic.SWEEP_LAYERS,
                  "gemms": "per layer: attn_v n=3314 m=4096 k=4096, ffn_down n=3314 m=4096 k=11008",
                  "layout": head, "cold": args.cold,
                  "step": "64 x (q6k_quantize_act + q6k_gemm)"}
    else:
        config = {"workload": args.workload, "n": g0.n, "m": g0.m, "k": g0.k, "layout": head,
                  "cold": args.cold, "step": "q6k_quantize_act + q6k_gemm"}
        if args.activations:
            config.update(activations=args.activations)
        if args.swiglu:
            config.update(producer="fused SwiGLU (gate, up f32 inputs)",
                          step="q6k_swiglu_quantize_act + q6k_gemm")
        if q4:
            config.update(weights="q4_K", step="q4k_quantize_act + q4k_gemm")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": config,
        "value_is": ("effective int8 TOPS (2*N*M*K / time) of the GEMM alone, kernel " +
                     KERNEL_NAMES[head] + "; mean per-launch time of the interleaved GEMM blocks"),
        "us_per_gmac": hd["us_per_gmac"],
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "step": {"ms": round(ms_per_step, 4), "tops": round(ops / (ms_per_step * 1e-3) / 1e12, 2),
                 "gemm_us_in_step_markers": round(float(stepgemm_us.sum(axis=1).mean()), 2),
                 "wall_s_timed": round(wall, 4)},
        "layouts": lay_out,
        "prepass": {"us_per_step": round(prep_total_us, 2),
                    "gbs": round(prep_bytes / (prep_total_us * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * prep_bytes / (prep_total_us * 1e-6) / 1e9
                                          / HBM_PEAK_GBS, 2)},
        "expand_us_once": {"m": g0.m, "k": g0.k, "layout": head, "us": round(expand_us, 1)},
        "setup_s": round(setup_s, 1),
        # the dominant kernel is the GEMM: algorithmic int8 ops over its event-timed duration
        "roofline": {"bound": "mfma", "achieved": value, "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(value / INT8_PEAK_TOPS, 4),
                     "traffic": (counter_traffic(args.workload, head)
                                 if not (sweep or args.cold or args.swiglu) else None),
                     "kernel": KERNEL_NAMES[head],
                     "algorithmic_per_launch": {"int8_ops": g0.ops(), "bytes": g0.bytes()}},
        # the unit that binds this method's GEMM: its f32 rescale on the vector ALU
        "alu_roofline": {
            "bound": "alu",
            "achieved": round(valu_head / (gemm_head_us * 1e-6) / 1e12, 2),
            "peak": round(alu_best, 2) if alu_best else round(VALU_SPEC_SINGLE, 1),
            "peak_is": ("best measured issue rate of the kernels' f32 instruction forms "
                        "(v_add_f32, v_fmac_f32, v_fma_f32) at 2 or 8 waves per SIMD, this run"
                        if alu_best else "spec, one wave64 instruction per SIMD per 4 cycles"),
            "unit": "T VALU lane-ops/s",
            "frac": round(valu_head / (gemm_head_us * 1e-6) / 1e12 /
                          (alu_best or VALU_SPEC_SINGLE), 4),
            "spec_single_issue": round(VALU_SPEC_SINGLE, 1),
            "spec_dual_issue": round(VALU_SPEC_DUAL, 1),
            "per_output": VALU_FORM[head],
            "algorithmic_per_launch": {"valu_lane_ops": g0.valu_lane_ops()},
            "measured": alu_meas},
    }
    if args.swiglu:
        # the unfused pair for comparison: h written by q6k_swiglu_f32, then q6k_quantize_act
        h = torch.empty((a0.n, a0.k), dtype=torch.float32, device=dev)
        e = [ev() for _ in range(3)]
        reps = 20
        for _ in range(3):
            q6k.q6k_swiglu_f32(a0.x, a0.up, h)
            q6k.q6k_quantize_act(h, a0.xq, a0.da)
        torch.cuda.synchronize()
        t_sw = t_q = 0.0
        for _ in range(reps):
            e[0].record(stream)
            q6k.q6k_swiglu_f32(a0.x, a0.up, h)
            e[1].record(stream)
            q6k.q6k_quantize_act(h, a0.xq, a0.da)
            e[2].record(stream)
            torch.cuda.synchronize()
            t_sw += e[0].elapsed_time(e[1]) * 1e3 / reps
            t_q += e[1].elapsed_time(e[2]) * 1e3 / reps
        out["producer"] = {"fused_us": out["prepass"]["us_per_step"],
                           "unfused_swiglu_us": round(t_sw, 2), "unfused_quantize_us": round(t_q, 2),
                           "unfused_total_us": round(t_sw + t_q, 2)}
    if not args.no_cpu_baseline and raw is not None and x is not None:
        out["cpu_baseline"] = cpu_baseline(raw, x, g0.m, g0.k, args.cpu_tokens, args.weights)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
