"""Benchmark of the q6_K x int8 prefill hot path on one MI355X.

One step = one pass of the hot path over one batch: the activation quantize-transpose prepass
(q6k_quantize_act) followed by the GEMM (q6k_gemm) on weights prepared once at load time
(q6k_expand_weights, outside the timed region).  Inputs are synthetic, seeded, and resident in HBM
before timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout 0|1|2] [--workload NAME]
                    [--weights q6k|q4k] [--cold] [--swiglu] [--no-cpu-baseline]
                    [--copy-probe-mib MIB]

Workloads: tiny, attn_v_n512, attn_v_n3314, ffn_down_n3314 (the default and headline case),
ffn_down_shard8 (3314 x 512 x 11008: one GPU's share of ffn_down under an 8-way split of the
output rows), and sweep32: 32 layers of (attn_v 4096x4096 + ffn_down 4096x11008) at 3314 tokens, 64 GEMMs back to
back on one stream over 1.6 GB of raw weights, inputs drawn on the device.  --cold writes a
512 MiB scrub buffer and then reads a 1 GiB one before every timed step, so weights and
activations come from HBM rather than the 256 MB Infinity Cache (the read leaves the cache
holding clean lines: evicting the write's dirty lines inside the timed step would time their
write-back instead).  --swiglu (single workloads) replaces the prepass by the fused
producer q6k_swiglu_quantize_act reading the two SwiGLU factors, and also times the unfused pair
(q6k_swiglu_f32 writing h, then q6k_quantize_act) once for comparison.  --weights q4k runs the
q4_K variant on the same shapes (synthetic q4_K weights): step = q6k_quantize_act +
q4k_act_sums + q4k_gemm.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
# f32 VALU lane-operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, x 2 with dual
# issue (the published 157.3 TFLOP/s fp32 vector figure counts one FMA as 2 flops)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12
METRIC = "q6_K GEMM effective int8 TOPS + µs/GMAC, % of MFMA peak (ffn_down, N=3314)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~50 steps (~30 ms on ffn_down) bring the GPU's clock to its loaded steady state; with 5, the
    # first timed steps still run several percent slow
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layout", type=int, default=2, choices=[0, 1, 2])
    ap.add_argument("--workload", default="ffn_down_n3314")
    ap.add_argument("--weights", default="q6k", choices=["q6k", "q4k"],
                    help="weight format: q6_K (the headline) or the q4_K variant")
    ap.add_argument("--cold", action="store_true")
    ap.add_argument("--swiglu", action="store_true",
                    help="feed the GEMM from the fused SwiGLU -> int8 producer (gate, up inputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=768)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def cpu_baseline(raw, x, m, k, tokens, weights="q6k"):
    """The oracle as it stands (single-threaded C), on the first `tokens` tokens of the same
    workload, all rows: quantize + reference GEMM."""
    import oracle
    tokens = min(tokens, x.shape[0])
    xs = x[:tokens]
    t0 = time.perf_counter()
    xq, da = oracle.quantize(xs)
    (oracle.q4_gemm if weights == "q4k" else oracle.gemm)(xq, da, raw, m)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * tokens * m * k / dt / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"first {tokens} tokens x all {m} rows x k={k} (quantize + reference GEMM), "
                      f"{dt:.1f} s single-threaded",
            "host": host_cpu()}


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


def counter_traffic(workload, layout):
    """HBM-side bytes of one GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None if there is none for this workload or the kernel code changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_code_sha256_16") != kernel_source_digest():
        return None
    entry = rec.get("layouts", {}).get(str(layout))
    return None if entry is None else int(entry["traffic_bytes"])


class Q4Problem:
    """Device buffers of one q4_K GEMM (same activations path plus the per-chunk sums)."""

    def __init__(self, q6k, torch, x_d, raw_d, n, m, k, dev):
        self.q6k, self.n, self.m, self.k, self.layout = q6k, n, m, k, "q4k"
        self.x, self.up = x_d, None
        xb, db = q6k.q6k_act_bytes(n, k)
        self.xq = torch.empty(xb, dtype=torch.uint8, device=dev)
        self.da = torch.empty(db // 4, dtype=torch.float32, device=dev)
        self.das = torch.empty(db // 4, dtype=torch.float32, device=dev)
        self.w = torch.empty(q6k.q4k_weight_bytes(m, k), dtype=torch.uint8, device=dev)
        self.y = torch.empty((n, m), dtype=torch.float32, device=dev)
        q6k.q4k_expand_weights(raw_d, m, k, self.w)

    def quantize(self):
        self.q6k.q6k_quantize_act(self.x, self.xq, self.da)
        self.q6k.q4k_act_sums(self.xq, self.da, self.n, self.k, self.das)

    def gemm(self):
        self.q6k.q4k_gemm(self.xq, self.da, self.das, self.n, self.w, self.m, self.k, self.y)

    def alg_bytes(self):
        a_bytes = self.n * self.k + self.n * (self.k // 32) * 8
        return {"gemm": self.w.numel() + a_bytes + self.n * self.m * 4,
                "prepass": self.n * self.k * 4 + a_bytes}


class Problem:
    """Device buffers of one GEMM: activations, prepared weights, quantized activations, output."""

    def __init__(self, q6k, torch, x_d, raw_d, n, m, k, layout, dev, up_d=None):
        self.q6k, self.n, self.m, self.k, self.layout = q6k, n, m, k, layout
        self.x = x_d
        self.up = up_d  # with up: x is the gate and the producer is the fused SwiGLU quantize
        xb, db = q6k.q6k_act_bytes(n, k)
        self.xq = torch.empty(xb, dtype=torch.uint8, device=dev)
        self.da = torch.empty(db // 4, dtype=torch.float32, device=dev)
        self.w = torch.empty(q6k.q6k_weight_bytes(m, k, layout), dtype=torch.uint8, device=dev)
        self.y = torch.empty((n, m), dtype=torch.float32, device=dev)
        q6k.q6k_expand_weights(raw_d, m, k, layout, self.w)

    def quantize(self):
        if self.up is None:
            self.q6k.q6k_quantize_act(self.x, self.xq, self.da)
        else:
            self.q6k.q6k_swiglu_quantize_act(self.x, self.up, self.xq, self.da)

    def gemm(self):
        self.q6k.q6k_gemm(self.xq, self.da, self.n, self.w, self.layout, self.m, self.k, self.y)

    def alg_bytes(self):
        """Algorithmic bytes: GEMM = weights as stored + int8 activations + f32 scales + f32 Y;
        prepass = f32 X + int8 activations + f32 scales."""
        a_bytes = self.n * self.k + self.n * (self.k // 32) * 4
        x_bytes = self.n * self.k * (4 if self.up is None else 8)
        return {"gemm": self.w.numel() + a_bytes + self.n * self.m * 4,
                "prepass": x_bytes + a_bytes}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU split is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import q6_int8_prefill_amd as q6k

    dev = torch.device("cuda:0")
    layout = args.layout
    stream = torch.cuda.current_stream()
    sweep = args.workload == "sweep32"

    # ------------------------------------------------------------ inputs resident in HBM
    t0 = time.perf_counter()
    raw = x = None
    problems = []
    if sweep:
        for layer in range(synthetic.SWEEP_LAYERS):
            for kind in ("attn_v", "ffn_down"):
                raw_d, x_d, sn, sm, sk = synthetic.sweep_inputs_torch(layer, kind, dev)
                problems.append(Problem(q6k, torch, x_d, raw_d, sn, sm, sk, layout, dev))
                del raw_d
    elif args.swiglu:
        spec = synthetic.WORKLOADS[args.workload]
        n, m, k = spec["n"], spec["m"], spec["k"]
        raw = synthetic.weights(m, k, spec["seed"])
        gate, up = synthetic.swiglu_inputs(n, k, spec["seed"])
        raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
        problems.append(Problem(q6k, torch, torch.from_numpy(gate).to(dev), raw_d, n, m, k,
                                layout, dev, up_d=torch.from_numpy(up).to(dev)))
        raw = None  # the CPU baseline quantizes x; here the input is the factor pair
    elif args.weights == "q4k":
        spec = synthetic.WORKLOADS[args.workload]
        n, m, k = spec["n"], spec["m"], spec["k"]
        raw = synthetic.weights_q4k(m, k, spec["seed"])
        x = synthetic.activations(n, k, spec["seed"], spec["x"])
        problems.append(Q4Problem(q6k, torch, torch.from_numpy(x).to(dev),
                                  torch.from_numpy(raw.reshape(-1)).to(dev), n, m, k, dev))
    else:
        raw, x, n, m, k = synthetic.workload(args.workload)
        x_d = torch.from_numpy(x).to(dev)
        raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
        problems.append(Problem(q6k, torch, x_d, raw_d, n, m, k, layout, dev))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0

    # load-time weight preparation of the first matrix, timed once on its own
    p0 = problems[0]
    raw0 = (torch.from_numpy(raw.reshape(-1)).to(dev) if raw is not None
            else synthetic.weights_torch(p0.m, p0.k, 7, dev))
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_a.record(stream)
    if args.weights == "q4k" and not sweep:
        q6k.q4k_expand_weights(raw0, p0.m, p0.k, p0.w)
    else:
        q6k.q6k_expand_weights(raw0, p0.m, p0.k, layout, p0.w)
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

    # 512 MiB written, then 1 GiB read, between steps: evicts the 256 MB Infinity Cache and leaves
    # it holding clean lines
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    scrub_rd = torch.ones(256 << 20, dtype=torch.float32, device=dev) if args.cold else None

    def step(evs=None):
        # evs[j] = events before the prepass, between prepass and GEMM, after the GEMM
        for j, p in enumerate(problems):
            if evs is not None:
                evs[j][0].record(stream)
            p.quantize()
            if evs is not None:
                evs[j][1].record(stream)
            p.gemm()
            if evs is not None:
                evs[j][2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in problems]
           for _ in range(args.steps)]
    if scrub is None:
        # the timed steps carry no instrumentation: the per-kernel breakdown (and the GEMM time the
        # roofline uses) comes from the same number of steps run again with events between kernels
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_per_step = start.elapsed_time(end) / args.steps
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
    else:
        # cold: the scrub runs between steps, outside the timed span of each step
        step_ms, wall = [], 0.0
        for i in range(args.steps):
            scrub.fill_(i & 255)
            scrub_rd.sum()
            torch.cuda.synchronize()
            s_ev = torch.cuda.Event(enable_timing=True)
            e_ev = torch.cuda.Event(enable_timing=True)
            wall0 = time.perf_counter()
            s_ev.record(stream)
            step(evs[i])
            e_ev.record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - wall0
            step_ms.append(s_ev.elapsed_time(e_ev))
        ms_per_step = float(np.mean(step_ms))

    gemm_us = np.array([[e[1].elapsed_time(e[2]) * 1e3 for e in st] for st in evs])
    prep_us = np.array([[e[0].elapsed_time(e[1]) * 1e3 for e in st] for st in evs])
    gemm_total_us = float(gemm_us.sum(axis=1).mean())
    prep_total_us = float(prep_us.sum(axis=1).mean())

    ops = sum(2.0 * p.n * p.m * p.k for p in problems)

    def valu_lane_ops(p):
        # rescale work the method needs per launch (f32 lane-operations)
        if args.weights == "q4k" or layout != 2:
            per_chunk = 3 if args.weights == "q4k" else 4
            return float(p.n) * p.m * per_chunk * (p.k // 32)
        return float(p.n) * p.m * (3 * (p.k // 32) + p.k // 256)

    valu_ops = sum(valu_lane_ops(p) for p in problems)
    valu_form = ("3 per 32-k chunk: t = fma(F, d*sc, bias term), two fma with da and da*S"
                 if args.weights == "q4k" else
                 "4 per 32-k chunk: two halves x (fma with d*sc, fma with da)" if layout != 2 else
                 "3 per 32-k chunk (digit fold: two adds; fma with da) + 1 per super-block (d)")
    gmac = ops / 2e9
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_total_us * 1e-6) / 1e12
    gemm_bytes = sum(p.alg_bytes()["gemm"] for p in problems)
    prep_bytes = sum(p.alg_bytes()["prepass"] for p in problems)

    if sweep:
        config = {"workload": "sweep32", "layers": synthetic.SWEEP_LAYERS,
                  "gemms": "per layer: attn_v n=3314 m=4096 k=4096, ffn_down n=3314 m=4096 k=11008",
                  "layout": layout, "cold": args.cold,
                  "step": "64 x (q6k_quantize_act + q6k_gemm)"}
    else:
        config = {"workload": args.workload, "n": p0.n, "m": p0.m, "k": p0.k, "layout": layout,
                  "cold": args.cold, "step": "q6k_quantize_act + q6k_gemm"}
        if args.swiglu:
            config["producer"] = "fused SwiGLU (gate, up f32 inputs)"
        if args.weights == "q4k":
            config.update(weights="q4_K", layout="q4k planes",
                          step="q6k_quantize_act + q4k_act_sums + q4k_gemm")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
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
        "us_per_gmac": round(ms_per_step * 1e3 / gmac, 4),
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "gemm": {"avg_us": round(float(gemm_us.mean()), 2),
                 "min_us": round(float(gemm_us.min()), 2),
                 "p10_p50_p90_us_per_step": [round(float(v), 2) for v in
                                             np.percentile(gemm_us.sum(axis=1), [10, 50, 90])],
                 "total_us_per_step": round(gemm_total_us, 2),
                 "tops": round(gemm_tops, 2), "us_per_gmac": round(gemm_total_us / gmac, 4),
                 "pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
                 "alg_gbs": round(gemm_bytes / (gemm_total_us * 1e-6) / 1e9, 1)},
        "prepass": {"total_us_per_step": round(prep_total_us, 2),
                    "gbs": round(prep_bytes / (prep_total_us * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * prep_bytes / (prep_total_us * 1e-6) / 1e9
                                          / HBM_PEAK_GBS, 2)},
        "expand_us_once": {"m": p0.m, "k": p0.k, "us": round(expand_us, 1)},
        "weight_bytes": {"prepared_total": int(sum(p.w.numel() for p in problems))},
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
        # the dominant kernel is the GEMM: algorithmic int8 ops over its event-timed duration
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": (counter_traffic(args.workload, layout)
                                 if not (sweep or args.cold or args.weights == "q4k") else None),
                     "kernel": ("q4k_gemm_kernel" if args.weights == "q4k" else
                                "folded_kernel (layout 2)" if layout == 2 else
                                f"gemm_kernel<layout {layout}>"),
                     "algorithmic_per_launch": {"int8_ops": 2.0 * p0.n * p0.m * p0.k,
                                                "bytes": p0.alg_bytes()["gemm"]}},
        # the unit that binds this method's GEMM: its f32 rescale on the vector ALU
        "alu_roofline": {"bound": "alu", "achieved": round(valu_ops / (gemm_total_us * 1e-6) / 1e12, 2),
                         "peak": round(VALU_PEAK_TOPS, 1), "unit": "T VALU lane-ops/s",
                         "frac": round(valu_ops / (gemm_total_us * 1e-6) / 1e12 / VALU_PEAK_TOPS, 4),
                         "per_output": valu_form,
                         "algorithmic_per_launch": {"valu_lane_ops": valu_lane_ops(p0)}},
    }
    if args.swiglu:
        # the unfused pair for comparison: h written by q6k_swiglu_f32, then q6k_quantize_act
        h = torch.empty((p0.n, p0.k), dtype=torch.float32, device=dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        reps = 20
        for _ in range(3):
            q6k.q6k_swiglu_f32(p0.x, p0.up, h)
            q6k.q6k_quantize_act(h, p0.xq, p0.da)
        torch.cuda.synchronize()
        t_sw = t_q = 0.0
        for _ in range(reps):
            e[0].record(stream)
            q6k.q6k_swiglu_f32(p0.x, p0.up, h)
            e[1].record(stream)
            q6k.q6k_quantize_act(h, p0.xq, p0.da)
            e[2].record(stream)
            torch.cuda.synchronize()
            t_sw += e[0].elapsed_time(e[1]) * 1e3 / reps
            t_q += e[1].elapsed_time(e[2]) * 1e3 / reps
        out["producer"] = {"fused_us": out["prepass"]["total_us_per_step"],
                           "unfused_swiglu_us": round(t_sw, 2), "unfused_quantize_us": round(t_q, 2),
                           "unfused_total_us": round(t_sw + t_q, 2)}
        out["config"]["step"] = "q6k_swiglu_quantize_act + q6k_gemm"
    if not args.no_cpu_baseline and raw is not None:
        out["cpu_baseline"] = cpu_baseline(raw, x, p0.m, p0.k, args.cpu_sample_tokens,
                                           args.weights)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
