"""Benchmark of the q6_K x int8 prefill hot path on one MI355X.

One step = one pass of the hot path over one batch: the activation quantize-transpose prepass
(q6k_quantize_act) followed by the GEMM (q6k_gemm) on weights prepared once at load time
(q6k_expand_weights, outside the timed region).  Inputs are synthetic, seeded, and resident in HBM
before timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout 0|1] [--workload NAME]
                    [--no-cpu-baseline]
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
METRIC = "q6_K GEMM effective int8 TOPS + µs/GMAC, % of MFMA peak (ffn_down, N=3314)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layout", type=int, default=1, choices=[0, 1])
    ap.add_argument("--workload", default="ffn_down_n3314")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=160)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def cpu_baseline(raw, x, m, k, tokens):
    """The oracle as it stands (single-threaded C), on the first `tokens` tokens of the same
    workload, all rows: quantize + reference GEMM."""
    import oracle
    xs = x[:tokens]
    t0 = time.perf_counter()
    xq, da = oracle.quantize(xs)
    oracle.gemm(xq, da, raw, m)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * tokens * m * k / dt / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"first {tokens} tokens x all {m} rows x k={k} (quantize + reference GEMM), "
                      f"{dt:.1f} s single-threaded"}


def counter_traffic(workload, layout):
    """HBM-side bytes of one GEMM launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None if there is none for this workload or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    src = os.path.join(ROOT, "q6_int8_prefill_amd", "csrc", "q6k.hip")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    if rec.get("kernel_source_sha256_16") != digest:
        return None
    entry = rec.get("layouts", {}).get(str(layout))
    return None if entry is None else int(entry["traffic_bytes"])


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
    raw, x, n, m, k = synthetic.workload(args.workload)
    layout = args.layout

    # inputs resident in HBM
    x_d = torch.from_numpy(x).to(dev)
    raw_d = torch.from_numpy(raw.reshape(-1)).to(dev)
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.empty(xb, dtype=torch.uint8, device=dev)
    da = torch.empty(db // 4, dtype=torch.float32, device=dev)
    w = torch.empty(q6k.q6k_weight_bytes(m, k, layout), dtype=torch.uint8, device=dev)
    y = torch.empty((n, m), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    t0 = time.perf_counter()
    q6k.q6k_expand_weights(raw_d, m, k, layout, w)
    torch.cuda.synchronize()
    expand_ms = (time.perf_counter() - t0) * 1e3

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

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        q6k.q6k_quantize_act(x_d, xq, da)
        if ev is not None:
            ev[1].record(stream)
        q6k.q6k_gemm(xq, da, n, w, layout, m, k, y)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    prep_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    gemm_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    gemm_avg_us = float(gemm_ms.mean() * 1e3)
    prep_avg_us = float(prep_ms.mean() * 1e3)

    ops = 2.0 * n * m * k
    gmac = n * m * k / 1e9
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_avg_us * 1e-6) / 1e12
    # algorithmic bytes of one GEMM launch: weights as stored, int8 activations, f32 scales, f32 Y
    w_bytes = w.numel()
    a_bytes = n * k + n * (k // 32) * 4
    y_bytes = n * m * 4
    gemm_bytes = w_bytes + a_bytes + y_bytes
    prep_bytes = n * k * 4 + a_bytes

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
        "config": {"workload": args.workload, "n": n, "m": m, "k": k, "layout": layout,
                   "step": "q6k_quantize_act + q6k_gemm"},
        "us_per_gmac": round(ms_per_step * 1e3 / gmac, 4),
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "gemm": {"avg_us": round(gemm_avg_us, 2), "min_us": round(float(gemm_ms.min() * 1e3), 2),
                 "tops": round(gemm_tops, 2), "us_per_gmac": round(gemm_avg_us / gmac, 4),
                 "pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2)},
        "prepass": {"avg_us": round(prep_avg_us, 2),
                    "gbs": round(prep_bytes / (prep_avg_us * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * prep_bytes / (prep_avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)},
        "expand_ms_once": round(expand_ms, 3),
        "weight_bytes": {"raw": int(raw.size), "prepared": int(w_bytes)},
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": counter_traffic(args.workload, layout),
                     "kernel": f"gemm_kernel<layout {layout}>",
                     "algorithmic_per_launch": {"int8_ops": ops, "bytes": gemm_bytes}},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(raw, x, m, k, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
