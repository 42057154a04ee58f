"""bench.py's contract on the host: more than one GPU is refused with a message (the GEMM runs on
one GPU), so are option combinations that would time something else than they name, and the
HBM traffic and fetch it reports come from the committed counter summary only while that summary
was taken on the current kernel code."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_only_for_the_profiled_kernel_code(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    real = bench.kernel_source_digest()
    assert len(real) == 16
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: real)
    t = bench.counter_traffic("ffn_down_n3314", 2)
    import json
    with open(os.path.join(ROOT, "profiles", "ffn_down_n3314_traffic.json")) as f:
        rec = json.load(f)
    if rec["kernel_code_sha256_16"] == real:
        assert t == rec["layouts"]["2"]["traffic_bytes"] and t > rec["layouts"]["2"]["algorithmic_bytes"]
    else:
        assert t is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.counter_traffic("ffn_down_n3314", 2) is None
    assert bench.counter_traffic("no_such_workload", 2) is None


def test_conflicting_modes_are_refused():
    for extra in (["--swiglu", "--activations", "zero"],
                  ["--workload", "sweep32", "--activations", "normal"],
                  ["--workload", "sweep32", "--timeline"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + extra,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, extra
        assert "bench.py:" in r.stderr


def test_fetch_only_for_the_profiled_kernel_code(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    import json
    with open(os.path.join(ROOT, "profiles", "ffn_down_n3314_traffic.json")) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: rec["kernel_code_sha256_16"])
    e = rec["layouts"]["2"]
    fetch = bench.counter_fetch("ffn_down_n3314", 2)
    assert fetch == int(e["gemm_fetch_size_kib"] * 1024 * rec["fetch_scale"])
    assert fetch < e["traffic_bytes"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.counter_fetch("ffn_down_n3314", 2) is None
