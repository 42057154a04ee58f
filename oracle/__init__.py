"""CPU oracle for the q6_K x int8 prefill GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product package never imports it and shares no code with it.

The arithmetic lives in ``q6k_oracle.c`` and ``q4k_oracle.c`` (plain C loops, f64 where floating
point is not fixed by the pages); this module only marshals numpy arrays through ctypes.  Each
wrapper names the C function and, through it, the passage it follows.  The functions over many
output rows (or tokens) split them into contiguous ranges over ``threads`` host threads (default
``default_threads()``); the result is the same bit for bit for every thread count.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "q6k_oracle.c"), os.path.join(_HERE, "q4k_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "_build", "libq6k_oracle.so")
_lib = None

BLOCK_BYTES = 210
QK = 256


def build():
    """Compile the C oracle (gcc, IEEE f32 semantics: no fast-math)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                           "-ffp-contract=off", *_SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.q6o_f16_to_f64.restype = ctypes.c_double
        lib.q6o_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.q6o_code.restype = ctypes.c_int
        lib.q6o_code.argtypes = [p, ctypes.c_int]
        lib.q6o_decode.argtypes = [p, i64, i64, p, p, p]
        lib.q6o_dequant.argtypes = [p, i64, i64, p]
        ci = ctypes.c_int
        lib.q6o_quantize.argtypes = [p, i64, i64, p, p, ci]
        lib.q6o_subdots.argtypes = [p, p, i64, i64, i64, p, ci]
        lib.q6o_chunkdots.argtypes = [p, p, i64, i64, i64, p, ci]
        lib.q6o_swiglu.argtypes = [p, p, i64, p]
        lib.q4o_scale_min.argtypes = [p, ctypes.c_int, p, p]
        lib.q4o_code.restype = ctypes.c_int
        lib.q4o_code.argtypes = [p, ctypes.c_int]
        lib.q4o_decode.argtypes = [p, i64, i64, p, p, p, p, p]
        lib.q4o_dequant.argtypes = [p, i64, i64, p]
        lib.q4o_chunkdots.argtypes = [p, p, i64, i64, i64, p, ci]
        lib.q4o_chunksums.argtypes = [p, i64, i64, p]
        lib.q4o_gemm.argtypes = [p, p, i64, p, i64, i64, p, p, ci]
        lib.q6o_gemm.argtypes = [p, p, i64, p, i64, i64, p, p, ci]
        _lib = lib
    return _lib


def default_threads():
    """Host threads the oracle uses by default: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set (a shared host's share of its cores)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        avail = min(avail, int(cap))
    return max(1, avail)


def _threads(threads):
    return default_threads() if threads is None else max(1, int(threads))


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _raw(raw, m, k):
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if k % QK or raw.size != m * (k // QK) * BLOCK_BYTES:
        raise ValueError(f"raw q6_K buffer of {raw.size} B does not hold {m} x {k} weights")
    return raw


def f16_to_f64(h):
    """IEEE binary16 bits -> float (exact)."""
    return _load().q6o_f16_to_f64(int(h))


def code(block, e):
    """6-bit code of element e of one 210-byte block (per-element index map)."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size >= BLOCK_BYTES and 0 <= e < QK
    return _load().q6o_code(_ptr(b), int(e))


def decode(raw, m, k):
    """-> (wc int8 [m][k] centered codes, sc int8 [m][k/16], d f64 [m][k/256])."""
    raw = _raw(raw, m, k)
    wc = np.empty((m, k), np.int8)
    sc = np.empty((m, k // 16), np.int8)
    d = np.empty((m, k // QK), np.float64)
    _load().q6o_decode(_ptr(raw), m, k, _ptr(wc), _ptr(sc), _ptr(d))
    return wc, sc, d


def dequant(raw, m, k):
    """-> w f64 [m][k] = d * sc * (q - 32)."""
    raw = _raw(raw, m, k)
    w = np.empty((m, k), np.float64)
    _load().q6o_dequant(_ptr(raw), m, k, _ptr(w))
    return w


def quantize(x, threads=None):
    """f32 [n][k] -> (xq int8 [n][k], da f32 [n][k/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    xq = np.empty((n, k), np.int8)
    da = np.empty((n, k // 32), np.float32)
    _load().q6o_quantize(_ptr(x), n, k, _ptr(xq), _ptr(da), _threads(threads))
    return xq, da


def subdots(xq, raw, m, threads=None):
    """-> int32 [n][m][k/16] per-sub-block integer dots."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n, k = xq.shape
    raw = _raw(raw, m, k)
    out = np.empty((n, m, k // 16), np.int32)
    _load().q6o_subdots(_ptr(xq), _ptr(raw), n, m, k, _ptr(out), _threads(threads))
    return out


def swiglu(gate, up):
    """-> f64 array of up * silu(gate) (same shape), from f32 inputs."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    assert gate.shape == up.shape
    out = np.empty(gate.shape, np.float64)
    _load().q6o_swiglu(_ptr(gate), _ptr(up), gate.size, _ptr(out))
    return out


def chunkdots(xq, raw, m, threads=None):
    """-> int32 [n][m][k/32] per-chunk integer numerators with the sub-block scales applied."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n, k = xq.shape
    raw = _raw(raw, m, k)
    out = np.empty((n, m, k // 32), np.int32)
    _load().q6o_chunkdots(_ptr(xq), _ptr(raw), n, m, k, _ptr(out), _threads(threads))
    return out


def gemm(xq, da, raw, m, threads=None):
    """-> (y f64 [n][m], t f64 [n][m]): reference output and its tolerance scale sum |terms|."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    n, k = xq.shape
    assert da.shape == (n, k // 32)
    raw = _raw(raw, m, k)
    y = np.empty((n, m), np.float64)
    t = np.empty((n, m), np.float64)
    _load().q6o_gemm(_ptr(xq), _ptr(da), n, _ptr(raw), m, k, _ptr(y), _ptr(t), _threads(threads))
    return y, t


# ------------------------------------------------------------------------------------------------
# q4_K (q4k_oracle.c)
# ------------------------------------------------------------------------------------------------
Q4_BLOCK_BYTES = 144


def _raw4(raw, m, k):
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    assert raw.size == m * (k // QK) * Q4_BLOCK_BYTES, (raw.size, m, k)
    return raw


def q4_scale_min(scales12, j):
    """-> (sc, m) 6-bit pair of sub-block j from the 12 scale bytes."""
    s = np.ascontiguousarray(scales12, dtype=np.uint8)
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    _load().q4o_scale_min(_ptr(s), int(j), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def q4_code(block, e):
    """-> 4-bit code of element e of one 144-byte block."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    return int(_load().q4o_code(_ptr(b), int(e)))


def q4_decode(raw, m, k):
    """-> (codes uint8 [m][k], sc uint8 [m][k/32], mn uint8 [m][k/32], d f64 [m][k/256],
    dmin f64 [m][k/256])."""
    raw = _raw4(raw, m, k)
    codes = np.empty((m, k), np.uint8)
    sc = np.empty((m, k // 32), np.uint8)
    mn = np.empty((m, k // 32), np.uint8)
    d = np.empty((m, k // QK), np.float64)
    dmin = np.empty((m, k // QK), np.float64)
    _load().q4o_decode(_ptr(raw), m, k, _ptr(codes), _ptr(sc), _ptr(mn), _ptr(d), _ptr(dmin))
    return codes, sc, mn, d, dmin


def q4_dequant(raw, m, k):
    """-> f64 [m][k] dequantized q4_K weights."""
    raw = _raw4(raw, m, k)
    w = np.empty((m, k), np.float64)
    _load().q4o_dequant(_ptr(raw), m, k, _ptr(w))
    return w


def q4_chunkdots(xq, raw, m, threads=None):
    """-> int32 [n][m][k/32] integer dots of the activation codes with the 4-bit weight codes."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n, k = xq.shape
    raw = _raw4(raw, m, k)
    out = np.empty((n, m, k // 32), np.int32)
    _load().q4o_chunkdots(_ptr(xq), _ptr(raw), n, m, k, _ptr(out), _threads(threads))
    return out


def q4_chunksums(xq):
    """-> int32 [n][k/32] sums of each chunk's activation codes."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    n, k = xq.shape
    out = np.empty((n, k // 32), np.int32)
    _load().q4o_chunksums(_ptr(xq), n, k, _ptr(out))
    return out


def q4_gemm(xq, da, raw, m, threads=None):
    """-> (y f64 [n][m], t f64 [n][m]) for q4_K weights."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    n, k = xq.shape
    assert da.shape == (n, k // 32)
    raw = _raw4(raw, m, k)
    y = np.empty((n, m), np.float64)
    t = np.empty((n, m), np.float64)
    _load().q4o_gemm(_ptr(xq), _ptr(da), n, _ptr(raw), m, k, _ptr(y), _ptr(t), _threads(threads))
    return y, t
