"""Shared helpers for GPU tests: upload, run the library's entry points, fetch results."""
import functools

import numpy as np
import torch

import q6_int8_prefill_amd as q6k
import synthetic

DEV = torch.device("cuda:0")


def quantize(x, ldx=None):
    n, k = x.shape
    xb, db = q6k.q6k_act_bytes(n, k)
    if ldx is not None and ldx != k:
        xp = np.zeros((n, ldx), np.float32)
        xp[:, :k] = x
        xg = torch.from_numpy(xp).to(DEV)[:, :k]
    else:
        xg = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    xq = torch.full((xb,), 0xA5, dtype=torch.uint8, device=DEV)  # poison: padding must be zeroed
    da = torch.full((db // 4,), float("nan"), dtype=torch.float32, device=DEV)
    q6k.q6k_quantize_act(xg, xq, da, n=n, k=k, ldx=xg.stride(0))
    return xq, da


def quantize_device(xg):
    """Prepass of an f32 [n][k] device tensor."""
    n, k = xg.shape
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.full((xb,), 0xA5, dtype=torch.uint8, device=DEV)
    da = torch.full((db // 4,), float("nan"), dtype=torch.float32, device=DEV)
    q6k.q6k_quantize_act(xg, xq, da)
    return xq, da


def expand_device(wr, m, k, layout):
    """Weight preparation from raw q6_K bytes already on the device."""
    w = torch.full((q6k.q6k_weight_bytes(m, k, layout),), 0x5A, dtype=torch.uint8, device=DEV)
    q6k.q6k_expand_weights(wr, m, k, layout, w)
    return w


def expand(raw, m, k, layout):
    wr = torch.from_numpy(np.ascontiguousarray(raw).reshape(-1)).to(DEV)
    w = torch.full((q6k.q6k_weight_bytes(m, k, layout),), 0x5A, dtype=torch.uint8, device=DEV)
    q6k.q6k_expand_weights(wr, m, k, layout, w)
    return w


def gemm(xq, da, n, w, layout, m, k, ldy=None):
    ldy = m if ldy is None else ldy
    y = torch.full((n, ldy), float("nan"), dtype=torch.float32, device=DEV)
    q6k.q6k_gemm(xq, da, n, w, layout, m, k, y, ldy=ldy)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def subdots(xq, da, n, w, layout, m, k, tok0=0, ntok=None, row0=0, nrow=None):
    """int32 [ntok][nrow][k/16] sub-block dots of a window (default: the whole problem)."""
    ntok = n - tok0 if ntok is None else ntok
    nrow = m - row0 if nrow is None else nrow
    dots = torch.full((ntok, nrow, k // 16), -7, dtype=torch.int32, device=DEV)
    q6k.q6k_gemm_subdots(xq, da, n, w, layout, m, k, dots, tok0=tok0, ntok=ntok, row0=row0,
                         nrow=nrow)
    torch.cuda.synchronize()
    return dots.cpu().numpy()


def chunkdots(xq, da, n, w, layout, m, k, tok0=0, ntok=None, row0=0, nrow=None):
    """int32 [ntok][nrow][k/32] per-chunk numerators of a window (default: the whole problem)."""
    ntok = n - tok0 if ntok is None else ntok
    nrow = m - row0 if nrow is None else nrow
    dots = torch.full((ntok, nrow, k // 32), -7, dtype=torch.int32, device=DEV)
    q6k.q6k_gemm_chunkdots(xq, da, n, w, layout, m, k, dots, tok0=tok0, ntok=ntok, row0=row0,
                           nrow=nrow)
    torch.cuda.synchronize()
    return dots.cpu().numpy()


def raw_rows(raw, m, k, row0, nrow):
    """The raw q6_K blocks of rows [row0, row0 + nrow) (a byte slice, no arithmetic)."""
    return np.ascontiguousarray(np.asarray(raw).reshape(m, k // 256, 210)[row0:row0 + nrow])


def within_tolerance(y, y_ref, t_ref, rel=1e-3):
    """|y - y_ref| <= rel * sum|terms| elementwise (t_ref = 0 demands y = 0)."""
    err = np.abs(y.astype(np.float64) - y_ref)
    ok = err <= rel * t_ref
    return bool(ok.all()), float((err / np.maximum(t_ref, 1e-300)).max())


@functools.lru_cache(maxsize=2)
def cached_workload(name):
    """synthetic.workload(name), generated once per test session."""
    return synthetic.workload(name)
