"""Seeded synthetic inputs for the q6_K x int8 prefill GEMM.

Shared by the tests, the smoke check and the benchmark; it holds none of the method's
arithmetic: it only draws random bytes and floats with the shapes and value distributions of the
workloads (uniform ql/qh bytes, int8 sub-block scales in [-32, 31], f16 d = |N(0,1)| * 1e-2, and
N(0,1) activations, optionally with outlier channels or a post-SwiGLU-like product).

Draw order for a weight set: ql bytes, qh bytes, scales, d.  Activations are drawn from a separate
generator seeded with ``seed + 10**6`` so weights and activations can be regenerated independently.
"""
import numpy as np

QK = 256
BLOCK_BYTES = 210

# Workloads (N tokens, M output rows, K reduction) and their seeds.
WORKLOADS = {
    "tiny": dict(n=64, m=256, k=512, seed=1, x="normal"),
    "attn_v_n512": dict(n=512, m=4096, k=4096, seed=2, x="normal"),
    "attn_v_n3314": dict(n=3314, m=4096, k=4096, seed=3, x="outlier"),
    "ffn_down_n3314": dict(n=3314, m=4096, k=11008, seed=4, x="swiglu"),
    # one GPU's share of ffn_down under an 8-way split of the output rows (M / 8 = 512)
    "ffn_down_shard8": dict(n=3314, m=512, k=11008, seed=5, x="swiglu"),
}


def weights(m, k, seed, sc_lo=-32, sc_hi=31):
    """Raw q6_K blocks, uint8 [m][k/256][210].

    Byte map of a block: ql[128] at 0, qh[64] at 128, int8 scales[16] at 192, f16 d at 208."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nsb = k // QK
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = rng.integers(0, 256, size=(m, nsb, 128), dtype=np.uint8)
    qh = rng.integers(0, 256, size=(m, nsb, 64), dtype=np.uint8)
    sc = rng.integers(sc_lo, sc_hi + 1, size=(m, nsb, 16), dtype=np.int16).astype(np.int8)
    d = (np.abs(rng.standard_normal(size=(m, nsb))) * 1e-2).astype(np.float16)
    raw = np.empty((m, nsb, BLOCK_BYTES), np.uint8)
    raw[:, :, 0:128] = ql
    raw[:, :, 128:192] = qh
    raw[:, :, 192:208] = sc.view(np.uint8)
    raw[:, :, 208:210] = d.astype("<f2").view(np.uint8).reshape(m, nsb, 2)
    return raw


def activations(n, k, seed, kind="normal"):
    """f32 [n][k] activations.

    normal  : N(0,1)
    outlier : N(0,1) with round(0.01*k) seeded channels scaled by 20
    swiglu  : a * silu(b), a, b ~ N(0,1), silu evaluated in f64
    zero    : all zeros (the degenerate input: every chunk's codes and scale are 0)
    """
    if kind == "zero":
        return np.zeros((n, k), dtype=np.float32)
    rng = np.random.Generator(np.random.PCG64(seed + 10**6))
    if kind == "normal":
        return rng.standard_normal(size=(n, k), dtype=np.float32)
    if kind == "outlier":
        x = rng.standard_normal(size=(n, k), dtype=np.float32)
        ch = rng.choice(k, size=int(round(0.01 * k)), replace=False)
        x[:, ch] *= np.float32(20.0)
        return x
    if kind == "swiglu":
        a = rng.standard_normal(size=(n, k))
        b = rng.standard_normal(size=(n, k))
        t = np.negative(b)
        np.exp(t, out=t)
        t += 1.0
        np.divide(b, t, out=b)  # silu(b) = b / (1 + exp(-b)), in f64
        b *= a
        return b.astype(np.float32)
    raise ValueError(kind)


Q4K_BLOCK_BYTES = 144


def weights_q4k(m, k, seed):
    """Raw q4_K blocks uint8 [m][k/256][144]: qs uniform bytes, the 12 scale bytes uniform (every
    6-bit scale and min uniform in 0..63), then d and dmin = f16(|N(0,1)| * 1e-2), little-endian
    at bytes 0 and 2."""
    assert k % QK == 0
    nsb = k // QK
    rng = np.random.Generator(np.random.PCG64(seed + 5 * 10**6))
    raw = np.zeros((m, nsb, Q4K_BLOCK_BYTES), np.uint8)
    raw[:, :, 16:144] = rng.integers(0, 256, size=(m, nsb, 128), dtype=np.uint8)
    raw[:, :, 4:16] = rng.integers(0, 256, size=(m, nsb, 12), dtype=np.uint8)
    d = (np.abs(rng.standard_normal(size=(m, nsb))) * 1e-2).astype(np.float16)
    dmin = (np.abs(rng.standard_normal(size=(m, nsb))) * 1e-2).astype(np.float16)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(m, nsb, 2)
    raw[:, :, 2:4] = dmin.view(np.uint8).reshape(m, nsb, 2)
    return raw


def swiglu_inputs(n, k, seed):
    """(gate, up) f32 [n][k]: the two factors of the post-SwiGLU activations that
    activations(n, k, seed, "swiglu") forms in f64 (up = a, gate = b, same draws)."""
    rng = np.random.Generator(np.random.PCG64(seed + 10**6))
    a = rng.standard_normal(size=(n, k))
    b = rng.standard_normal(size=(n, k))
    return b.astype(np.float32), a.astype(np.float32)


def workload(name):
    """-> (raw weights, activations, n, m, k) for a named workload."""
    w = WORKLOADS[name]
    raw = weights(w["m"], w["k"], w["seed"])
    x = activations(w["n"], w["k"], w["seed"], w["x"])
    return raw, x, w["n"], w["m"], w["k"]


# ------------------------------------------------------------------------------------------------
# Device-side generators with the same distributions, for workloads too large to draw on the host
# (the 32-layer sweep).  They draw from torch's seeded CUDA generator, so their values differ from
# the numpy generators above; the sweep's parity tests copy these device draws to the host and
# hand them to the oracle.
# ------------------------------------------------------------------------------------------------
def weights_torch(m, k, seed, device, sc_lo=-32, sc_hi=31):
    """Raw q6_K blocks as a flat uint8 device tensor of m*(k/256)*210 bytes."""
    import torch
    nsb = k // QK
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    raw = torch.empty((m, nsb, BLOCK_BYTES), dtype=torch.uint8, device=device)
    raw[:, :, 0:192] = torch.randint(0, 256, (m, nsb, 192), generator=g, device=device,
                                     dtype=torch.int32).to(torch.uint8)
    sc = torch.randint(sc_lo, sc_hi + 1, (m, nsb, 16), generator=g, device=device, dtype=torch.int32)
    raw[:, :, 192:208] = sc.to(torch.int8).view(torch.uint8)
    d = (torch.randn((m, nsb), generator=g, device=device).abs() * 1e-2).to(torch.float16)
    raw[:, :, 208:210] = d.view(torch.uint8).reshape(m, nsb, 2)
    return raw.reshape(-1)


def activations_torch(n, k, seed, device, kind="normal"):
    """f32 [n][k] device activations with the distributions of activations()."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed + 10**6)
    if kind == "normal":
        return torch.randn((n, k), generator=g, device=device)
    if kind == "outlier":
        x = torch.randn((n, k), generator=g, device=device)
        ch = torch.randperm(k, generator=g, device=device)[: int(round(0.01 * k))]
        x[:, ch] *= 20.0
        return x
    if kind == "swiglu":
        a = torch.randn((n, k), generator=g, device=device, dtype=torch.float64)
        b = torch.randn((n, k), generator=g, device=device, dtype=torch.float64)
        return (a * (b * torch.sigmoid(b))).to(torch.float32)
    raise ValueError(kind)


SWEEP_LAYERS = 32


def sweep_layer(layer, kind):
    """Shape and seed of one GEMM of the 32-layer sweep: kind 'attn_v' (4096x4096, outlier
    activations, seed 1000+layer) or 'ffn_down' (4096x11008, post-SwiGLU-like, seed 2000+layer)."""
    if kind == "attn_v":
        return dict(n=3314, m=4096, k=4096, seed=1000 + layer, x="outlier")
    return dict(n=3314, m=4096, k=11008, seed=2000 + layer, x="swiglu")


def sweep_inputs_torch(layer, kind, device):
    """-> (raw weights flat uint8, activations f32 [n][k], n, m, k) of one sweep GEMM, drawn on the
    device; each draw has its own seeded generator, so a layer's inputs are the same whatever was
    drawn before them (the benchmark and the parity tests get identical values)."""
    s = sweep_layer(layer, kind)
    raw = weights_torch(s["m"], s["k"], s["seed"], device)
    x = activations_torch(s["n"], s["k"], s["seed"], device, s["x"])
    return raw, x, s["n"], s["m"], s["k"]
