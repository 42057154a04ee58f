"""Test-side views of the library's tiled buffers (byte order as documented in include/q6k.h).

These only reorder bytes; they hold none of the method's arithmetic.
"""
import numpy as np


def round_up(v, q):
    return (v + q - 1) // q * q


def untile_xq(buf, n, k):
    """tiled xq bytes -> int8 [NP][k] (NP = n rounded up to 128)."""
    np_ = round_up(n, 128)
    nchunk = k // 32
    t = np.asarray(buf, np.uint8)[: np_ * k].view(np.int8).reshape(np_ // 32, nchunk, 2, 32, 2, 8)
    # axes: T, c, g, p, h, e  ->  token 32T + p, k = 32c + 16h + 8g + e
    return t.transpose(0, 3, 1, 4, 2, 5).reshape(np_, k)


def untile_da(buf, n, k):
    """tiled da floats -> f32 [NP][k/32]."""
    np_ = round_up(n, 128)
    nchunk = k // 32
    t = np.asarray(buf, np.float32)[: np_ * nchunk].reshape(np_ // 32, nchunk, 2, 4, 4)
    # axes: T, c, g, q, r -> token 32T + 8q + 4g + r
    return t.transpose(0, 3, 2, 4, 1).reshape(np_, nchunk)


def untile_expanded(buf, m, k):
    """layout 1 bytes -> (codes int8 [MP][k], dsc f32 [MP][k/16])."""
    mp = round_up(m, 128)
    nchunk = k // 32
    b = np.asarray(buf, np.uint8)
    codes = b[: mp * k].view(np.int8).reshape(mp // 32, nchunk, 2, 32, 2, 8)
    codes = codes.transpose(0, 3, 1, 4, 2, 5).reshape(mp, k)
    sc = b[mp * k: mp * k + mp * (k // 16) * 4].view(np.float32).reshape(mp // 32, nchunk, 32, 2)
    dsc = sc.transpose(0, 2, 1, 3).reshape(mp, k // 16)
    return codes, dsc


def untile_packed(buf, m, k):
    """layout 0 bytes -> (6-bit codes uint8 [MP][k], dsc f32 [MP][k/16]).

    Per lane three words X, Y, Z: byte t of X / Y / Z holds a_t / a_{t+4} / b_t in bits 2-7 and
    bits 0-1 / 2-3 / 4-5 of b_{t+4} in bits 0-1."""
    mp = round_up(m, 128)
    nchunk = k // 32
    b = np.asarray(buf, np.uint8)
    nb = mp * k * 3 // 4
    w = b[:nb].reshape(mp // 32, nchunk, 2, 32, 3, 4).astype(np.int32)  # T,c,g,p,word,byte
    x, y, z = w[..., 0, :], w[..., 1, :], w[..., 2, :]
    a = np.zeros(x.shape[:-1] + (8,), np.int32)
    bb = np.zeros_like(a)
    a[..., 0:4] = x >> 2
    a[..., 4:8] = y >> 2
    bb[..., 0:4] = z >> 2
    bb[..., 4:8] = (x & 3) | ((y & 3) << 2) | ((z & 3) << 4)
    full = np.stack([a, bb], axis=4)  # T,c,g,p,h,e
    codes = full.transpose(0, 3, 1, 4, 2, 5).reshape(mp, k).astype(np.uint8)
    sc = b[nb: nb + mp * (k // 16) * 4].view(np.float32).reshape(mp // 32, nchunk, 32, 2)
    return codes, sc.transpose(0, 2, 1, 3).reshape(mp, k // 16)


def untile_folded(buf, m, k):
    """layout 2 bytes -> (low digits int8 [MP][k], high digits int8 [MP][k], d f32 [MP][k/256])."""
    mp = round_up(m, 128)
    nchunk = k // 32
    b = np.asarray(buf, np.uint8)
    planes = b[: mp * k * 2].view(np.int8).reshape(mp // 32, nchunk, 2, 2, 32, 2, 8)
    # axes: R, c, h (digit), g, p, hh, e  ->  row 32R + p, k = 32c + 16hh + 8g + e
    planes = planes.transpose(2, 0, 4, 1, 5, 3, 6).reshape(2, mp, k)
    nsb = k // 256
    d = b[mp * k * 2: mp * k * 2 + mp * nsb * 4].view(np.float32).reshape(mp // 32, nsb, 32)
    return planes[0], planes[1], d.transpose(0, 2, 1).reshape(mp, nsb)


def untile_q4k(buf, m, k):
    """q4_K prepared weights -> (codes uint8 [MP][k], pairs f32 [MP][k/32][2] = (d*sc, -dmin*m))."""
    mp = round_up(m, 128)
    nchunk = k // 32
    b = np.asarray(buf, np.uint8)
    codes = b[: mp * k].reshape(mp // 32, nchunk, 2, 32, 2, 8)
    codes = codes.transpose(0, 3, 1, 4, 2, 5).reshape(mp, k)
    nsb = k // 256
    pr = b[mp * k: mp * k + mp * nchunk * 8].view(np.float32).reshape(mp // 32, nsb, 8, 32, 2)
    pairs = pr.transpose(0, 3, 1, 2, 4).reshape(mp, nchunk, 2)
    return codes, pairs


def untile_xq_tile(buf, tile, k):
    """The 32 tokens of token tile `tile` from tiled xq bytes -> int8 [32][k]."""
    nchunk = k // 32
    b = np.asarray(buf, np.uint8)[tile * nchunk * 1024: (tile + 1) * nchunk * 1024]
    # axes: c, g, p, h, e  ->  token p, k = 32c + 16h + 8g + e
    return b.view(np.int8).reshape(nchunk, 2, 32, 2, 8).transpose(2, 0, 3, 1, 4).reshape(32, k)


def untile_da_tile(buf, tile, k):
    """The 32 tokens of token tile `tile` from tiled da floats -> f32 [32][k/32]."""
    nchunk = k // 32
    t = np.asarray(buf, np.float32)[tile * nchunk * 32: (tile + 1) * nchunk * 32]
    # axes: c, g, q, r  ->  token 8q + 4g + r
    return t.reshape(nchunk, 2, 4, 4).transpose(2, 1, 3, 0).reshape(32, nchunk)
