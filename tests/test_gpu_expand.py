"""GPU parity of q6k_expand_weights (all three layouts) against the oracle decode: byte-exact
codes, exact scales.  Shapes include those of the pages' byte-exactness test ("r53 — q6_K bundle:
W_exp pre-expansion plane + cp.async B staging (LANDED)", sec. 4: (64,256), (40,512), (24,768))."""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import round_up, untile_expanded, untile_folded, untile_packed

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256), (40, 512), (24, 768), (1, 256), (129, 1024), (256, 512)]


def raw_for(m, k, seed, wide=False):
    raw = synthetic.weights(m, k, seed, sc_lo=-128 if wide else -32, sc_hi=127 if wide else 31)
    if wide:  # special d values: subnormal, zero, negative, max
        d = raw.reshape(m, k // 256, 210)[:, :, 208:210]
        specials = [(0x01, 0x00), (0x00, 0x00), (0x00, 0xBC), (0xFF, 0x7B), (0xFF, 0x03)]
        for i, (lo, hi) in enumerate(specials):
            if i < d.shape[0]:
                d[i, 0] = (lo, hi)
    return raw


def check_expanded(raw, m, k):
    import gpu_util
    print(f"expand layout 1 m={m} k={k}", flush=True)
    w = gpu_util.expand(raw, m, k, 1).cpu().numpy()
    codes, dsc = untile_expanded(w, m, k)
    wc, sc, d = oracle.decode(raw, m, k)
    np.testing.assert_array_equal(codes[:m], wc)
    want = (np.repeat(d, 16, axis=1) * sc.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(dsc[:m].view(np.uint32), want.view(np.uint32))
    assert (codes[m:] == 0).all() and (dsc[m:] == 0).all()


def check_packed(raw, m, k):
    import gpu_util
    print(f"expand layout 0 m={m} k={k}", flush=True)
    w = gpu_util.expand(raw, m, k, 0).cpu().numpy()
    codes, dsc = untile_packed(w, m, k)
    wc, sc, d = oracle.decode(raw, m, k)
    np.testing.assert_array_equal(codes[:m].astype(np.int32) - 32, wc.astype(np.int32))
    want = (np.repeat(d, 16, axis=1) * sc.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(dsc[:m].view(np.uint32), want.view(np.uint32))
    assert (codes[m:] == 0).all() and (dsc[m:] == 0).all()
    assert w.size == round_up(m, 128) * k


def check_folded(raw, m, k):
    # the two digits must rebuild sc * (q - 32) exactly, with the low digit in [-32, 31] (which
    # makes the pair unique); d is the f16 d of each super-block as f32
    import gpu_util
    print(f"expand layout 2 m={m} k={k}", flush=True)
    w = gpu_util.expand(raw, m, k, 2).cpu().numpy()
    lo, hi, d = untile_folded(w, m, k)
    wc, sc, d_ref = oracle.decode(raw, m, k)
    v = np.repeat(sc.astype(np.int32), 16, axis=1) * wc.astype(np.int32)
    np.testing.assert_array_equal(64 * hi[:m].astype(np.int32) + lo[:m], v)
    assert lo.min() >= -32 and lo.max() <= 31
    np.testing.assert_array_equal(d[:m].view(np.uint32), d_ref.astype(np.float32).view(np.uint32))
    assert (lo[m:] == 0).all() and (hi[m:] == 0).all() and (d[m:] == 0).all()
    assert w.size == round_up(m, 128) * k * 2 + round_up(m, 128) * (k // 256) * 4


@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("wide", [False, True])
def test_expand_layouts_small(m, k, wide):
    raw = raw_for(m, k, seed=m * 7 + k, wide=wide)
    check_expanded(raw, m, k)
    check_packed(raw, m, k)
    check_folded(raw, m, k)


def test_expand_all_byte_values():
    # every byte value in every ql/qh position of a block, rows differ by a byte rotation
    m, k = 256, 256
    raw = np.zeros((m, 1, 210), np.uint8)
    for r in range(m):
        raw[r, 0, :192] = (np.arange(192) + r) % 256
        raw[r, 0, 192:208] = (np.arange(16) * 17 + r) % 256
        raw[r, 0, 208:210] = (0x00, 0x3C)
    check_expanded(raw, m, k)
    check_packed(raw, m, k)
    check_folded(raw, m, k)


@pytest.mark.parametrize("name", ["attn_v_n512", "ffn_down_n3314"])
def test_expand_full_size(name):
    import gpu_util
    raw, _, _, m, k = gpu_util.cached_workload(name)
    check_expanded(raw, m, k)
    check_packed(raw, m, k)
    check_folded(raw, m, k)
