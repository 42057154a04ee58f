"""GPU parity of q6k_quantize_act against the oracle: bit-exact int8 codes and f32 scales."""
import numpy as np
import pytest

import oracle
import synthetic
from layouts import round_up, untile_da, untile_xq

pytestmark = pytest.mark.gpu


def check(x, ldx=None):
    import gpu_util
    n, k = x.shape
    print(f"prepass case n={n} k={k} ldx={ldx}", flush=True)
    xq, da = gpu_util.quantize(x, ldx=ldx)
    xq_ref, da_ref = oracle.quantize(x)
    got_q = untile_xq(xq.cpu().numpy(), n, k)
    got_d = untile_da(da.cpu().numpy(), n, k)
    np.testing.assert_array_equal(got_q[:n], xq_ref)
    np.testing.assert_array_equal(got_d[:n].view(np.uint32), da_ref.view(np.uint32))
    # padding tokens are zeros
    assert (got_q[n:] == 0).all() and (got_d[n:] == 0).all()
    assert got_q.shape[0] == round_up(n, 128)


@pytest.mark.parametrize("n,k,kind", [(64, 512, "normal"), (65, 768, "outlier"), (1, 256, "swiglu"),
                                      (128, 256, "normal"), (300, 1024, "swiglu")])
def test_prepass_small(n, k, kind):
    check(synthetic.activations(n, k, seed=n + k, kind=kind))


def test_prepass_leading_dimension():
    check(synthetic.activations(33, 512, seed=9), ldx=520)


def test_prepass_special_values():
    x = np.zeros((40, 256), np.float32)
    x[0, :8] = [127, -127, 2.5, -2.5, 0.5, -0.5, 1.5, 126.5]     # ties go away from zero
    x[1, 32:64] = 1e-40                                           # subnormal chunk
    x[2, 64] = 1e-45                                              # amax/127 underflows to 0
    x[3, :32] = np.linspace(-1, 1, 32)
    x[4, :] = 3.0e38                                              # huge but finite
    x[5, 100] = -7.0                                              # single nonzero
    rng = np.random.default_rng(1)
    x[6:] = rng.standard_normal((34, 256)).astype(np.float32) * 1e-30
    # exact ties x/da = j + 0.5: with amax = 127*s, x = (j + 0.5) * s for a power of two s
    for j in range(20):
        x[6 + j, 0] = 127 * 0.25
        x[6 + j, 1] = (j + 0.5) * 0.25
        x[6 + j, 2] = -(j + 0.5) * 0.25
    check(x)


@pytest.mark.parametrize("name", ["ffn_down_n3314", "attn_v_n3314"])
def test_prepass_full_size(name):
    import gpu_util
    check(gpu_util.cached_workload(name)[1])


def test_prepass_near_ties():
    """Values whose quotient x / da lies within a few ulps of a half-integer, on either side and
    exactly on it, for scales that are not powers of two: the codes must still be those of
    roundf on the correctly rounded quotient (the kernel's fast reciprocal path must hand every
    such value to the exact division)."""
    rng = np.random.default_rng(11)
    n, k = 64, 2048
    x = np.zeros((n, k), np.float32)
    for t in range(n):
        for c in range(k // 32):
            amax = np.float32(rng.uniform(0.5, 4.0) * 10.0 ** rng.integers(-20, 20))
            da = np.float32(amax / np.float32(127.0))
            row = np.empty(32, np.float32)
            row[0] = amax
            for i in range(1, 32):
                j = rng.integers(0, 127)
                target = np.float32((j + 0.5) * np.float64(da))
                steps = int(rng.integers(-3, 4))
                v = target
                for _ in range(abs(steps)):
                    v = np.nextafter(v, np.float32(np.inf if steps > 0 else -np.inf), dtype=np.float32)
                row[i] = v if rng.integers(0, 2) else -v
            x[t, 32 * c: 32 * c + 32] = row
    check(x)


def test_prepass_more_token_tiles_than_one_launch_holds():
    """Over 65535 token tiles (2,097,120 tokens) the prepass is issued as several launches with a
    token-tile offset: tiles on both sides of the seam, the last real tile and the zero padding
    tiles are checked bit for bit against the oracle (k = 256: 2.1 GB of activations)."""
    import torch
    import gpu_util
    import q6_int8_prefill_amd as q6k
    from layouts import untile_da_tile, untile_xq_tile
    n, k = 65535 * 32 + 45, 256
    print(f"prepass multi-launch n={n} k={k}", flush=True)
    x = synthetic.activations_torch(n, k, 31, gpu_util.DEV, "outlier")
    xb, db = q6k.q6k_act_bytes(n, k)
    xq = torch.full((xb,), 0xA5, dtype=torch.uint8, device=gpu_util.DEV)
    da = torch.full((db // 4,), float("nan"), dtype=torch.float32, device=gpu_util.DEV)
    q6k.q6k_quantize_act(x, xq, da)
    torch.cuda.synchronize()
    ntiles = round_up(n, 128) // 32
    last = (n - 1) // 32
    tiles = sorted({0, 1, 65533, 65534, 65535, 65536, last} |
                   set(np.random.default_rng(3).integers(0, last, 4).tolist()))
    nchunk = k // 32
    for t in tiles:
        lo, hi = 32 * t, min(32 * t + 32, n)
        xs = x[lo:hi].cpu().numpy()
        q_ref, d_ref = oracle.quantize(xs)
        qb = xq[t * nchunk * 1024:(t + 1) * nchunk * 1024].cpu().numpy()
        dbuf = da[t * nchunk * 32:(t + 1) * nchunk * 32].cpu().numpy()
        got_q = untile_xq_tile(qb, 0, k)
        got_d = untile_da_tile(dbuf, 0, k)
        np.testing.assert_array_equal(got_q[:hi - lo], q_ref, err_msg=f"tile {t}")
        np.testing.assert_array_equal(got_d[:hi - lo].view(np.uint32), d_ref.view(np.uint32),
                                      err_msg=f"tile {t}")
        assert (got_q[hi - lo:] == 0).all() and (got_d[hi - lo:] == 0).all()
    for t in range(last + 1, ntiles):  # padding tiles
        assert (xq[t * nchunk * 1024:(t + 1) * nchunk * 1024] == 0).all()
        assert (da[t * nchunk * 32:(t + 1) * nchunk * 32] == 0).all()
