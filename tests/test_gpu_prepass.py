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
