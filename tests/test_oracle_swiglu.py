"""Pins for the oracle's SwiGLU product h = up * silu(gate) (CPU only), the input of the fused
quantize producer.  Checked against closed forms of the logistic function, not against itself:
  * silu(0) = 0 and silu(ln 3) = (3/4) ln 3, silu(-ln 3) = -(1/4) ln 3 (sigma(ln 3) = 3/4);
  * the reflection silu(-g) = silu(g) - g;
  * the limits silu(g) -> g for large g and -> 0 for very negative g;
  * h is linear in up (h(g, 2u) = 2 h(g, u), h(g, 0) = 0).
"""
import math

import numpy as np


def test_closed_forms(oracle_mod):
    g = np.array([0.0, math.log(3.0), -math.log(3.0)], np.float32)
    u = np.ones_like(g)
    h = oracle_mod.swiglu(g, u)
    gl = float(np.float32(math.log(3.0)))  # the f32 input actually passed
    sig = 1.0 / (1.0 + math.exp(-gl))
    assert h[0] == 0.0
    assert abs(h[1] - gl * sig) <= 1e-15
    assert abs(sig - 0.75) < 1e-7
    assert abs(h[2] + gl * (1.0 - sig)) <= 1e-15


def test_reflection_and_limits(oracle_mod):
    rng = np.random.default_rng(3)
    g = rng.standard_normal(1000).astype(np.float32) * 4
    u = np.ones_like(g)
    pos = oracle_mod.swiglu(g, u)
    neg = oracle_mod.swiglu(-g, u)
    np.testing.assert_allclose(neg, pos - g.astype(np.float64), rtol=0, atol=1e-12)
    big = np.array([40.0, 80.0], np.float32)
    np.testing.assert_allclose(oracle_mod.swiglu(big, np.ones_like(big)), big.astype(np.float64), rtol=1e-15)
    tiny = oracle_mod.swiglu(np.array([-80.0], np.float32), np.ones(1, np.float32))
    assert 0 > tiny[0] > -1e-30


def test_linear_in_up(oracle_mod):
    rng = np.random.default_rng(4)
    g = rng.standard_normal(500).astype(np.float32)
    u = rng.standard_normal(500).astype(np.float32)
    np.testing.assert_array_equal(oracle_mod.swiglu(g, 2 * u), 2 * oracle_mod.swiglu(g, u))
    assert (oracle_mod.swiglu(g, np.zeros_like(u)) == 0).all()
