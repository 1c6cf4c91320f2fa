"""Pins of the oracle's gated RMS normalisation (y = weight * o / sqrt(mean(o^2) + eps)
* silu(z), over d_v) against closed forms: a one-hot vector, scale invariance, the gate's
known values, and the weight applied elementwise."""
import math

import numpy as np

import oracle


def test_one_hot_uses_the_mean_over_dv():
    dv = 16
    o = np.zeros((1, dv)); o[0, 3] = 2.5
    z = np.full((1, dv), math.log(3.0))          # sigmoid(ln 3) = 3/4
    w = np.linspace(0.5, 2.0, dv)
    y = oracle.gated_norm(o, z, w, eps=0.0)
    expect = np.zeros(dv)
    expect[3] = w[3] * math.sqrt(dv) * 0.75 * math.log(3.0)   # |o| / sqrt(o^2 / dv) = sqrt(dv)
    np.testing.assert_allclose(y[0], expect, rtol=1e-14, atol=1e-15)


def test_constant_vector_with_eps():
    dv, c, eps = 8, -0.3, 1e-2
    o = np.full((2, dv), c)
    y = oracle.gated_norm(o, np.full((2, dv), 20.0), np.ones(dv), eps=eps)
    silu20 = 20.0 / (1.0 + math.exp(-20.0))
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * silu20, rtol=1e-14)


def test_scale_invariance_and_zero_gate():
    rng = np.random.default_rng(0)
    o, z, w = rng.standard_normal((5, 32)), rng.standard_normal((5, 32)), rng.standard_normal(32)
    y1 = oracle.gated_norm(o, z, w, eps=0.0)
    y2 = oracle.gated_norm(7.0 * o, z, w, eps=0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    z[:, 5] = 0.0                                  # silu(0) = 0
    assert np.all(oracle.gated_norm(o, z, w)[:, 5] == 0.0)


def test_per_vector_normalisation():
    """Each (row, token, head) vector is normalised on its own: the rms of
    y / (weight * silu(z)) is 1 for every vector (eps = 0)."""
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 4, 2, 24)) * np.array([0.01, 1.0, 100.0])[:, None, None, None]
    z, w = rng.uniform(0.5, 2.0, o.shape), rng.uniform(0.5, 2.0, 24)
    y = oracle.gated_norm(o, z, w, eps=0.0)
    u = y / (w * z / (1.0 + np.exp(-z)))
    np.testing.assert_allclose(np.sqrt(np.mean(u * u, axis=-1)), 1.0, rtol=1e-13)
