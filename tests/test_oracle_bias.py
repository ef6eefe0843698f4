"""Pins of the oracle's aux-loss-free balancing step: the expert bias moves by
gamma towards balance after each batch ("Reflection AI Introduces Beam ..."
load-balancing paragraph: DeepSeek-V3's bias-update balancing with a cosine
decay of the update speed)."""
import math

import numpy as np

import oracle
from synth import BEAM


def test_closed_form_on_crafted_loads():
    # E = 4, T = 3, K = 2: mean load 1.5
    idx = np.array([[0, 1], [0, 2], [0, 1]], np.int32)   # loads 3, 2, 1, 0
    b = oracle.bias_update(4, idx, 0.25, np.zeros(4, np.float32))
    np.testing.assert_array_equal(b, np.array([-0.25, -0.25, 0.25, 0.25], np.float32))
    # exactly balanced: no change
    idx = np.array([[0, 1], [2, 3]], np.int32)
    b0 = np.array([0.1, -0.2, 0.3, 0.0], np.float32)
    np.testing.assert_array_equal(oracle.bias_update(4, idx, 0.5, b0), b0)


def test_cosine_gamma():
    assert oracle.bias_gamma(0, 100, 1e-3, 1e-5) == np.float32(1e-3)
    assert abs(oracle.bias_gamma(100, 100, 1e-3, 1e-5) - 1e-5) < 1e-12
    mid = oracle.bias_gamma(50, 100, 1e-3, 1e-5)
    assert abs(mid - (1e-5 + (1e-3 - 1e-5) * 0.5)) < 1e-9
    g = [oracle.bias_gamma(t, 100, 1e-3, 1e-5) for t in range(101)]
    assert all(a >= b for a, b in zip(g, g[1:]))


def test_rounds_drive_load_towards_balance():
    # Fixed logits with a strong skew; repeated route + update rounds must
    # bring the most-loaded expert down towards the mean.
    rng = np.random.default_rng(0)
    T = 2048
    lg = (rng.standard_normal((T, 256)) + np.where(np.arange(256) < 16, 1.0, 0.0)).astype(np.float32)
    bias = np.zeros(256, np.float32)

    def maxmean(b):
        idx, _, _ = oracle.route(BEAM, lg, b)
        c = np.bincount(idx.ravel(), minlength=256)
        return c.max() / c.mean(), idx
    r0, idx = maxmean(bias)
    for t in range(60):
        bias = oracle.bias_update(256, idx, oracle.bias_gamma(t, 60, 0.02, 0.002), bias)
        r, idx = maxmean(bias)
    assert r0 > 3.0
    assert r < 1.6, r
