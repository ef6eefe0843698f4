"""Pins of the oracle's post-block epilogue: RMSNorm of the block output and
the depth-scaled residual stream ("Reflection Beam", section "Hybrid
Attention and Unusual Residuals": the stream is multiplied by sqrt((k-1)/k)
and the sublayer output added with weight 1/sqrt(k), so the squared weights
sum to one and after K steps every addend carries the same weight)."""
import numpy as np
import pytest

import oracle



def _rows_with_rms(rng, T, H, rms):
    """Rows whose mean square is exactly rms^2: +-rms entries."""
    return rms * rng.choice([-1.0, 1.0], size=(T, H))


def test_telescoped_stream():
    # the norm of a +-c row is known exactly; K steps give
    # r_K = (n_1 + ... + n_K) / sqrt(K): each addend the same weight 1/sqrt(K)
    rng = np.random.default_rng(0)
    T, H, K, c, eps = 3, 64, 12, 0.75, 1e-6
    gamma = np.full(H, np.sqrt(c * c + eps), np.float64).astype(np.float32)
    g64 = gamma.astype(np.float64)
    r = rng.standard_normal((T, H))          # discarded at step 1 (weight 0)
    total = np.zeros((T, H))
    for k in range(1, K + 1):
        u = _rows_with_rms(rng, T, H, c)
        total += u / np.sqrt(c * c + eps) * g64   # the norm of a +-c row
        r = oracle.residual_epilogue(u, gamma, eps, k, r)
    np.testing.assert_allclose(r, total / np.sqrt(K), rtol=1e-12, atol=1e-12)


def test_step_one_discards_stream():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((4, 32))
    gamma = rng.uniform(0.5, 1.5, 32).astype(np.float32)
    r0 = rng.standard_normal((4, 32))
    a = oracle.residual_epilogue(o, gamma, 1e-5, 1, r0)
    b = oracle.residual_epilogue(o, gamma, 1e-5, 1, np.zeros_like(r0))
    np.testing.assert_array_equal(a, b)


def test_unit_scale_of_orthogonal_update():
    # r and the normalised output orthogonal with unit RMS: the update keeps
    # RMS 1 at every step because (k-1)/k + 1/k = 1
    H = 64
    had = np.array([[1.0]])
    while had.shape[0] < H:
        had = np.block([[had, had], [had, -had]])
    r = had[1][None, :]                      # RMS 1
    o = 3.0 * had[2][None, :]                # orthogonal to r, RMS 3
    gamma = np.ones(H, np.float32)
    for k in (2, 5, 17, 104):
        out = oracle.residual_epilogue(o, gamma, 0.0, k, r)
        assert abs(np.sqrt(np.mean(out ** 2)) - 1.0) < 1e-12


def test_norm_constant_rows_and_scale_invariance():
    H, eps = 48, 1e-3
    gamma = np.linspace(0.5, 2.0, H).astype(np.float32)
    for c in (1e-2, 0.3, 7.0):
        o = np.full((1, H), c)
        got = oracle.residual_epilogue(o, gamma, eps, 1, np.zeros((1, H)))
        np.testing.assert_allclose(got[0], c / np.sqrt(c * c + eps) * gamma.astype(np.float64),
                                   rtol=1e-14)
    rng = np.random.default_rng(2)
    o = rng.standard_normal((2, H))
    a = oracle.residual_epilogue(o, gamma, 0.0, 1, np.zeros((2, H)))
    b = oracle.residual_epilogue(37.5 * o, gamma, 0.0, 1, np.zeros((2, H)))
    np.testing.assert_allclose(a, b, rtol=1e-13)
