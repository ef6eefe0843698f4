"""Pins of the oracle's router: the group-limited sigmoid router of
"Reflection Releases Beam ...", section "Where Beam Saves and Where the Memory
Bill Comes In" (sigmoid scores, 8 groups of 32, 4 best groups, top-8 inside
them, weights normalised and scaled by 2.5), with the selection-only expert
bias of the load-balancing paragraph of "Reflection AI Introduces Beam ...".

The oracle sorts; the brute force enumerates every subset with exact
rationals; the all-groups-kept case is a stable argsort.  Invariants cover
the Beam shape, where enumeration is out of reach.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import bruteforce as bf
from synth import BEAM, TINY, Shape, WORKLOADS, make_inputs

MID = Shape(hidden=64, intermediate=32, n_experts=32, n_groups=8, topk_groups=4,
            top_k=8)


def _logits(T, E, seed, scale=1.0, grid=None):
    rng = np.random.default_rng(seed)
    l = (rng.standard_normal((T, E)) * scale).astype(np.float32)
    if grid is not None:                       # coarse grid => many exact ties
        l = (np.round(l / grid) * grid).astype(np.float32)
    return l


def _check_same(shape, lg, bias):
    i0, w0, k0 = oracle.route(shape, lg, bias)
    i1, w1, k1 = bf.route(shape, lg, bias)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_array_equal(w0.view(np.uint32), w1.view(np.uint32))
    np.testing.assert_array_equal(k0, k1)


def test_bruteforce_tiny_workload():
    inp = make_inputs(WORKLOADS["tiny"])
    lg = oracle.logits(TINY, inp.x, inp.w_router).astype(np.float32)
    _check_same(TINY, lg, inp.bias.numpy())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_tiny_random(seed):
    lg = _logits(48, TINY.n_experts, seed, scale=2.0)
    bias = np.random.default_rng(100 + seed).uniform(-0.05, 0.05, 16).astype(np.float32)
    _check_same(TINY, lg, bias)


def test_bruteforce_tiny_ties():
    # Logits on a 0.25 grid and zero bias: equal scores inside and across
    # groups, equal group scores, ties at the top-k boundary.
    lg = _logits(64, TINY.n_experts, 5, scale=1.0, grid=0.25)
    _check_same(TINY, lg, None)
    lg = np.zeros((2, 16), np.float32)          # everything tied
    _check_same(TINY, lg, None)
    i, w, k = oracle.route(TINY, lg)
    np.testing.assert_array_equal(k[0], [0, 1])
    np.testing.assert_array_equal(i[0], [0, 1, 2, 3])


def test_bruteforce_mid():
    lg = _logits(12, MID.n_experts, 11, scale=1.5)
    bias = np.random.default_rng(3).uniform(-0.02, 0.02, 32).astype(np.float32)
    _check_same(MID, lg, bias)
    lg = _logits(6, MID.n_experts, 12, grid=0.5)
    _check_same(MID, lg, None)


def test_bruteforce_single_score_groups():
    sh = dataclasses.replace(TINY, group_score_topn=1)
    lg = _logits(32, 16, 21, grid=0.25)
    _check_same(sh, lg, None)
    lg = _logits(32, 16, 22)
    _check_same(sh, lg, np.full(16, 0.01, np.float32))


def _exact_s(lg):
    return np.array([[bf.sigmoid32_exact(float(v))[0] for v in row] for row in lg],
                    np.float32)


@pytest.mark.parametrize("groups", [8, 1])
def test_all_groups_kept_is_stable_argsort(groups):
    sh = dataclasses.replace(BEAM, n_groups=groups, topk_groups=groups)
    lg = _logits(24, 256, 31 + groups)
    bias = np.random.default_rng(9).uniform(-0.02, 0.02, 256).astype(np.float32)
    idx, w, _ = oracle.route(sh, lg, bias)
    u = _exact_s(lg) + bias
    want = np.argsort(-u, axis=1, kind="stable")[:, :8]
    np.testing.assert_array_equal(idx, want)


def _beam_invariants(idx, w, kept, lg, bias, sh):
    T, K = idx.shape
    gs = sh.n_experts // sh.n_groups
    s = oracle.sigmoid32(lg.ravel()).reshape(lg.shape)
    u = s + (0 if bias is None else bias)
    for t in range(T):
        assert len(set(idx[t])) == K
        groups = idx[t] // gs
        assert set(groups) <= set(kept[t])
        assert len(set(kept[t])) == sh.topk_groups
        assert np.all(w[t] > 0)
        # rank order: u non-increasing, equal u => increasing index
        ut = u[t, idx[t]]
        assert np.all(ut[:-1] >= ut[1:])
        # nothing eligible and unselected beats the last selected expert
        elig = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in kept[t]])
        rest = np.setdiff1d(elig, idx[t])
        assert np.all(u[t, rest] <= ut[-1])
        # sum of weights is the routed scale up to K+2 binary32 roundings
        assert abs(float(np.sum(w[t].astype(np.float64))) - sh.routed_scale) <= \
            sh.routed_scale * (K + 2) * 2.0 ** -24


@pytest.mark.parametrize("bias_kind", ["zero", "uniform", "skew"])
def test_beam_invariants(bias_kind):
    lg = _logits(1024, 256, 41)
    rng = np.random.default_rng(5)
    bias = {"zero": None,
            "uniform": rng.uniform(-0.02, 0.02, 256).astype(np.float32),
            "skew": np.where(np.isin(np.arange(256), [0, 1, 2, 3, 32, 33, 34, 35]),
                             0.5, 0.0).astype(np.float32)}[bias_kind]
    idx, w, kept = oracle.route(BEAM, lg, bias)
    _beam_invariants(idx, w, kept, lg, bias, BEAM)


def test_weights_use_unbiased_scores():
    # The bias only steers selection: w_k / 2.5 equals s_k / sum(s) with the
    # exact sigmoid of the selected experts' logits, whatever the bias.
    lg = _logits(64, 256, 51)
    bias = np.random.default_rng(2).uniform(-0.3, 0.3, 256).astype(np.float32)
    idx, w, _ = oracle.route(BEAM, lg, bias)
    for t in range(64):
        s = np.array([float(bf.exact_sigmoid(float(lg[t, e]))) for e in idx[t]])
        np.testing.assert_allclose(w[t] / 2.5, s / s.sum(), rtol=2e-6)


def test_routed_scale_is_one_rounding():
    lg = _logits(256, 256, 61)
    i1, w1, _ = oracle.route(dataclasses.replace(BEAM, routed_scale=1.0), lg)
    i2, w2, _ = oracle.route(BEAM, lg)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(w2, (w1 * np.float32(2.5)).astype(np.float32))


def test_token_permutation():
    lg = _logits(512, 256, 71)
    perm = np.random.default_rng(0).permutation(512)
    i0, w0, _ = oracle.route(BEAM, lg)
    i1, w1, _ = oracle.route(BEAM, lg[perm])
    np.testing.assert_array_equal(i0[perm], i1)
    np.testing.assert_array_equal(w0[perm], w1)


def test_group_preserving_relabel():
    # Permute the groups and the experts inside each group: the selection
    # follows the relabelling (continuous random logits: no ties).
    rng = np.random.default_rng(8)
    lg = _logits(256, 256, 81)
    gperm = rng.permutation(8)
    inner = [rng.permutation(32) for _ in range(8)]
    new_of_old = np.empty(256, np.int64)
    for g in range(8):
        for j in range(32):
            new_of_old[g * 32 + j] = gperm[g] * 32 + inner[g][j]
    lg2 = np.empty_like(lg)
    lg2[:, new_of_old] = lg
    i0, w0, _ = oracle.route(BEAM, lg)
    i1, w1, _ = oracle.route(BEAM, lg2)
    np.testing.assert_array_equal(new_of_old[i0], i1)
    np.testing.assert_array_equal(w0, w1)


def test_duplicated_rows_break_ties_by_index():
    # Two experts with bit-identical logits: the lower index ranks first.
    lg = _logits(64, 256, 91)
    lg[:, 7] = 9.0
    lg[:, 5] = 9.0
    lg[:, 200] = 9.0
    idx, _, _ = oracle.route(BEAM, lg)
    for t in range(64):
        pos = {e: list(idx[t]).index(e) for e in (5, 7, 200) if e in idx[t]}
        if 5 in pos and 7 in pos:
            assert pos[5] < pos[7]
