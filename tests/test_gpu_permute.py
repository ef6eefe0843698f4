"""GPU token permutation vs a numpy stable sort of the same routing:
bit-exact counts, offsets, slot lists and slot-of map."""
import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
from synth import BEAM, TINY
from gpu_util import device

pytestmark = pytest.mark.gpu


def _expected(idx, E):
    T, K = idx.shape
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")          # by expert, then (t, k)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    slot_token = (order // K).astype(np.int32)
    slot_of = np.empty(T * K, np.int32)
    slot_of[order] = np.arange(T * K, dtype=np.int32)
    return counts, offsets, slot_token, slot_of.reshape(T, K)


def _random_routing(T, E, K, rng, hot=None):
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        if hot is not None and rng.random() < 0.7:
            pool = np.concatenate([hot, rng.choice(E, K, replace=False)])
            idx[t] = np.array(list(dict.fromkeys(pool.tolist())))[:K]
        else:
            idx[t] = rng.choice(E, K, replace=False)
    return idx


@pytest.mark.parametrize("T", [1, 7, 255, 256, 257, 1000, 4096, 16384])
def test_permute_matches_stable_sort(T):
    dev = device()
    rng = np.random.default_rng(T)
    hot = np.array([0, 1, 2, 3, 32, 33, 34, 35]) if T >= 4096 else None
    idx = _random_routing(T, 256, 8, rng, hot)
    d = gl.make_desc(BEAM, gl.BF16, gl.BF16)
    got = gl.permute(d, torch.as_tensor(idx, device=dev))
    want = _expected(idx, 256)
    for name, w in zip(("counts", "offsets", "slot_token", "slot_of"), want):
        np.testing.assert_array_equal(got[name].cpu().numpy(), w, err_msg=name)


def test_permute_tiny_shape():
    dev = device()
    rng = np.random.default_rng(5)
    idx = _random_routing(300, 16, 4, rng)
    d = gl.make_desc(TINY, gl.F32, gl.F32)
    got = gl.permute(d, torch.as_tensor(idx, device=dev))
    for name, w in zip(("counts", "offsets", "slot_token", "slot_of"), _expected(idx, 16)):
        np.testing.assert_array_equal(got[name].cpu().numpy(), w, err_msg=name)


@pytest.mark.parametrize("T,E,G,K", [(256, 1024, 64, 16), (200, 1024, 64, 16), (100, 64, 8, 1),
                                     (3, 96, 3, 16), (700, 1024, 64, 16)])
def test_permute_expert_and_k_bounds(T, E, G, K):
    # the most experts and picks per token the boundary accepts, and one pick:
    # the one-workgroup form (T <= 256) and the three-kernel form (T = 700)
    import dataclasses
    dev = device()
    rng = np.random.default_rng(T + E + K)
    idx = _random_routing(T, E, K, rng)
    sh = dataclasses.replace(BEAM, n_experts=E, n_groups=G, topk_groups=G, top_k=K)
    d = gl.make_desc(sh, gl.BF16, gl.BF16)
    got = gl.permute(d, torch.as_tensor(idx, device=dev))
    for name, w in zip(("counts", "offsets", "slot_token", "slot_of"), _expected(idx, E)):
        np.testing.assert_array_equal(got[name].cpu().numpy(), w, err_msg=name)
