"""GPU router vs the oracle: indices and weights bit-exact given the GPU's
fp32 logits; logits within a derived binary32 error bound of the binary64
oracle; crafted ties; determinism; token-permutation invariance."""
import dataclasses

import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, TINY, WORKLOADS, small_shape
from gpu_util import desc_for, device, inputs, logits_bound

pytestmark = pytest.mark.gpu


def _route_and_check(inp, shape, desc):
    idx, w, lg = gl.route(desc, inp.x, inp.w_router, inp.bias)
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    oi, ow, _ = oracle.route(shape, lg_np, inp.bias.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    return idx, w, lg


@pytest.mark.parametrize("name,tokens,shape", [
    ("tiny", None, None),
    ("decode64", None, None),
    ("prefill4k", 333, small_shape()),
    ("prefill4k", None, None),
    ("prefill16k_skew", None, None),
    # expert counts that are multiples of 32 but not of 64 (partial blocks)
    ("prefill4k", 300, small_shape(n_experts=32, n_groups=1, topk_groups=1)),
    ("prefill4k", 300, small_shape(n_experts=96, n_groups=3, topk_groups=2)),
    ("ep8_share16k", None, None),
])
def test_route_bit_exact_from_gpu_logits(name, tokens, shape):
    w = WORKLOADS[name]
    sh = shape or w.shape
    inp = inputs(name, tokens=tokens, shape=shape)
    idx, wt, lg = _route_and_check(inp, sh, desc_for(w, sh))
    T = inp.x.shape[0]
    rows = np.arange(T) if T <= 512 else np.random.default_rng(0).choice(T, 256, replace=False)
    sub = dataclasses.replace(inp, x=inp.x[torch.as_tensor(rows, device=inp.x.device)])
    want = oracle.logits(sh, sub.x, inp.w_router)
    err = np.abs(lg.cpu().numpy()[rows] - want)
    assert np.all(err <= logits_bound(sub, sh)), float(err.max())
    print(f"{name}: max |logit - oracle| = {err.max():.3e}")


def test_route_logits_in_ties():
    device()
    sh = BEAM
    rng = np.random.default_rng(3)
    T = 500
    lg = (np.round(rng.standard_normal((T, 256)) * 4) / 4).astype(np.float32)
    lg[:, 40] = lg[:, 7]                  # duplicated experts
    lg[:, 96:128] = lg[:, 64:96]          # duplicated group
    lg[:10] = 0.0                         # everything tied
    lg[10:20, :] = -95.0                  # subnormal sigmoid scores
    lg[10:20, 3] = -90.0
    bias = np.zeros(256, np.float32)
    bias[200:] = 0.001
    d = gl.make_desc(sh, gl.BF16, gl.BF16, gl.ROUTE_LOGITS_IN)
    dev = device()
    lt = torch.as_tensor(lg, device=dev)
    idx, w, _ = gl.route(d, None, None, torch.as_tensor(bias, device=dev), logits=lt)
    oi, ow, _ = oracle.route(sh, lg, bias)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    # tiny shape, single-score groups, no bias pointer
    for topn in (1, 2):
        s2 = dataclasses.replace(TINY, group_score_topn=topn)
        l2 = (np.round(rng.standard_normal((300, 16)) * 2) / 2).astype(np.float32)
        d2 = gl.make_desc(s2, gl.F32, gl.F32, gl.ROUTE_LOGITS_IN)
        i2, w2, _ = gl.route(d2, None, None, None, logits=torch.as_tensor(l2, device=dev))
        oi2, ow2, _ = oracle.route(s2, l2)
        np.testing.assert_array_equal(i2.cpu().numpy(), oi2)
        np.testing.assert_array_equal(w2.cpu().numpy().view(np.uint32), ow2.view(np.uint32))


def test_route_deterministic_and_permutation_invariant():
    w = WORKLOADS["prefill4k"]
    inp = inputs("prefill4k")
    d = desc_for(w, BEAM)
    a = gl.route(d, inp.x, inp.w_router, inp.bias)
    b = gl.route(d, inp.x, inp.w_router, inp.bias)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    perm = torch.randperm(inp.x.shape[0], generator=torch.Generator().manual_seed(0)).to(inp.x.device)
    c = gl.route(d, inp.x[perm].contiguous(), inp.w_router, inp.bias)
    for u, v in zip(a, c):
        assert torch.equal(u[perm], v)


@pytest.mark.parametrize("E,G,TG,K,topn", [
    (16, 4, 2, 4, 2),      # a group is 4 lanes of one expert each
    (24, 3, 2, 4, 2),      # 8-lane groups, lanes 24..63 hold no expert
    (48, 4, 2, 6, 2),      # 12 experts per group: not a power-of-two lane segment
    (100, 10, 3, 7, 1),    # two experts per lane, 5-lane groups (not a power of two)
    (160, 5, 2, 8, 2),     # four experts per lane (rounded up from three)
    (192, 64, 8, 8, 2),    # 3 experts per group, four per lane: groups straddle lanes
    (512, 16, 4, 8, 2),    # eight experts per lane, 4-lane groups
    (1024, 64, 16, 16, 2), # sixteen experts per lane, one lane per group
    (1024, 64, 1, 16, 1),  # a single kept group of 16
])
def test_route_logits_in_group_layouts(E, G, TG, K, topn):
    # every expert-to-lane layout of the selection kernel, from given logits
    # on a coarse grid (many ties) and a coarse bias
    dev = device()
    sh = dataclasses.replace(BEAM, n_experts=E, n_groups=G, topk_groups=TG, top_k=K,
                             group_score_topn=topn)
    rng = np.random.default_rng(E * 131 + G)
    T = 300
    lg = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    lg[:5] = 0.0
    bias = (np.round(rng.standard_normal(E) * 8) / 256).astype(np.float32)
    d = gl.make_desc(sh, gl.BF16, gl.BF16, gl.ROUTE_LOGITS_IN)
    oi, ow, _ = oracle.route(sh, lg, bias)
    idx, w, _ = gl.route(d, None, None, torch.as_tensor(bias, device=dev),
                         logits=torch.as_tensor(lg, device=dev))
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
