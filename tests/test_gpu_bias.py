"""GPU expert-bias balancing step vs the oracle: bit-exact updated bias (the
same integer sign decision and one binary32 addition), and a balancing run
on the Beam shape that brings the 4K workload's max/mean expert load down."""
import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, WORKLOADS
from gpu_util import device, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1, 37, 4096])
def test_bias_update_bit_exact(T):
    dev = device()
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(256, 8, replace=False) for _ in range(T)]).astype(np.int32)
    b = rng.uniform(-0.05, 0.05, 256).astype(np.float32)
    d = gl.make_desc(BEAM, gl.BF16, gl.BF16)
    g = gl.bias_gamma(3, 10, 1e-3, 1e-4)
    assert g == oracle.bias_gamma(3, 10, 1e-3, 1e-4)
    bt = torch.as_tensor(b, device=dev)
    gl.bias_update(d, torch.as_tensor(idx, device=dev), g, bt)
    want = oracle.bias_update(256, idx, g, b)
    np.testing.assert_array_equal(bt.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_balancing_rounds_on_gpu():
    inp = inputs("prefill4k")
    d = gl.make_desc(BEAM, gl.BF16, gl.BF16)
    bias = inp.bias.clone()

    def load_ratio():
        idx, _, _ = gl.route(d, inp.x, inp.w_router, bias)
        c = torch.bincount(idx.flatten().long(), minlength=256).float()
        return float(c.max() / c.mean()), idx
    r0, idx = load_ratio()
    for t in range(40):
        gl.bias_update(d, idx, gl.bias_gamma(t, 40, 2e-3, 2e-4), bias)
        r, idx = load_ratio()
    print(f"prefill4k max/mean expert load {r0:.3f} -> {r:.3f} after 40 balancing rounds")
    assert r < r0 and r < 1.3, (r0, r)
