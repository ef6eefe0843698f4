"""Decode/verify batch sweep on the Beam layer: the block output at token
counts from a single decode token to a 2K-token batch, on both expert paths
(weight streaming and grouped tiles), checked against the binary64 oracle on
sampled tokens with routing taken bit-exact from the GPU's logits."""
import dataclasses

import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, WORKLOADS
from gpu_util import desc_for, inputs, max_rel_err, oracle_forward

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _tokens(T, seed):
    base = inputs("decode64")
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, BEAM.hidden, generator=g).to(torch.bfloat16).to(base.x.device)
    return dataclasses.replace(base, x=x)


@pytest.mark.parametrize("T", [1, 16, 512, 2048])
@pytest.mark.parametrize("path", [gl.PATH_STREAM, gl.PATH_GROUPED])
def test_sweep_sampled(T, path):
    inp = _tokens(T, 1000 + T)
    d = desc_for(WORKLOADS["decode64"], BEAM, path)
    out, idx, w, lg = gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up,
                                 inp.w_down, return_routing=True)
    torch.cuda.synchronize()
    oi, ow, _ = oracle.route(BEAM, lg.cpu().numpy(), inp.bias.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    rows = np.arange(T) if T <= 16 else np.sort(
        np.random.default_rng(T).choice(T, 12, replace=False))
    rows[-1] = T - 1
    ref = oracle_forward(inp, BEAM, rows, oi, ow)
    err = max_rel_err(out.float().cpu().numpy()[rows], ref)
    print(f"sweep T={T} path={'stream' if path == gl.PATH_STREAM else 'grouped'}: "
          f"max rel err {err:.3e} over {len(rows)} tokens")
    assert err <= BF16_TOL, err
