"""Fused post-block epilogue on the GPU (beam_moe_forward_residual): the
post-sublayer RMSNorm and the depth-scaled FP32 residual stream, checked
against the binary64 oracle (block output, then oracle.residual_epilogue)
on the same routing; error max |r - ref| / max |ref|, bars as the block's
(2e-2 bf16, 1e-5 fp32).  Bit-exact properties: the block output written
alongside equals beam_moe_forward's, and step 1 ignores the incoming
residual."""
import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, TINY, WORKLOADS, make_inputs, small_shape
from gpu_util import desc_for, device, inputs, max_rel_err, oracle_forward

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _case(inp, shape, desc, rows, k, tol, label):
    dev = inp.x.device
    T, H = inp.x.shape[0], shape.hidden
    g = torch.Generator().manual_seed(k)
    gamma = torch.empty(H).uniform_(0.5, 1.5, generator=g).to(dev)
    r0 = torch.randn(T, H, generator=g).to(dev)
    out_ref, idx, w, lg = gl.forward(desc, inp.x, inp.w_router, inp.bias, inp.w_gate_up,
                                     inp.w_down, inp.s_gate_up, inp.s_down,
                                     return_routing=True)
    r = r0.clone()
    out = torch.empty_like(out_ref)
    gl.forward_residual(desc, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                        gamma, EPS, k, r, inp.s_gate_up, inp.s_down, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref), "block output differs from beam_moe_forward"
    oi, ow, _ = oracle.route(shape, lg.cpu().numpy(), inp.bias.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    blk = oracle_forward(inp, shape, rows, oi, ow, act_quant=inp.s_gate_up is not None)
    ref = oracle.residual_epilogue(blk, gamma.cpu().numpy(), EPS, k, r0.cpu().numpy()[rows])
    err = max_rel_err(r.cpu().numpy()[rows], ref)
    print(f"{label} step {k}: max rel err {err:.3e} over {len(rows)} tokens")
    assert err <= tol, err
    return r


@pytest.mark.parametrize("path", [gl.PATH_STREAM, gl.PATH_GROUPED])
@pytest.mark.parametrize("k", [1, 2, 37])
def test_small_bf16(path, k):
    sh = small_shape()
    inp = make_inputs(WORKLOADS["prefill4k"], device=device(), tokens=150, shape=sh, seed=60)
    _case(inp, sh, desc_for(WORKLOADS["prefill4k"], sh, path), np.arange(150), k, 2e-2,
          f"small path={path}")


def test_tiny_fp32():
    w = WORKLOADS["tiny"]
    _case(inputs("tiny"), TINY, desc_for(w, TINY), np.arange(16), 5, 1e-5, "tiny fp32")


def test_beam_decode64():
    w = WORKLOADS["decode64"]
    _case(inputs("decode64"), BEAM, desc_for(w, BEAM), np.arange(64), 104, 2e-2,
          "decode64")


def test_fp8_small():
    sh = small_shape()
    w = WORKLOADS["fp8_8k"]
    inp = make_inputs(w, device=device(), tokens=90, shape=sh, seed=61)
    _case(inp, sh, desc_for(w, sh), np.arange(90), 3, 6e-2, "fp8 small")


def test_step_one_and_null_out():
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=40, shape=sh, seed=62)
    d = desc_for(w, sh)
    gamma = torch.ones(sh.hidden, device=inp.x.device)
    a = torch.randn(40, sh.hidden, device=inp.x.device)
    b = torch.randn(40, sh.hidden, device=inp.x.device) * 100
    gl.forward_residual(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                        gamma, EPS, 1, a)
    gl.forward_residual(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                        gamma, EPS, 1, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(gl.BeamError):
        gl.forward_residual(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                            gamma, EPS, 0, a)
