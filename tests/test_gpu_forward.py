"""GPU block output vs the binary64 oracle.

The oracle routes from the GPU's fp32 logits (routing is bit-exact given the
logits) and evaluates the experts and the combine in binary64.  Error metric:
max |y - r| / max |r| over the compared rows; bars: 2e-2 for bf16 weights and
activations, 1e-5 for the fp32 path (all-fp32 arithmetic, depth <= H+I)."""
import dataclasses

import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, TINY, WORKLOADS, small_shape, make_inputs
from gpu_util import desc_for, device, inputs, max_rel_err, oracle_forward

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5


def _run(inp, shape, desc):
    out, idx, w, lg = gl.forward(desc, inp.x, inp.w_router, inp.bias,
                                 inp.w_gate_up, inp.w_down, inp.s_gate_up,
                                 inp.s_down, return_routing=True)
    torch.cuda.synchronize()
    oi, ow, _ = oracle.route(shape, lg.cpu().numpy(), inp.bias.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    return out, oi, ow


def _check(inp, shape, desc, tokens, tol, label):
    out, oi, ow = _run(inp, shape, desc)
    ref = oracle_forward(inp, shape, tokens, oi, ow)
    got = out.float().cpu().numpy()[np.asarray(tokens)]
    err = max_rel_err(got, ref)
    print(f"{label}: max rel err {err:.3e} over {len(tokens)} tokens")
    assert err <= tol, err
    return out


def test_tiny_fp32():
    w = WORKLOADS["tiny"]
    inp = inputs("tiny")
    _check(inp, TINY, desc_for(w, TINY), np.arange(16), F32_TOL, "tiny fp32")


@pytest.mark.parametrize("T", [1, 3, 200])
@pytest.mark.parametrize("path", [gl.PATH_STREAM, gl.PATH_GROUPED])
def test_small_bf16_both_paths(T, path):
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=T, shape=sh, seed=10 + T)
    _check(inp, sh, desc_for(w, sh, path), np.arange(T), BF16_TOL,
           f"small T={T} path={path}")


def test_small_bf16_skewed_long_chunks():
    # hot experts with hundreds of tokens: several 16-token chunks on the
    # streaming path and several M tiles of either height on the grouped path
    sh = small_shape()
    w = WORKLOADS["prefill16k_skew"]
    inp = make_inputs(w, device=device(), tokens=700, shape=sh, seed=77)
    for path in (gl.PATH_STREAM, gl.PATH_GROUPED | gl.TILE_128,
                 gl.PATH_GROUPED | gl.TILE_160, gl.PATH_GROUPED | gl.TILE_256):
        _check(inp, sh, desc_for(w, sh, path), np.arange(0, 700, 3), BF16_TOL,
               f"small skew path={path}")


@pytest.mark.parametrize("T", [1, 37, 700, 2100])
def test_tile_heights_bitwise_equal(T):
    # 128-, 160- and 256-row tiles add the same products in the same order:
    # equal bits, including tails of 1..255 rows and experts with many tiles
    sh = small_shape()
    w = WORKLOADS["prefill16k_skew"]
    inp = make_inputs(w, device=device(), tokens=T, shape=sh, seed=500 + T)
    outs = []
    for tile in (gl.TILE_128, gl.TILE_160, gl.TILE_256):
        d = desc_for(w, sh, gl.PATH_GROUPED | tile)
        outs.append(gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up,
                               inp.w_down))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[2])


@pytest.mark.parametrize("path", [gl.PATH_STREAM, gl.PATH_GROUPED | gl.TILE_128,
                                  gl.PATH_GROUPED | gl.TILE_160, gl.PATH_GROUPED | gl.TILE_256])
def test_odd_widths_skewed(path):
    # hidden and intermediate multiples of 128 but not of 256: the last
    # 256-wide down tile of the grouped path is half outside H
    sh = small_shape(hidden=384, intermediate=384)
    w = WORKLOADS["prefill16k_skew"]
    inp = make_inputs(w, device=device(), tokens=600, shape=sh, seed=91)
    _check(inp, sh, desc_for(w, sh, path), np.arange(0, 600, 2), BF16_TOL,
           f"H=I=384 skew path={path}")


# default choice (the grouped path at 64 tokens) and the streaming path forced
@pytest.mark.parametrize("path", [0, gl.PATH_STREAM])
def test_beam_decode64(path):
    w = WORKLOADS["decode64"]
    inp = inputs("decode64")
    _check(inp, BEAM, desc_for(w, BEAM, path), np.arange(64), BF16_TOL,
           f"decode64 path={path}")


@pytest.mark.parametrize("name", ["prefill4k", "prefill16k_skew", "ep8_share16k"])
def test_beam_prefill_sampled(name):
    # in the launch configuration the bench times (default tile choice)
    w = WORKLOADS[name]
    inp = inputs(name)
    T = inp.x.shape[0]
    rows = np.sort(np.random.default_rng(1).choice(T, 24, replace=False))
    rows[-1] = T - 1                       # last token of the ragged tail
    _check(inp, w.shape, desc_for(w, w.shape), rows, BF16_TOL, f"{name} sampled")


def test_beam_max_tokens_sampled():
    # the largest batch the boundary accepts for the Beam layer
    # (T*K*max(H, I) < 2^31: T = 52,428), sampled rows including the last
    w = WORKLOADS["prefill16k_skew"]
    T = (2**31 - 1) // (BEAM.top_k * max(BEAM.hidden, BEAM.intermediate))
    assert gl.validate(desc_for(w, BEAM), T) == gl.OK
    assert gl.validate(desc_for(w, BEAM), T + 1) != gl.OK
    inp = make_inputs(w, device=device(), tokens=T)
    rows = np.sort(np.random.default_rng(5).choice(T, 12, replace=False))
    rows[-1] = T - 1
    _check(inp, BEAM, desc_for(w, BEAM), rows, BF16_TOL, f"Beam T={T} sampled")


def test_forward_deterministic_and_permutation():
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=300, shape=sh, seed=3)
    for path in (gl.PATH_STREAM, gl.PATH_GROUPED):
        d = desc_for(w, sh, path)
        a = gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down)
        b = gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down)
        assert torch.equal(a, b)
        perm = torch.randperm(300, generator=torch.Generator().manual_seed(1)).to(a.device)
        c = gl.forward(d, inp.x[perm].contiguous(), inp.w_router, inp.bias,
                       inp.w_gate_up, inp.w_down)
        assert torch.equal(a[perm], c), f"path {path}"


def test_identical_experts():
    # all experts equal: out = (sum of weights) * FFN(x) whatever the routing
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=50, shape=sh, seed=4)
    inp.w_gate_up[:] = inp.w_gate_up[0]
    inp.w_down[:] = inp.w_down[0]
    for path in (gl.PATH_STREAM, gl.PATH_GROUPED):
        out, oi, ow = _run(inp, sh, desc_for(w, sh, path))
        x = inp.x.double().cpu()
        I = sh.intermediate
        wgu = inp.w_gate_up[0].double().cpu()
        ffn = (torch.nn.functional.silu(x @ wgu[:I].T) * (x @ wgu[I:].T)) @ inp.w_down[0].double().cpu().T
        ref = ffn.numpy() * ow.astype(np.float64).sum(1)[:, None]
        assert max_rel_err(out.float().cpu().numpy(), ref) <= BF16_TOL


def test_zero_tokens_and_small_workspace():
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=4, shape=sh, seed=5)
    d = desc_for(w, sh)
    empty = inp.x[:0]
    out = gl.forward(d, empty, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down)
    assert out.shape == (0, sh.hidden)
    ws = gl.Workspace()
    ws.buf = torch.empty(256, dtype=torch.uint8, device=inp.x.device)
    small = gl.Workspace()
    with pytest.raises(gl.BeamError) as ei:
        import ctypes
        L = gl.lib()
        o = torch.empty(4, sh.hidden, dtype=torch.bfloat16, device=inp.x.device)
        st = L.beam_moe_forward(ctypes.byref(d), 4, gl._p(inp.x), gl._p(inp.w_router),
                                gl._p(inp.bias), gl._p(inp.w_gate_up), None,
                                gl._p(inp.w_down), None, gl._p(o), None, None, None,
                                gl._p(ws.buf), 256, gl._stream())
        gl._check(st, "forward")
    assert ei.value.status == gl.ERR_WORKSPACE


@pytest.mark.parametrize("top_k,topk_groups", [(1, 1), (16, 4)])
@pytest.mark.parametrize("T", [300, 2100])
@pytest.mark.parametrize("path", [gl.PATH_STREAM, gl.PATH_GROUPED])
def test_top_k_bounds(top_k, topk_groups, T, path):
    # the smallest and the largest K the boundary accepts, on both expert
    # paths and every combine form (several workgroups per token with 8 or
    # 16 rows' loads in flight; for K = 16 one workgroup per token from 2K
    # tokens on), sampled rows against the oracle
    sh = small_shape(top_k=top_k, topk_groups=topk_groups)
    w = WORKLOADS["prefill4k"]
    inp = make_inputs(w, device=device(), tokens=T, shape=sh, seed=120 + T + top_k)
    rows = np.arange(0, T, 7)
    _check(inp, sh, desc_for(w, sh, path), rows, BF16_TOL,
           f"top_k={top_k} T={T} path={path}")
