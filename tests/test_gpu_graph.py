"""The forward captured in a HIP graph.

beam_moe_forward issues kernel launches only (no allocation, memset, copy or
host synchronisation), so a caller can capture it on a stream and replay it.
Each case captures one forward into a torch.cuda.CUDAGraph, then replays it
several times with other eager forwards (same workspace, other inputs) and
synchronisations in between, and checks every replay bit for bit against the
eager forward of the same inputs: the replays must not depend on what the
workspace held before them.  The eager forward itself is checked against the
oracle by the other GPU tests."""
import dataclasses

import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
from synth import WORKLOADS, make_inputs, small_shape, BEAM
from gpu_util import desc_for, device, inputs

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _fwd(d, inp, out, ws):
    return gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                      inp.s_gate_up, inp.s_down, out=out, workspace=ws)


def _graph_case(wl, shape, T, flags, seed, big=None):
    dev = device()
    w = WORKLOADS[wl]
    inp = big if big is not None else make_inputs(w, device=dev, tokens=T, shape=shape,
                                                   seed=seed)
    # a second batch on the same weights (tokens negated and reversed, so routed
    # elsewhere), run eagerly between replays
    other = dataclasses.replace(inp, x=(-inp.x).flip(0).contiguous())
    d = desc_for(w, shape, flags)
    ws = gl.Workspace(dev)
    out = torch.empty(T, shape.hidden, dtype=inp.x.dtype, device=dev)
    out_other = torch.empty_like(out)
    ref = _fwd(d, inp, out, ws).clone()
    ref_other = _fwd(d, other, out_other, ws).clone()
    torch.cuda.synchronize()

    # warm the capture stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _fwd(d, inp, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fwd(d, inp, out, ws)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        out.fill_(float("nan"))
        _fwd(d, other, out_other, ws)          # eager work on the shared workspace
        torch.cuda.synchronize()
        assert torch.equal(out_other, ref_other), f"eager run {r} between replays"
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager forward"
    print(f"{wl} T={T} flags={flags}: {REPLAYS} replays equal the eager forward")


@pytest.mark.parametrize("T,flags", [(5, 0), (5, gl.PATH_STREAM), (300, 0),
                                     (300, gl.PATH_GROUPED | gl.TILE_256)])
def test_graph_bf16_small(T, flags):
    _graph_case("prefill4k", small_shape(), T, flags, 1200 + T)


def test_graph_fp8_small():
    _graph_case("fp8_8k", small_shape(), 260, 0, 1300)


@pytest.mark.parametrize("T", [40, 700])
def test_graph_mxfp4_small(T):
    _graph_case("mxfp4_8k", small_shape(hidden=1024, intermediate=512), T, 0, 1400 + T)


def test_graph_beam_decode64():
    # the decode batch on the Beam layer (grouped 128-row tiles, split combine)
    inp = inputs("decode64")
    _graph_case("decode64", BEAM, inp.x.shape[0], 0, 1500, big=inp)
