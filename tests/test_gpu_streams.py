"""Calls through the binding on two streams at once, without a workspace
argument: each (device, stream) pair gets its own default workspace, so the
results equal those of the same calls made one after another, bit for bit,
also when a call on one stream grows its workspace while the other stream's
kernels are still queued."""
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
from gpu_util import desc_for, device
from synth import WORKLOADS, make_inputs, small_shape

pytestmark = pytest.mark.gpu


def test_two_streams_match_serial_results():
    dev = device()
    sh = small_shape()
    w = WORKLOADS["prefill4k"]
    d = desc_for(w, sh, gl.PATH_GROUPED)
    a = make_inputs(w, device=dev, tokens=300, shape=sh, seed=21)
    b = make_inputs(w, device=dev, tokens=700, shape=sh, seed=22)
    big = make_inputs(w, device=dev, tokens=2000, shape=sh, seed=23)

    def run(inp, stream=None):
        return gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up,
                          inp.w_down, stream=stream)

    want = [run(a), run(b), run(big)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    cur = torch.cuda.current_stream(dev)
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    got = []
    for rep in range(3):
        # a on s1 and b on s2 overlap; then s1 grows its workspace (big)
        # while s2's last call may still be running
        got.append((run(a, s1), run(b, s2), run(big, s1)))
    torch.cuda.synchronize()
    for ga, gb, gbig in got:
        assert torch.equal(ga, want[0])
        assert torch.equal(gb, want[1])
        assert torch.equal(gbig, want[2])
