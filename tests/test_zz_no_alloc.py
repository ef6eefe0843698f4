"""beam_moe_forward_noalloc (the forward for callers that cannot allocate,
whose workspace is the library's per-device scratch array) against
beam_moe_forward with a caller workspace, through the C ABI: bitwise equal
outputs and routing on two calls in a row, the second with fewer tokens, on
the Beam decode layer (bf16 and FP8 weights); and the host-side refusal of
a batch whose workspace exceeds the array."""
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
from gpu_util import desc_for, device, inputs
from synth import WORKLOADS, BEAM

pytestmark = pytest.mark.gpu


def _pair(d, inp, rows):
    dev = inp.x.device
    x = inp.x[:rows].contiguous()
    T = x.shape[0]

    def bufs():
        return (torch.empty(T, d.hidden, dtype=x.dtype, device=dev),
                torch.empty(T, d.top_k, dtype=torch.int32, device=dev),
                torch.empty(T, d.top_k, dtype=torch.float32, device=dev),
                torch.empty(T, d.n_experts, dtype=torch.float32, device=dev))

    ref = gl.forward(d, x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down,
                     inp.s_gate_up, inp.s_down, return_routing=True,
                     workspace=gl.Workspace(dev))
    out, idx, w, lg = bufs()
    gl.forward_noalloc(d, x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down, out,
                       inp.s_gate_up, inp.s_down, idx, w, lg)
    return ref, (out, idx, w, lg)


@pytest.mark.parametrize("name", ["decode64", "fp8_decode64"])
def test_noalloc_matches_forward(name):
    device()
    w = WORKLOADS[name]
    inp = inputs(name)
    d = desc_for(w, w.shape)
    for rows in (64, 9):           # the second call is smaller
        print(f"noalloc {name} T={rows}", flush=True)
        ref, got = _pair(d, inp, rows)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def test_noalloc_refuses_large_batch():
    device()
    d = gl.make_desc(BEAM, gl.BF16, gl.BF16)
    T = 4096
    assert gl.workspace_bytes(d, T) > gl.NOALLOC_SCRATCH_BYTES
    null = None
    st = gl.lib().beam_moe_forward_noalloc(d, T, *([null] * 12))
    assert st == gl.ERR_WORKSPACE
