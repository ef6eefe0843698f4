"""FP8 expert path on the GPU.

The activation quantiser is bit-exact against the oracle's (same binary32
decisions on identical inputs).  Layer outputs: against the binary64 oracle
on the dequantised e4m3 weights with unquantised activations, max rel err
<= 6e-2; against the oracle that also round-trips x and h through e4m3 (the
emulation of the recipe) the error is reported and held to 2e-2."""
import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import BEAM, WORKLOADS, make_inputs, small_shape
from gpu_util import desc_for, device, inputs, max_rel_err, oracle_forward

pytestmark = pytest.mark.gpu

FP8_TOL = 6e-2
EMU_TOL = 2e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_bit_exact(dtype):
    dev = device()
    g = torch.Generator().manual_seed(0)
    v = torch.randn(37, 640, generator=g) * torch.logspace(-3, 3, 37)[:, None]
    v[3, :128] = 0.0                                  # all-zero block
    v[5, 130] = 1e-30                                 # tiny amax block
    v[7, 256:384] = torch.linspace(-448.0, 448.0, 128)
    # subnormal block maxima: a coarse scale puts v/scale past 448 (the
    # recipe saturates), or amax/448 underflows to zero (scale 1)
    v[9, 512:640] = torch.linspace(-1.0, 1.0, 128) * 1e-39
    v[11, :128] = 0.0
    v[11, 7] = -8.8e-43
    v[13, 128:256] = 0.0
    v[13, 130] = 3e-43
    v[15, 384:512] = torch.arange(1, 129) * 1e-40
    v = v.to(dtype)
    q, s = gl.quant_e4m3(v.to(dev))
    oq, os_ = oracle.quant_e4m3(v.float().numpy(), 128)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def _check(inp, shape, tokens, label, flags=0):
    d = desc_for(WORKLOADS["fp8_8k"], shape, flags)
    out, idx, w, lg = gl.forward(d, inp.x, inp.w_router, inp.bias, inp.w_gate_up,
                                 inp.w_down, inp.s_gate_up, inp.s_down,
                                 return_routing=True)
    torch.cuda.synchronize()
    oi, ow, _ = oracle.route(shape, lg.cpu().numpy(), inp.bias.cpu().numpy())
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))
    got = out.float().cpu().numpy()[np.asarray(tokens)]
    ref = oracle_forward(inp, shape, tokens, oi, ow, act_quant=False)
    emu = oracle_forward(inp, shape, tokens, oi, ow, act_quant=True)
    e_ref, e_emu = max_rel_err(got, ref), max_rel_err(got, emu)
    print(f"{label}: max rel err {e_ref:.3e} vs dequantised-weight oracle, "
          f"{e_emu:.3e} vs e4m3 emulation oracle")
    assert e_ref <= FP8_TOL, e_ref
    assert e_emu <= EMU_TOL, e_emu
    return out, idx


@pytest.mark.parametrize("T", [1, 5, 300])
def test_fp8_small(T):
    sh = small_shape()
    inp = make_inputs(WORKLOADS["fp8_8k"], device=device(), tokens=T, shape=sh,
                      seed=20 + T)
    _check(inp, sh, np.arange(T), f"fp8 small T={T}")


def test_fp8_beam_sampled():
    inp = inputs("fp8_8k")
    T = inp.x.shape[0]
    rows = np.sort(np.random.default_rng(2).choice(T, 16, replace=False))
    rows[-1] = T - 1
    _check(inp, BEAM, rows, "fp8_8k sampled")


def test_fp8_decode64():
    # the Beam layer at 64 tokens: 128-row tiles with the three-stage copy
    # ring, one to a few rows per expert; every row against the oracle
    inp = inputs("fp8_decode64")
    _check(inp, BEAM, np.arange(64), "fp8_decode64")


@pytest.mark.parametrize("T", [300, 700])
def test_fp8_odd_widths_skewed(T):
    # hidden and intermediate multiples of 128 but not of 256 (the last
    # 256-wide down tile is half outside H); hot experts with several
    # 256-slot M tiles and a ragged last tile
    sh = small_shape(hidden=384, intermediate=384)
    inp = make_inputs(WORKLOADS["fp8_8k"], device=device(), tokens=T, shape=sh,
                      seed=40 + T, bias="skew:0.5:0,1,2,3,32,33,34,35")
    _check(inp, sh, np.arange(0, T, 2), f"fp8 H=I=384 skew T={T}")


@pytest.mark.parametrize("T", [2100, 4300])
@pytest.mark.parametrize("hidden", [512, 384])
def test_fp8_extended_last_tiles(T, hidden):
    # 262 / 537 rows per expert on average: many experts end in a tile of
    # 257..288 rows (one 256-row tile extended by up to 32 rows), some in a
    # plain one.  Against the oracle with and without the extension, and the
    # two bit-identical (same products, same order, same scale steps).
    sh = small_shape(hidden=hidden, intermediate=384 if hidden == 384 else 256)
    inp = make_inputs(WORKLOADS["fp8_8k"], device=device(), tokens=T, shape=sh,
                      seed=60 + T + hidden)
    a, idx = _check(inp, sh, np.arange(0, T, 7), f"fp8 extended tiles T={T} H={hidden}")
    b, _ = _check(inp, sh, np.arange(0, T, 7), f"fp8 256-row tiles T={T} H={hidden}",
                  gl.TILE_256)
    counts = torch.bincount(idx.flatten().long(), minlength=sh.n_experts).cpu()
    ext = ((counts % 256 >= 1) & (counts % 256 <= 32) & (counts > 256)).sum().item()
    print(f"experts whose last tile is extended: {ext} of {sh.n_experts}")
    assert ext > 0
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,hidden,skew", [(5, 256, False), (300, 256, False),
                                           (700, 384, True), (2100, 512, False)])
def test_fp8_128_row_tiles(T, hidden, skew):
    # 128-row tiles with the three-stage copy ring: one, two and several
    # tiles per expert, partial last tiles, a 256-wide down tile half outside
    # H (H = 384); against the oracle and bit-identical to the 256-row form
    sh = small_shape(hidden=hidden, intermediate=384 if hidden == 384 else 256)
    inp = make_inputs(WORKLOADS["fp8_8k"], device=device(), tokens=T, shape=sh,
                      seed=80 + T + hidden,
                      bias="skew:0.5:0,1,2,3,32,33,34,35" if skew else None)
    rows = np.arange(0, T, max(1, T // 300))
    a, _ = _check(inp, sh, rows, f"fp8 128-row tiles T={T} H={hidden}", gl.TILE_128)
    b, _ = _check(inp, sh, rows, f"fp8 256-row tiles T={T} H={hidden}", gl.TILE_256)
    assert torch.equal(a, b)


@pytest.mark.parametrize("hidden,intermediate", [(128, 128), (256, 128), (128, 256)])
def test_fp8_one_and_two_blocks(hidden, intermediate):
    # products only one or two 128-deep blocks deep (gate/up K = hidden, down
    # K = intermediate): the rescale pipeline's first and last stages meet;
    # 256-row tiles (with extended last tiles) and 128-row tiles against the
    # oracle, and bit-identical to each other
    sh = small_shape(hidden=hidden, intermediate=intermediate)
    T = 2100
    inp = make_inputs(WORKLOADS["fp8_8k"], device=device(), tokens=T, shape=sh,
                      seed=90 + hidden + intermediate)
    rows = np.arange(0, T, 7)
    a, _ = _check(inp, sh, rows, f"fp8 256-row tiles H={hidden} I={intermediate}", gl.TILE_160)
    b, _ = _check(inp, sh, rows, f"fp8 128-row tiles H={hidden} I={intermediate}", gl.TILE_128)
    assert torch.equal(a, b)


def test_fp8_max_tokens_sampled():
    # the largest batch the boundary accepts for the Beam layer (T = 52,428:
    # 419,424 slots, the slot-major scale words up to block 39), sampled rows
    # including the last
    w = WORKLOADS["fp8_8k"]
    T = (2**31 - 1) // (BEAM.top_k * max(BEAM.hidden, BEAM.intermediate))
    assert gl.validate(desc_for(w, BEAM), T) == gl.OK
    inp = make_inputs(w, device=device(), tokens=T)
    rows = np.sort(np.random.default_rng(6).choice(T, 12, replace=False))
    rows[-1] = T - 1
    _check(inp, BEAM, rows, f"fp8 Beam T={T} sampled")
