"""Pins of the oracle's expert MLPs and combine: each expert a SwiGLU MLP
(hidden 5,120 -> intermediate 2,560 -> hidden), eight per token, no shared
expert, outputs combined with the routing weights ("Hugging Face releases
Beam ..." MoE paragraph; "Reflection Releases Beam ...", section "Where Beam
Saves and Where the Memory Bill Comes In").  Special cases reduce the layer
to torch float64 library routines.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import TINY, WORKLOADS, Shape, make_inputs


def _ffn64(x, wgu, wd):
    """Dense SwiGLU in torch float64: silu(x Wg^T) * (x Wu^T) Wd^T."""
    I = wd.shape[1]
    x = x.double()
    g = x @ wgu[:I].double().T
    u = x @ wgu[I:].double().T
    return (torch.nn.functional.silu(g) * u) @ wd.double().T


@pytest.mark.parametrize("wdt", [torch.float32, torch.bfloat16])
def test_single_expert_is_dense_swiglu(wdt):
    sh = Shape(hidden=256, intermediate=128, n_experts=1, n_groups=1,
               topk_groups=1, top_k=1, group_score_topn=1, routed_scale=1.0)
    g = torch.Generator().manual_seed(3)
    x = torch.randn(9, 256, generator=g)
    wgu = (torch.randn(1, 256, 256, generator=g) * 0.05).to(wdt)
    wd = (torch.randn(1, 256, 128, generator=g) * 0.05).to(wdt)
    idx, w, _ = oracle.route(sh, np.zeros((9, 1), np.float32))
    assert np.all(w == 1.0)
    out = oracle.forward_tokens(sh, np.arange(9), x, idx, w, wgu, wd)
    want = _ffn64(x, wgu[0], wd[0]).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)


def test_identical_experts_scale_by_weight_sum():
    inp = make_inputs(WORKLOADS["tiny"])
    wgu = inp.w_gate_up[:1].expand_as(inp.w_gate_up).contiguous()
    wd = inp.w_down[:1].expand_as(inp.w_down).contiguous()
    lg = oracle.logits(TINY, inp.x, inp.w_router).astype(np.float32)
    idx, w, _ = oracle.route(TINY, lg, inp.bias)
    out = oracle.forward_tokens(TINY, np.arange(16), inp.x, idx, w, wgu, wd)
    want = _ffn64(inp.x, wgu[0], wd[0]).numpy() * w.astype(np.float64).sum(1)[:, None]
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-13)


def test_weight_goes_with_its_expert():
    # Experts differ only by an exact power-of-two factor on W_d: the output
    # is (sum_k w_k c_{e_k}) * FFN_0(x).  Pairing a weight with the wrong
    # expert, or dropping one, changes the factor.
    inp = make_inputs(WORKLOADS["tiny"])
    c = 2.0 ** (np.arange(16) - 8.0)
    wgu = inp.w_gate_up[:1].expand_as(inp.w_gate_up).contiguous()
    wd = torch.stack([inp.w_down[0] * float(c[e]) for e in range(16)])
    lg = oracle.logits(TINY, inp.x, inp.w_router).astype(np.float32)
    idx, w, _ = oracle.route(TINY, lg, inp.bias)
    out = oracle.forward_tokens(TINY, np.arange(16), inp.x, idx, w, wgu, wd)
    fac = (w.astype(np.float64) * c[idx]).sum(1)
    want = _ffn64(inp.x, wgu[0], inp.w_down[0]).numpy() * fac[:, None]
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-13)


def test_token_permutation_layer():
    inp = make_inputs(WORKLOADS["tiny"])
    lg = oracle.logits(TINY, inp.x, inp.w_router).astype(np.float32)
    idx, w, _ = oracle.route(TINY, lg, inp.bias)
    perm = np.random.default_rng(1).permutation(16)
    out = oracle.forward_tokens(TINY, np.arange(16), inp.x, idx, w,
                                inp.w_gate_up, inp.w_down)
    out_p = oracle.forward_tokens(TINY, perm, inp.x, idx, w,
                                  inp.w_gate_up, inp.w_down)
    np.testing.assert_array_equal(out[perm], out_p)


def test_logits_match_torch_float64():
    inp = make_inputs(WORKLOADS["tiny"])
    lg = oracle.logits(TINY, inp.x, inp.w_router)
    want = (inp.x.double() @ inp.w_router.double().T).numpy()
    np.testing.assert_allclose(lg, want, rtol=1e-13, atol=1e-13)
    sh = dataclasses.replace(TINY, hidden=512)
    g = torch.Generator().manual_seed(0)
    xb = torch.randn(5, 512, generator=g).to(torch.bfloat16)
    wr = torch.randn(16, 512, generator=g)
    np.testing.assert_allclose(oracle.logits(sh, xb, wr),
                               (xb.double() @ wr.double().T).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_forward_fp8_weights_dequantise_blockwise():
    # e4m3 weights with per-128x128 scales equal f32 weights holding
    # code * scale, element by element.  Power-of-two scales keep the f32
    # products exact, so both sides see the same real weights.
    sh = Shape(hidden=256, intermediate=128, n_experts=4, n_groups=2,
               topk_groups=1, top_k=2)
    inp = make_inputs(WORKLOADS["fp8_8k"], tokens=6, shape=sh)
    g = torch.Generator().manual_seed(1)
    inp.s_gate_up = 2.0 ** torch.randint(-14, -6, inp.s_gate_up.shape, generator=g).float()
    inp.s_down = 2.0 ** torch.randint(-14, -6, inp.s_down.shape, generator=g).float()
    deq_gu = inp.w_gate_up.view(torch.float8_e4m3fn).float() * \
        inp.s_gate_up.repeat_interleave(128, 1).repeat_interleave(128, 2)
    deq_d = inp.w_down.view(torch.float8_e4m3fn).float() * \
        inp.s_down.repeat_interleave(128, 1).repeat_interleave(128, 2)
    lg = oracle.logits(sh, inp.x, inp.w_router).astype(np.float32)
    idx, w, _ = oracle.route(sh, lg, inp.bias)
    a = oracle.forward_tokens(sh, np.arange(6), inp.x, idx, w, inp.w_gate_up,
                              inp.w_down, inp.s_gate_up, inp.s_down)
    b = oracle.forward_tokens(sh, np.arange(6), inp.x, idx, w, deq_gu, deq_d)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_act_quant_lossless_when_representable():
    # If each 128-block already is (e4m3 value) * 2^k with block amax
    # 448 * 2^k, the scale is exactly 2^k and the round trip is lossless.
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7E, (3, 256)).astype(np.uint8)
    vals = oracle.e4m3_decode(codes).reshape(3, 256)
    vals[:, 0] = 448.0
    vals[:, 128] = -448.0
    x = (vals * np.array([[2.0 ** -6], [1.0], [2.0 ** 3]])).astype(np.float32)
    q, s = oracle.quant_e4m3(x, 128)
    np.testing.assert_array_equal(s, np.repeat(np.array([[2.0 ** -6], [1.0], [8.0]],
                                                        np.float32), 2, 1))
    deq = oracle.e4m3_decode(q).reshape(3, 256) * np.repeat(s, 128, 1)
    np.testing.assert_array_equal(deq, x)


def test_act_quant_scale_equivariance():
    # Scaling a block by 2^j leaves the codes unchanged and scales the scale.
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    q0, s0 = oracle.quant_e4m3(x, 128)
    for j in (-5, 3, 11):
        q1, s1 = oracle.quant_e4m3(x * np.float32(2.0 ** j), 128)
        np.testing.assert_array_equal(q0, q1)
        np.testing.assert_array_equal(s1, s0 * np.float32(2.0 ** j))
    # and the dequantised block is within half an e4m3 step of x
    deq = oracle.e4m3_decode(q0).reshape(4, 512) * np.repeat(s0, 128, 1)
    amax = np.repeat(np.abs(x).reshape(4, 4, 128).max(2), 128, 1)
    assert np.all(np.abs(deq - x) <= amax * 2.0 ** -4 + 1e-30)
