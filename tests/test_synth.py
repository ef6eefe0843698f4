"""The seeded input generators are deterministic and follow the stated
recipe (shapes, dtypes, bias patterns)."""
import torch

from synth import WORKLOADS, make_inputs, small_shape


def test_same_seed_same_bytes():
    a = make_inputs(WORKLOADS["tiny"])
    b = make_inputs(WORKLOADS["tiny"])
    for f in ("x", "w_router", "bias", "w_gate_up", "w_down"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    c = make_inputs(WORKLOADS["tiny"], seed=5)
    assert not torch.equal(a.x, c.x)


def test_recipe():
    sh = small_shape()
    a = make_inputs(WORKLOADS["prefill16k_skew"], tokens=40, shape=sh)
    assert a.x.dtype == torch.bfloat16 and a.x.shape == (40, sh.hidden)
    assert a.w_gate_up.shape == (sh.n_experts, 2 * sh.intermediate, sh.hidden)
    assert a.w_down.shape == (sh.n_experts, sh.hidden, sh.intermediate)
    assert a.w_router.dtype == torch.float32
    hot = torch.nonzero(a.bias).flatten().tolist()
    assert hot == [0, 1, 2, 3, 32, 33, 34, 35] and float(a.bias.max()) == 0.5
    assert abs(float(a.w_router.std()) - sh.hidden ** -0.5) < 0.1 * sh.hidden ** -0.5
    assert abs(float(a.w_gate_up.float().std()) - 0.02) < 0.002
    u = make_inputs(WORKLOADS["prefill4k"], tokens=4, shape=sh)
    assert float(u.bias.abs().max()) <= 0.02 and float(u.bias.abs().min()) > 0


def test_fp8_weights():
    sh = small_shape(hidden=256, intermediate=128, n_experts=8, n_groups=2,
                     topk_groups=1, top_k=2)
    a = make_inputs(WORKLOADS["fp8_8k"], tokens=4, shape=sh)
    assert a.w_gate_up.dtype == torch.uint8
    codes = a.w_gate_up.flatten()
    assert not torch.any((codes & 0x7F) == 0x7F)          # no NaN codes
    assert a.s_gate_up.shape == (8, 2, 2) and bool((a.s_gate_up > 0).all())
    # each 128x128 block reaches the largest code magnitude
    blk = a.w_gate_up.view(torch.float8_e4m3fn).float().abs().reshape(8, 2, 128, 2, 128)
    assert bool((blk.amax(dim=(2, 4)) == 448.0).all())


def test_mxfp4_checkpoint_preparation_matches_oracle_codec():
    # the synthetic 4-bit checkpoint follows the OCP MX FP4 rule the oracle
    # implements (independently: torch ops here, C there)
    import numpy as np
    import oracle
    from synth import _mxfp4_rows
    g = torch.Generator().manual_seed(0)
    w = torch.randn(64, 256, generator=g) * 0.02
    w[3, :32] = 0.0
    w[5, 40] = -0.0
    w[7, 64:96] = torch.linspace(-7.0, 7.0, 32)
    q, s = _mxfp4_rows(w)
    oq, os_ = oracle.quant_mx(w.numpy(), 4)
    np.testing.assert_array_equal(q.numpy(), oq)
    np.testing.assert_array_equal(s.numpy(), os_)
