"""Pins of the oracle's OCP MX codecs (MXFP4 weights, MXFP8 activations) and
of its MXFP4 expert forward.  The 4-bit variant stands in for the pages'
4-bit checkpoint on CDNA4 (its MFMA applies E8M0 block scales); the format
definitions come from the OCP MX v1.0 specification (tests/golden)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import small_shape

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ocp_mx_e2m1.json")))
MAG = np.array(G["e2m1_magnitudes"])
TABLE = np.concatenate([MAG, -MAG])          # value of code c


def test_e2m1_values_match_specification():
    got = oracle.e2m1_decode(range(16))
    np.testing.assert_array_equal(got[:8], MAG)
    np.testing.assert_array_equal(np.abs(got[8:]), MAG)
    assert np.all(np.signbit(got[8:]))


def _brute_e2m1(v):
    """Nearest table value; ties to the even code; saturation at 6."""
    out = []
    for a in np.asarray(v, np.float64).ravel():
        d = np.abs(TABLE[:8] - abs(a))
        best = min(range(8), key=lambda c: (d[c], c & 1))
        out.append(best | (8 if np.signbit(a) else 0))
    return np.array(out, np.uint8)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(0)
    mids = (MAG[:-1] + MAG[1:]) / 2
    v = np.concatenate([rng.uniform(-8, 8, 3000), mids, -mids, MAG, -MAG,
                        [6.5, 100.0, -1e9, 0.25, 0.75, 5.0, -5.0]])
    np.testing.assert_array_equal(oracle.e2m1_encode(v), _brute_e2m1(v))


@pytest.mark.parametrize("emax", [G["e2m1_emax"], G["e4m3_emax"]])
def test_scale_rule_top_binade(emax):
    rng = np.random.default_rng(emax)
    amax = np.exp(rng.uniform(np.log(1e-20), np.log(1e20), 2000))
    for a in amax:
        s = oracle.mx_scale(a, emax)
        ratio = a / 2.0 ** (s - G["e8m0_bias"])
        assert 2.0 ** emax <= ratio < 2.0 ** (emax + 1), (a, s)
    assert oracle.mx_scale(0.0, emax) == 0
    codes = torch.tensor([0, 1, 100, 127, 128, 200, 254], dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref, 2.0 ** (codes.numpy().astype(np.float64) - 127))


def test_activation_scale_rule_no_saturation():
    # the 4-bit variant's activation exponent: smallest power of two with
    # amax / 2^x <= 448, i.e. the block maximum lands in (224, 448]
    rng = np.random.default_rng(9)
    amax = np.concatenate([np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 3000)),
                           [448.0, 449.0, 224.0, 224.5, 1.0, 2.0 ** -120]])
    for a in amax:
        s = oracle.mx8_act_scale(a)
        ratio = a / 2.0 ** (s - G["e8m0_bias"])
        # (at the bottom of the E8M0 range the block maximum may sit lower)
        assert (224.0 < ratio or s == 0) and ratio <= 448.0, (a, s)
    assert oracle.mx8_act_scale(0.0) == 0
    v = (rng.standard_normal((50, 64)) * 3.0).astype(np.float32)
    q, sc = oracle.quant_mx(v, 8)
    vals = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all(np.abs(vals) <= 448.0)
    for r in range(50):
        for b in range(2):
            blk = np.abs(v[r, 32 * b:32 * b + 32]).max()
            assert sc[r, b] == oracle.mx8_act_scale(blk)


def test_mxfp8_elements_match_torch():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((9, 256)) * np.logspace(-3, 3, 9)[:, None]).astype(np.float32)
    v[2, :32] = 0.0
    q, s = oracle.quant_mx(v, 8)
    scale = 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=1) - 127)
    u = np.clip(v.astype(np.float64) / scale, -448.0, 448.0)
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)


def test_mxfp4_elements_and_packing():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((5, 128)) * 3).astype(np.float32)
    q, s = oracle.quant_mx(v, 4)
    lo, hi = q & 15, q >> 4
    codes = np.empty(v.shape, np.uint8)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    scale = 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=1) - 127)
    np.testing.assert_array_equal(codes.ravel(), _brute_e2m1((v / scale).ravel()))


def _dequant_mxfp4(q, s):
    codes = np.empty(q.shape[:-1] + (2 * q.shape[-1],), np.uint8)
    codes[..., 0::2], codes[..., 1::2] = q & 15, q >> 4
    return (TABLE[codes] * 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=-1) - 127)).astype(np.float32)


def test_forward_mxfp4_equals_dequantised_f32():
    sh = small_shape(hidden=128, intermediate=64, n_experts=8, n_groups=2, topk_groups=2, top_k=2)
    rng = np.random.default_rng(5)
    T = 6
    x = rng.standard_normal((T, sh.hidden)).astype(np.float32)
    wgu = (rng.standard_normal((sh.n_experts, 2 * sh.intermediate, sh.hidden)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((sh.n_experts, sh.hidden, sh.intermediate)) * 0.05).astype(np.float32)
    qgu, sgu = oracle.quant_mx(wgu, 4)
    qd, sd = oracle.quant_mx(wd, 4)
    idx = np.stack([rng.choice(sh.n_experts, 2, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.5, 1.5, (T, 2)).astype(np.float32)
    a = oracle.forward_tokens(sh, np.arange(T), x, idx, w, qgu, qd, sgu, sd)
    b = oracle.forward_tokens(sh, np.arange(T), x, idx, w, _dequant_mxfp4(qgu, sgu),
                              _dequant_mxfp4(qd, sd))
    np.testing.assert_array_equal(a, b)


def test_forward_mxfp4_activation_recipe_single_expert():
    # one expert, weight 1: the act_quant forward is a dense SwiGLU whose x
    # and h go through MXFP8 (numpy matmuls on the dequantised values)
    sh = small_shape(hidden=128, intermediate=64, n_experts=1, n_groups=1, topk_groups=1, top_k=1)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    wgu = (rng.standard_normal((1, 128, 128)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((1, 128, 64)) * 0.05).astype(np.float32)
    qgu, sgu = oracle.quant_mx(wgu, 4)
    qd, sd = oracle.quant_mx(wd, 4)
    got = oracle.forward_tokens(sh, np.arange(4), x, np.zeros((4, 1), np.int32),
                                np.ones((4, 1), np.float32), qgu, qd, sgu, sd, act_quant=True)

    def mx8(v):
        q, s = oracle.quant_mx(v.astype(np.float32), 8)
        vals = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return vals * 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=-1) - 127)
    Wgu = _dequant_mxfp4(qgu, sgu)[0].astype(np.float64)
    Wd = _dequant_mxfp4(qd, sd)[0].astype(np.float64)
    xq = mx8(x)
    g, u = xq @ Wgu[:64].T, xq @ Wgu[64:].T
    h = g / (1 + np.exp(-g)) * u
    ref = mx8(h) @ Wd.T
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_mx_recipe_study_reproduces():
    # The stored study behind the 4-bit GPU bar (tests/golden/mx_recipe_study.py,
    # oracle only): re-run two of its layers, a single token and a 33-token
    # batch, and check the stored figures and summary.
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import mx_recipe_study as st
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "mx_recipe_study.json")) as f:
        data = json.load(f)
    assert data["n"] == len(data["cases"]) >= 20
    assert any(c["T"] == 1 for c in data["cases"])
    errs = [c["layer_err"] for c in data["cases"]]
    assert data["max"] == max(errs)
    for c in (data["cases"][0], data["cases"][11]):
        whole, rows = st.study_one(c["H"], c["I"], c["E"], c["T"], c["seed"])
        assert whole == pytest.approx(c["layer_err"], rel=1e-12)
        assert rows == pytest.approx(c["worst_row_err"], rel=1e-12)
