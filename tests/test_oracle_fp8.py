"""Pin the oracle's OCP e4m3fn codec (the FP8 checkpoint form named in "Hugging
Face releases Beam ..." and "Reflection Beam", section "Where to run it")
against torch.float8_e4m3fn: every code decodes to torch's value, and binary32
values encode to torch's round-to-nearest-even code; and the FP8 activation
recipe inside the forward, against numpy matmuls on the round-tripped x and h,
with copies of the oracle carrying planted mistakes that the pin must catch."""
import numpy as np
import pytest
import torch

import oracle


def test_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(want)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    mags = 2.0 ** rng.uniform(-12, np.log2(448.0), 60000)
    v = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    # exact code values, midpoints between neighbouring codes, and zeros
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    v = np.concatenate([v, vals.astype(np.float32), -vals.astype(np.float32),
                        mids.astype(np.float32), -mids.astype(np.float32),
                        np.array([0.0, -0.0], np.float32)])
    v = v[np.abs(v) <= 448.0]
    got = oracle.e4m3_encode(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)


def test_encode_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e9, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode(v) == 0x7E)
    assert np.all(oracle.e4m3_encode(-v) == 0xFE)
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


# ---- the FP8 activation recipe inside the forward (act_quant=True) --------
# One expert at routing weight 1 turns the forward into a dense SwiGLU whose
# x and h go through the e4m3 recipe; weights are e4m3 codes with power-of-
# two block scales, so their dequantised values are exact.  The reference is
# numpy float64 matmuls on values decoded by torch's e4m3fn, h rounded to
# binary32 and then to bfloat16 by torch before its quantisation.

def _fp8_layer(seed):
    from synth import small_shape
    sh = small_shape(hidden=256, intermediate=256, n_experts=1, n_groups=1,
                     topk_groups=1, top_k=1)
    rng = np.random.default_rng(seed)
    T = 5
    x = rng.standard_normal((T, sh.hidden)).astype(np.float32)
    x[1, :128] *= 1e-3                  # blocks of one row on different scales
    x[3, 128:] *= 40.0
    H, I = sh.hidden, sh.intermediate
    codes_gu = rng.integers(0, 0x7F, (1, 2 * I, H)).astype(np.uint8)
    codes_gu[codes_gu & 0x78 == 0x78] &= 0x70      # keep codes finite (no 0x7F)
    codes_gu |= (rng.integers(0, 2, codes_gu.shape) << 7).astype(np.uint8)
    codes_d = rng.integers(0, 0x7F, (1, H, I)).astype(np.uint8)
    codes_d[codes_d & 0x78 == 0x78] &= 0x70
    codes_d |= (rng.integers(0, 2, codes_d.shape) << 7).astype(np.uint8)
    s_gu = (2.0 ** rng.integers(-14, -10, (1, 2 * I // 128, H // 128))).astype(np.float32)
    s_d = (2.0 ** rng.integers(-14, -10, (1, H // 128, I // 128))).astype(np.float32)
    return sh, x, codes_gu, s_gu, codes_d, s_d


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _fp8_reference(x, codes_gu, s_gu, codes_d, s_d, I):
    def dq_w(codes, s):
        return _e4m3_values(codes[0]) * np.repeat(np.repeat(s[0].astype(np.float64), 128, 0), 128, 1)

    def round_trip(v):
        q, s = oracle.quant_e4m3(v.astype(np.float32), 128)
        return _e4m3_values(q) * np.repeat(s.astype(np.float64), 128, axis=-1)

    Wgu, Wd = dq_w(codes_gu, s_gu), dq_w(codes_d, s_d)
    xq = round_trip(x)
    g, u = xq @ Wgu[:I].T, xq @ Wgu[I:].T
    h = g / (1.0 + np.exp(-g)) * u
    h_bf = torch.from_numpy(h.astype(np.float32)).bfloat16().float().numpy()
    return round_trip(h_bf) @ Wd.T


def _fp8_forward(sh, x, codes_gu, s_gu, codes_d, s_d):
    T = x.shape[0]
    return oracle.forward_tokens(sh, np.arange(T), x, np.zeros((T, 1), np.int32),
                                 np.ones((T, 1), np.float32), codes_gu, codes_d,
                                 s_gu, s_d, act_quant=True)


def test_forward_fp8_activation_recipe_single_expert():
    sh, x, cgu, sgu, cd, sd = _fp8_layer(11)
    got = _fp8_forward(sh, x, cgu, sgu, cd, sd)
    ref = _fp8_reference(x, cgu, sgu, cd, sd, sh.intermediate)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # without the activation recipe the output differs well beyond that
    plain = oracle.forward_tokens(sh, np.arange(x.shape[0]), x,
                                  np.zeros((x.shape[0], 1), np.int32),
                                  np.ones((x.shape[0], 1), np.float32), cgu, cd, sgu, sd)
    assert np.abs(plain - ref).max() > 1e-3 * np.abs(ref).max()


# Copies of the oracle's source with one planted mistake each in the FP8
# activation branch; every one must fail the pin above.
FP8_MUTANTS = {
    "h not round-tripped": (
        "      else if (act_quant) fake_quant_row(hv, I, 128, hv, tf, tq, ts, 1);",
        "      else if (0) fake_quant_row(hv, I, 128, hv, tf, tq, ts, 1);"),
    "x not round-tripped": (
        "    else if (act_quant) fake_quant_row(xr, H, 128, xr, tf, tq, ts, 0);",
        "    else if (0) fake_quant_row(xr, H, 128, xr, tf, tq, ts, 0);"),
    "h not rounded to bf16": (
        "      else if (act_quant) fake_quant_row(hv, I, 128, hv, tf, tq, ts, 1);",
        "      else if (act_quant) fake_quant_row(hv, I, 128, hv, tf, tq, ts, 0);"),
    "scale of the wrong block": (
        "    out[i] = bo_e4m3_decode(tmpq[i]) * (double)tmps[i / block];",
        "    out[i] = bo_e4m3_decode(tmpq[i]) * (double)tmps[(i / block) ^ 1];"),
    "codes left unscaled": (
        "    out[i] = bo_e4m3_decode(tmpq[i]) * (double)tmps[i / block];",
        "    out[i] = bo_e4m3_decode(tmpq[i]);"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_recipe_pin_catches_planted_mistakes(name, tmp_path):
    from oracle import build as ob
    old, new = FP8_MUTANTS[name]
    src = open(ob.SRC).read()
    assert src.count(old) == 1, "the mutation site moved"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = ob.compile_to(str(path), str(tmp_path / "libmutant.so"))
    sh, x, cgu, sgu, cd, sd = _fp8_layer(11)
    ref = _fp8_reference(x, cgu, sgu, cd, sd, sh.intermediate)
    with oracle.library(so):
        got = _fp8_forward(sh, x, cgu, sgu, cd, sd)
    assert not np.allclose(got, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_quant_scale_rule_on_tiny_blocks():
    # scale = amax/448 in binary32, 1 where that quotient is zero; codes
    # saturate (a subnormal scale is coarse, so v/scale can pass 448)
    v = np.zeros((4, 128), np.float32)
    v[0, :] = np.linspace(-1, 1, 128, dtype=np.float32) * np.float32(1e-39)
    v[1, 5] = np.float32(3e-43)            # 3e-43/448 underflows to zero
    v[2, 7] = np.float32(-8.8e-43)         # quotient rounds to the smallest subnormal
    v[3, :] = np.float32(1e-40) * np.arange(1, 129, dtype=np.float32)
    q, s = oracle.quant_e4m3(v, 128)
    for r in range(4):
        amax = np.float32(np.abs(v[r]).max())
        sc = np.float32(amax / np.float32(448.0))
        sc = sc if sc > 0 else np.float32(1.0)
        assert s[r, 0].view(np.uint32) == sc.view(np.uint32)
        want = oracle.e4m3_encode(np.minimum(np.maximum(v[r] / sc, -448), 448))
        np.testing.assert_array_equal(q[r], want)
        assert not np.any((q[r] & 0x7F) == 0x7F)           # never a NaN code
    assert s[1, 0] == 1.0 and np.all(q[1] == 0)
    # the coarse scale of row 2 puts its maximum past 448: saturated, not NaN
    assert abs(v[2, 7] / s[2, 0]) > 448 and q[2, 7] == 0xFE
