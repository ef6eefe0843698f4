"""Pin the oracle's OCP e4m3fn codec (the FP8 checkpoint form named in "Hugging
Face releases Beam ..." and "Reflection Beam", section "Where to run it")
against torch.float8_e4m3fn: every code decodes to torch's value, and binary32
values encode to torch's round-to-nearest-even code."""
import numpy as np
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
