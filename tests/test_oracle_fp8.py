"""Pins of the oracle's e4m3 decoding (FP8 Q/K/V inputs): every one of the
256 codes against torch's float8_e4m3fn, and the format's closed forms."""
import numpy as np
import torch

import oracle


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_decode(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_decode_closed_forms():
    d = oracle.fp8_e4m3_decode
    assert d(0x38) == 1.0 and d(0xB8) == -1.0          # exponent 7 = bias
    assert d(0x7E) == 448.0                            # largest finite
    assert d(0x01) == 2.0 ** -9                        # smallest subnormal
    assert d(0x08) == 2.0 ** -6                        # smallest normal
    assert d(0x3C) == 1.5 and d(0x40) == 2.0
    assert np.signbit(d(0x80)) and d(0x80) == 0.0


def test_dequant_scales():
    codes = np.array([[[0x38, 0x40, 0xB8]]], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.dequant_fp8(codes, 0.25), [[[0.25, 0.5, -0.25]]])
