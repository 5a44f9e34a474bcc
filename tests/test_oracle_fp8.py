"""Pins for the oracle's E4M3 decoder (oracle/fp8.py).

The format is OCP E4M3FN (reading of "FP8 E4M3" in the rvLLM post, section
"PagedAttention과 FlashAttention-3").  Pinned against the format's own special
values and against torch's independent float8_e4m3fn implementation.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_table
import pkv_inputs as inp


def test_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9), (0x01, 2.0 ** -9), (0x40, 2.0), (0x3F, 1.875),
])
def test_special_values(code, value):
    got = e4m3_decode(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_nan_codes_only():
    t = e4m3_table()
    assert set(np.nonzero(np.isnan(t))[0].tolist()) == {0x7F, 0xFF}
    assert np.nanmax(np.abs(t)) == 448.0


def test_monotone_positive_codes():
    t = e4m3_table()[:0x7F]
    assert np.all(np.diff(t) > 0)


def test_quantiser_roundtrip_and_saturation():
    vals = e4m3_table()[np.r_[0:0x7F, 0x80:0xFF]].astype(np.float32)
    codes, s = inp.quantize_e4m3(vals, amax=448.0)
    assert s == 1.0
    assert np.array_equal(e4m3_decode(codes), vals.astype(np.float64))
    c2, s2 = inp.quantize_e4m3(np.array([1e6, -1e6, 3.0], np.float32), amax=448.0)
    assert e4m3_decode(c2).tolist() == [448.0, -448.0, 3.0]
    assert not np.any(np.isnan(e4m3_decode(c2)))
