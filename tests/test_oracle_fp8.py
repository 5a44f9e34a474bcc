"""Pins for the oracle's E4M3 decoder and encoder (oracle/fp8.py).

The format is OCP E4M3FN (reading of "FP8 E4M3" in the rvLLM post, section
"PagedAttention과 FlashAttention-3").  Pinned against the format's own special
values and against torch's independent float8_e4m3fn implementation.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, e4m3_quantize, e4m3_table
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


# ------------------------------------------------------------------ encoder

def _torch_cast(x):
    """torch's float8_e4m3fn conversion (round to nearest even), as codes."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_roundtrips_every_finite_code():
    codes = np.r_[0:0x7F, 0x80:0xFF].astype(np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes).astype(np.float32)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    assert np.array_equal(e4m3_encode(x), _torch_cast(x))


def test_encode_ties_go_to_even_code():
    t = e4m3_table()[:0x7F]
    mid = ((t[:-1] + t[1:]) / 2).astype(np.float32)       # exact in float32
    assert np.array_equal(mid.astype(np.float64), (t[:-1] + t[1:]) / 2)
    got = e4m3_encode(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    assert np.array_equal(e4m3_encode(-mid), got | 0x80)
    assert np.array_equal(got, _torch_cast(mid))


def test_encode_saturates_and_keeps_nan():
    x = np.array([448.0, 460.0, 464.0, 1e9, np.inf, -500.0, -np.inf, np.nan, -np.nan, 0.0, -0.0], np.float32)
    got = e4m3_encode(x)
    assert got.tolist()[:7] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[7] in (0x7F, 0xFF) and got[8] in (0x7F, 0xFF)
    assert got[9] == 0x00 and got[10] == 0x80


def test_quantize_decides_in_float32():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(5000) * 3).astype(np.float16)
    s = np.float32(0.0137)
    q = (x.astype(np.float32) / s).astype(np.float32)
    got = e4m3_quantize(x, s)
    inr = np.abs(q) < 448
    assert np.array_equal(got[inr], _torch_cast(q[inr]))
    assert np.all(got[~inr] & 0x7F == 0x7E)
    back = e4m3_decode(got) * s
    assert np.max(np.abs(back - x.astype(np.float64))[inr] / np.maximum(np.abs(x[inr]), 1e-3)) < 0.07
