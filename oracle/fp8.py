"""OCP FP8 E4M3 ("E4M3FN") decoding and encoding, written from the format's
definition.

The rvLLM post (discuss.pytorch.kr, section "PagedAttention과 FlashAttention-3")
names an FP8 E4M3 quantised KV cache without fixing the variant or the scale
granularity.  Reading taken: the OCP 8-bit floating point E4M3 format
(1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
is subnormal; the all-ones exponent with all-ones mantissa is NaN; no
infinities; largest finite magnitude 448), with one float32 scale per tensor
(value = decoded code * scale).

Test infrastructure only (see the package docstring).
"""
import numpy as np


def e4m3_decode(codes, acc=np.float64):
    """Decode uint8 E4M3 codes to real values, exactly, in ``acc``.

    Follows the format definition field by field: sign s = bit 7,
    exponent e = bits 6..3, mantissa m = bits 2..0.
      e == 0:             (-1)^s * (m / 8) * 2^(1 - 7)
      e == 15 and m == 7: NaN
      otherwise:          (-1)^s * (1 + m / 8) * 2^(e - 7)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 8.0) * 2.0 ** (1 - 7)
    nor = sign * (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    out = np.where(e == 0, sub, nor)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out.astype(acc)


def e4m3_table(acc=np.float64):
    """All 256 codes decoded, indexed by code."""
    return e4m3_decode(np.arange(256, dtype=np.uint8), acc)


def e4m3_encode(x):
    """Encode float32 values to E4M3 codes: the nearest representable value,
    ties to the even code (even mantissa), magnitudes beyond the largest
    finite value (448) saturated to it, NaN to the NaN code 0x7F with the
    input's sign.

    Written as a search over the 254 finite values of the decode table, so it
    shares no bit manipulation with any other encoder: for each input the
    candidate codes at minimal distance are found and, of two, the one whose
    lowest code bit is 0 is taken (adjacent codes differ by one in the last
    mantissa bit, including across exponent steps).  The sign is handled
    separately so that -0.0 keeps its sign bit.
    """
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    mags = e4m3_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0x00..0x7E: 0 .. 448
    codes = np.arange(0x7F)
    out = np.empty(flat.shape, dtype=np.uint8)
    for c0 in range(0, flat.size, 4096):
        v = flat[c0:c0 + 4096]
        a = np.abs(v)
        dist = np.abs(a[:, None] - mags[None, :])          # [n, 127]
        near = dist == dist.min(axis=1, keepdims=True)     # one or two candidates
        # of two equally near codes, the even one; else the only one
        pick = np.where(near & (codes[None, :] % 2 == 0), codes[None, :], -1).max(axis=1)
        only = np.where(near, codes[None, :], -1).max(axis=1)
        code = np.where(near.sum(axis=1) > 1, pick, only)
        code = np.where(a >= 448.0, 0x7E, code)             # saturate (inf included)
        code = np.where(np.isnan(v), 0x7F, code)
        sign = np.where(np.signbit(v), 0x80, 0)
        out[c0:c0 + 4096] = (code | sign).astype(np.uint8)
    return out.reshape(x.shape)


def e4m3_quantize(x_f16, scale):
    """E4M3 codes of f16 values under a per-tensor scale: the quotient
    f32(x) / scale is formed in float32 (the precision in which the code is
    decided), then encoded by e4m3_encode."""
    q = np.asarray(x_f16, dtype=np.float16).astype(np.float32) / np.float32(scale)
    return e4m3_encode(q)
