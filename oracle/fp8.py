"""OCP FP8 E4M3 ("E4M3FN") decoding, written from the format's definition.

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
