"""The tile layouts include/pkv.h documents for the paged KV cache, checked
against the converters the GPU tests use to load pools (CPU only)."""
import numpy as np
import pytest

from gpu_util import k_from_lib, k_to_lib, v_from_lib, v_to_lib


def _pool(dtype, d):
    x = (np.arange(2 * 3 * 16 * d, dtype=np.int64) * 7919 % 251).reshape(2, 3, 16, d)
    return x.astype(np.uint8) if dtype == "fp8" else x.astype(np.float16)


@pytest.mark.parametrize("dtype", ["f16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_k_tile_layout(dtype, d):
    k = _pool(dtype, d)                       # [NB, Hkv, 16 tokens, D]
    lib = k_to_lib(k).reshape(2, 3, -1)
    c = 16 if dtype == "fp8" else 8
    for t in range(16):
        for dd in range(d):
            assert lib[1, 2, ((dd // c) * 16 + t) * c + dd % c] == k[1, 2, t, dd]
    assert np.array_equal(k_from_lib(k_to_lib(k)), k)


@pytest.mark.parametrize("dtype", ["f16", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_v_tile_layout(dtype, d):
    v = _pool(dtype, d)                       # [NB, Hkv, 16 tokens, D], as K
    lib = v_to_lib(v).reshape(2, 3, -1)
    for t in range(16):
        for dd in range(d):
            if dtype == "fp8":
                off = (((dd // 64) * 4 + t // 4) * 16 + dd % 16) * 16 + ((dd // 16) % 4) * 4 + t % 4
            else:
                off = dd * 16 + t
            assert lib[0, 1, off] == v[0, 1, t, dd]
    assert np.array_equal(v_from_lib(v_to_lib(v)), v)
