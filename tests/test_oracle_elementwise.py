"""Pins for the oracle's RMSNorm, SiLU and RoPE (oracle/decoder.py).

Each is checked against closed forms, invariants, and an independent library
routine or formulation (torch.nn.functional, complex rotation).
"""
import numpy as np
import torch

from oracle import rmsnorm, silu, rope


def test_rmsnorm_vs_torch_and_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 96))
    w = 1 + 0.1 * rng.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(rmsnorm(x, w, 1e-6), ref, rtol=1e-12, atol=1e-12)
    # constant row c: each entry is c / sqrt(c^2 + eps)
    c = 3.0
    got = rmsnorm(np.full(8, c), np.ones(8), 1e-6)
    np.testing.assert_allclose(got, c / np.sqrt(c * c + 1e-6), rtol=1e-15)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(256)
    a = rmsnorm(x, np.ones(256), 0.0)
    b = rmsnorm(7.5 * x, np.ones(256), 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean(a * a)), 1.0, rtol=1e-13)


def test_silu_vs_torch_and_identities():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-12, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(x) - silu(-x), x, rtol=1e-12, atol=1e-12)


def _rope_complex(x, pos, theta):
    """Independent formulation: pair (x_i, x_{i+D/2}) as x_i + i x_{i+D/2},
    multiplied by exp(i * pos * theta^(-2i/D))."""
    d = x.shape[-1]
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = theta ** (-np.arange(0, d, 2) / d)
    z = z * np.exp(1j * pos * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_vs_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 128))
    for pos in (0, 1, 17, 4095, 32767):
        np.testing.assert_allclose(rope(x, pos, 1e6), _rope_complex(x, pos, 1e6), rtol=1e-9, atol=1e-9)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_array_equal(rope(q, 0, 1e6), q)
    r = rope(q, 123, 1e6)
    pairs = lambda v: v[:32] ** 2 + v[32:] ** 2
    np.testing.assert_allclose(pairs(r), pairs(q), rtol=1e-12)
    # <R_m q, R_n k> depends only on m - n
    a = rope(q, 50, 1e4) @ rope(k, 20, 1e4)
    b = rope(q, 1030, 1e4) @ rope(k, 1000, 1e4)
    np.testing.assert_allclose(a, b, rtol=1e-9)


def test_rope_d2_is_plain_rotation_by_pos_radians():
    got = rope(np.array([1.0, 0.0]), 2, 1e6)
    np.testing.assert_allclose(got, [np.cos(2.0), np.sin(2.0)], rtol=1e-15)


def test_rope_batched_positions():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 3, 16))
    pos = np.array([0, 5, 9, 100])
    got = rope(x, pos, 1e6)
    for b in range(4):
        np.testing.assert_allclose(got[b], _rope_complex(x[b], pos[b], 1e6), rtol=1e-10, atol=1e-12)
