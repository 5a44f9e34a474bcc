"""Pins for the oracle's paged GQA decode attention (oracle/decoder.py).

What pins it, independent of its own code: torch's scaled_dot_product_attention
on contiguous K/V (a library routine the oracle does not use), bit-exact
invariance under physical block permutations (paged == contiguous), closed
forms (one token, constant V, q = 0, one-hot scores, two tokens, a designed
log-sum-exp), GQA == MHA with repeated KV heads, probabilities summing to 1,
fp8 == f16 on the dequantised values, and NaN poison outside the context.
"""
import numpy as np
import pytest
import torch

from oracle import paged_attention, paged_attention_batch, kv_append, e4m3_decode
import pkv_inputs as inp

BS = 16


def _scatter(k_tok, v_tok, n_blocks, rng=None, order=None):
    """Write contiguous per-token K/V [c, Hkv, D] into fresh NaN pools through the
    oracle's own append, one token at a time, on a block table drawn from a
    permutation.  Returns (k_pool, v_pool, block_row)."""
    c, hkv, d = k_tok.shape
    need = (c + BS - 1) // BS
    ids = order if order is not None else rng.permutation(n_blocks)[:need]
    kp = np.full((n_blocks, hkv, BS, d), np.nan, np.float16)
    vp = np.full((n_blocks, hkv, BS, d), np.nan, np.float16)
    row = np.full(need, -1, np.int32)
    row[:] = ids[:need]
    for t in range(c):
        kv_append(kp, vp, k_tok[t][None], v_tok[t][None], row[None], np.array([t + 1]))
    return kp, vp, row


def _sdpa(q, k, v, scale):
    """torch SDPA with GQA on contiguous K/V: q [Hq,D], k/v [c,Hkv,D]."""
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]     # [1,Hq,1,D]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]  # [1,Hkv,c,D]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,d,c", [(4, 2, 64, 37), (12, 2, 128, 200), (7, 1, 8, 16), (6, 6, 32, 5), (28, 4, 128, 129)])
def test_vs_torch_sdpa(hq, hkv, d, c):
    rng = np.random.default_rng(hq * 1000 + c)
    k = rng.standard_normal((c, hkv, d)).astype(np.float16)
    v = rng.standard_normal((c, hkv, d)).astype(np.float16)
    q = rng.standard_normal((hq, d)).astype(np.float16)
    kp, vp, row = _scatter(k, v, (c + BS - 1) // BS + 5, rng)
    got = paged_attention(q, kp, vp, row, c, 1 / np.sqrt(d))
    np.testing.assert_allclose(got, _sdpa(q, k, v, 1 / np.sqrt(d)), rtol=1e-12, atol=1e-12)


def test_block_permutation_invariance_bit_exact():
    rng = np.random.default_rng(5)
    c, hkv, d = 150, 2, 64
    k = rng.standard_normal((c, hkv, d)).astype(np.float16)
    v = rng.standard_normal((c, hkv, d)).astype(np.float16)
    q = rng.standard_normal((6, d)).astype(np.float16)
    need = (c + BS - 1) // BS
    a = _scatter(k, v, need, order=np.arange(need))            # contiguous
    b = _scatter(k, v, need + 7, rng)                           # permuted
    oa = paged_attention(q, *a, c, 0.125)
    ob = paged_attention(q, *b, c, 0.125)
    assert np.array_equal(oa, ob)


def test_single_token_returns_v():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((1, 2, 64)).astype(np.float16)
    v = rng.standard_normal((1, 2, 64)).astype(np.float16)
    q = rng.standard_normal((4, 64)).astype(np.float16)
    kp, vp, row = _scatter(k, v, 3, rng)
    o = paged_attention(q, kp, vp, row, 1, 0.125)
    assert np.array_equal(o, np.repeat(v[0].astype(np.float64), 2, axis=0))


def test_constant_v_and_zero_q():
    rng = np.random.default_rng(7)
    c = 45
    k = rng.standard_normal((c, 1, 32)).astype(np.float16)
    v = np.full((c, 1, 32), 0.75, np.float16)
    kp, vp, row = _scatter(k, v, 6, rng)
    o = paged_attention(rng.standard_normal((3, 32)).astype(np.float16), kp, vp, row, c, 0.2)
    np.testing.assert_allclose(o, 0.75, rtol=1e-14)
    v2 = rng.standard_normal((c, 1, 32)).astype(np.float16)
    kp, vp, row = _scatter(k, v2, 6, rng)
    o0 = paged_attention(np.zeros((2, 32), np.float16), kp, vp, row, c, 0.2)
    np.testing.assert_allclose(o0, np.repeat(v2.astype(np.float64).mean(0), 2, axis=0), rtol=1e-12, atol=1e-14)


def test_one_hot_probe_selects_token_exactly():
    """q = 64 e_0, K_t[0] = 64 only at t*: the t* score is 4096 / sqrt(D) and every
    other score 0, so exp(-512) underflows the weights of all other tokens."""
    rng = np.random.default_rng(8)
    c, d = 70, 64
    for tstar in (0, 15, 16, 69):
        k = np.zeros((c, 1, d), np.float16)
        k[tstar, 0, 0] = 64
        v = rng.standard_normal((c, 1, d)).astype(np.float16)
        q = np.zeros((1, d), np.float16)
        q[0, 0] = 64
        kp, vp, row = _scatter(k, v, 9, rng)
        o = paged_attention(q, kp, vp, row, c, 1 / np.sqrt(d))
        assert np.array_equal(o[0], v[tstar, 0].astype(np.float64))


def test_two_tokens_closed_form():
    d = 4
    k = np.zeros((2, 1, d), np.float16)
    k[0, 0, 0], k[1, 0, 0] = 1, 3
    v = np.zeros((2, 1, d), np.float16)
    v[0, 0, 1], v[1, 0, 1] = 2, -6
    q = np.zeros((1, d), np.float16)
    q[0, 0] = 1
    kp, vp, row = _scatter(k, v, 1, order=np.array([0]))
    o, lse, p = paged_attention(q, kp, vp, row, 2, 0.5, return_weights=True)
    # scores 0.5 and 1.5: p1 = 1 / (1 + e^-1)
    p1 = 1 / (1 + np.exp(-1.0))
    np.testing.assert_allclose(p[0], [1 - p1, p1], rtol=1e-15)
    np.testing.assert_allclose(o[0, 1], 2 * (1 - p1) - 6 * p1, rtol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(np.exp(0.5) + np.exp(1.5)), rtol=1e-15)


def test_lse_geometric_series_and_weights_sum_to_one():
    """K_t[0] = t/8 and q = e_0 * 8 with scale a give scores a*t: lse = log sum e^{a t}."""
    c, d, a = 40, 16, 0.05
    k = np.zeros((c, 1, d), np.float16)
    k[:, 0, 0] = (np.arange(c) / 8).astype(np.float16)
    v = np.random.default_rng(9).standard_normal((c, 1, d)).astype(np.float16)
    q = np.zeros((1, d), np.float16)
    q[0, 0] = 8
    kp, vp, row = _scatter(k, v, 4, order=np.array([3, 0, 2]))
    _, lse, p = paged_attention(q, kp, vp, row, c, a, return_weights=True)
    r = np.exp(a)
    np.testing.assert_allclose(lse[0], np.log((r ** c - 1) / (r - 1)), rtol=1e-13)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=1e-14)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(10)
    c, hkv, grp, d = 33, 2, 3, 16
    k = rng.standard_normal((c, hkv, d)).astype(np.float16)
    v = rng.standard_normal((c, hkv, d)).astype(np.float16)
    q = rng.standard_normal((hkv * grp, d)).astype(np.float16)
    gq = paged_attention(q, *_scatter(k, v, 5, rng), c, 0.3)
    km, vm = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    mh = paged_attention(q, *_scatter(km, vm, 5, rng), c, 0.3)
    assert np.array_equal(gq, mh)


def test_fp8_equals_f16_on_dequantised_values():
    case = inp.attention_case(3, 7, 1, 64, 1, 50, seed=11, kv_dtype="fp8")
    k_real = (e4m3_decode(case.k_pool) * case.k_scale)
    v_real = (e4m3_decode(case.v_pool) * case.v_scale)
    o8, _ = paged_attention_batch(case.q, case.k_pool, case.v_pool, case.block_tables, case.ctx_lens,
                                  case.scale, k_scale=case.k_scale, v_scale=case.v_scale)
    # f64 pools hold the dequantised values exactly
    of = np.stack([paged_attention(case.q[b], k_real, v_real, case.block_tables[b], int(case.ctx_lens[b]), case.scale)
                   for b in range(3)]).astype(np.float16)
    assert np.array_equal(o8, of)


def test_poisoned_slots_never_read_and_inactive_rows():
    case = inp.attention_case(5, 4, 2, 64, 1, 40, seed=12, ctx_lens=[1, 16, 17, 0, 40])
    assert np.isnan(case.k_pool).any() and np.isnan(case.v_pool).any()
    o, lse = paged_attention_batch(case.q, case.k_pool, case.v_pool, case.block_tables, case.ctx_lens, case.scale)
    assert np.all(np.isfinite(o))
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3]))
