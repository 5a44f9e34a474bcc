"""Pins for the oracle's sampler (oracle/sampling.py): greedy at temperature
0, closed-form probabilities on a 3-token example (the logits of the rvLLM
post's usage example), the inverse-CDF draw against torch's softmax, top-k /
top-p kept sets against brute-force enumeration, and ties at both thresholds
kept (the reading of zingnex.cn, section 支持的参数)."""
import numpy as np
import pytest
import torch

from oracle import candidates, greedy_argmax, sample, sample_row


def test_temperature_zero_is_greedy():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((5, 300)).astype(np.float16)
    lg[1, [7, 200]] = 20.0            # tie: lowest index
    lg[2, 50] = np.nan
    got = sample(lg, [0.0] * 5, [-1] * 5, [1.0] * 5, [0.3] * 5)
    assert got.tolist() == greedy_argmax(np.nan_to_num(lg, nan=-np.inf)).tolist()


@pytest.mark.parametrize("u", [0.0, 0.4, 0.999])
def test_top_k_one_is_argmax(u):
    rng = np.random.default_rng(2)
    lg = rng.standard_normal(1000).astype(np.float16)
    assert sample_row(lg, 0.7, 1, 1.0, u) == int(np.argmax(lg))


def test_three_token_example_closed_form():
    # softmax([1, 2, 3] / 0.8): weights exp((x - 3) / 0.8) = e^-2.5, e^-1.25, 1
    w = np.array([np.exp(-2.5), np.exp(-1.25), 1.0])
    c = np.cumsum(w) / w.sum()            # CDF boundaries in index order
    lg = np.array([1.0, 2.0, 3.0], np.float16)
    for u, tok in ((0.0, 0), (c[0] - 1e-6, 0), (c[0] + 1e-6, 1), (c[1] - 1e-6, 1), (c[1] + 1e-6, 2), (0.999999, 2)):
        assert sample_row(lg, 0.8, 50, 1.0, u) == tok, (u, tok)


def test_inverse_cdf_matches_torch_softmax():
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal(20) * 2).astype(np.float16)
    n = 20000
    us = (np.arange(n) + 0.5) / n
    counts = np.bincount([sample_row(lg, 1.3, -1, 1.0, u) for u in us], minlength=20) / n
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)) / 1.3, 0).numpy()
    assert np.max(np.abs(counts - p)) <= 2.0 / n


def test_top_k_keeps_ties_and_disables():
    lg = np.array([5, 4, 4, 4, 1, 0], np.float16)
    ids, _ = candidates(lg, 1.0, 2, 1.0)
    assert ids.tolist() == [0, 1, 2, 3]
    for k in (-1, 0, 6, 100):
        assert candidates(lg, 1.0, k, 1.0)[0].tolist() == list(range(6))


def test_top_p_is_the_smallest_descending_prefix():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal(50).astype(np.float16)
    lg = np.unique(lg)[:40]                              # distinct values
    rng.shuffle(lg)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), 0).numpy()
    order = np.argsort(-p, kind="stable")
    for top_p in (0.05, 0.3, 0.5, 0.9, 0.999):
        n = 1
        while p[order[:n]].sum() < top_p:                # enumerate prefix sizes
            n += 1
        ids, w = candidates(lg, 1.0, -1, top_p)
        assert sorted(order[:n].tolist()) == ids.tolist(), top_p
        q = w / w.sum()                                  # renormalised kept probabilities
        assert np.allclose(q, p[ids] / p[ids].sum(), rtol=1e-12, atol=0)


def test_top_p_keeps_ties_at_the_threshold():
    lg = np.array([3.0, 3.0, 1.0, 0.0], np.float16)
    # one of the two tied tokens alone would carry > 0.4 of the mass; both are kept
    assert candidates(lg, 1.0, -1, 0.4)[0].tolist() == [0, 1]


def test_draw_walks_kept_tokens_in_index_order():
    lg = np.array([0.0, 2.0, 1.0, 2.0], np.float16)
    ids, w = candidates(lg, 1.0, 2, 1.0)                 # keeps 1 and 3 (tied at 2.0)
    assert ids.tolist() == [1, 3]
    assert sample_row(lg, 1.0, 2, 1.0, 0.49) == 1 and sample_row(lg, 1.0, 2, 1.0, 0.51) == 3


def test_top_p_matches_enumeration_with_many_ties():
    """Logits on a coarse grid (long runs of equal weights): the kept set is the
    one found by trying every distinct weight from the top down."""
    rng = np.random.default_rng(5)
    lg = rng.integers(-4, 5, 300).astype(np.float16)
    z = lg.astype(np.float64) / 0.9
    w = np.exp(z - z.max())
    for top_p in (0.0, 0.1, 0.35, 0.6, 0.95):
        for t in np.unique(w)[::-1]:
            if w[w >= t].sum() >= top_p * w.sum():
                break
        want = np.nonzero(w >= t)[0]
        assert candidates(lg, 0.9, -1, top_p)[0].tolist() == want.tolist(), top_p
