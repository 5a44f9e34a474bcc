"""Pins for the oracle's sampler (oracle/sampling.py): greedy at temperature
0, closed-form probabilities on a 3-token example (the logits of the rvLLM
post's usage example), the inverse-CDF draw against torch's softmax, top-k /
top-p kept sets against brute-force enumeration, ties at both thresholds kept
(the reading of zingnex.cn, section 支持的参数), the float32 exponential and
the 2^-40 fixed-point weights against numpy's double-precision exp, and the
repetition / frequency / presence penalties (zingnex.cn, section CPU操作优化)
in closed form."""
import numpy as np
import pytest
import torch

from oracle import candidates, greedy_argmax, sample, sample_row
from oracle.sampling import apply_penalties, draw, exp_f32, sample_penalized, weight_fixed


def test_temperature_zero_is_greedy():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((5, 300)).astype(np.float16)
    lg[1, [7, 200]] = 20.0            # tie: lowest index
    lg[2, 50] = np.nan
    got = sample(lg, [0.0] * 5, [-1] * 5, [1.0] * 5, [0.3] * 5)
    assert got.tolist() == greedy_argmax(lg).tolist()


# Reading R10 by hand: the lowest index among the largest logits, a NaN never
# winning (so -inf beats NaN), token 0 for a row of NaNs only.
GREEDY_CORNERS = [
    ([np.nan, -np.inf, -np.inf], 1),
    ([np.nan, np.nan, np.nan], 0),
    ([-np.inf, np.nan, -np.inf], 0),
    ([1.0, np.nan, 3.0, 3.0], 2),
    ([np.nan, np.inf, 5.0, np.inf], 1),
    ([-0.0, 0.0, np.nan], 0),
    ([np.nan, -2.0, -1.0, -1.0], 2),
]


@pytest.mark.parametrize("row,tok", GREEDY_CORNERS)
def test_greedy_corners_by_hand(row, tok):
    lg = np.array(row, np.float16)
    assert int(greedy_argmax(lg[None])[0]) == tok
    assert sample_row(lg, 0.0, -1, 1.0, 0.5) == tok


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
        w = w.astype(np.float64)
        q = w / w.sum()                                  # renormalised kept probabilities
        # fixed-point weights of a float32 exponential: a few float32 roundings
        assert np.allclose(q, p[ids] / p[ids].sum(), rtol=2e-6, atol=0)


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


def test_exp_f32_against_double_exp():
    """The float32 exponential within 3 float32 roundings of numpy's double exp
    on every float32 value in [-30, 0] sampled densely, exact at 0, 0 below
    -30 and non-decreasing."""
    y = np.concatenate([np.linspace(-30, 0, 1_000_001, dtype=np.float32),
                        -np.logspace(-30, 1, 20001).astype(np.float32), np.float32([0.0, -0.0])])
    y.sort()
    e = exp_f32(y)
    ref = np.exp(y.astype(np.float64))
    assert np.max(np.abs(e - ref) / ref) <= 3 * 2.0 ** -24
    assert np.all(np.diff(e) >= 0)
    assert exp_f32(np.float32(0.0)) == 1.0
    assert np.all(exp_f32(np.float32([-30.5, -100.0, -np.inf])) == 0.0)


def test_weight_fixed_closed_forms():
    # the maximum weighs exactly 2^40; one step of ln 2 below it, 2^39 within rounding
    assert int(weight_fixed(np.float16(3.0), np.float16(3.0), 0.7)) == 1 << 40
    assert int(weight_fixed(np.float16(3.0), np.float16(3.0), 1e-40)) == 1 << 40   # 1/T overflows
    w = int(weight_fixed(np.float16(-np.log(2.0)), np.float16(0.0), 1.0))
    assert abs(w - (1 << 39)) <= (1 << 39) * 4e-4        # the f16 rounding of -ln 2
    x = np.arange(-40.0, 0.25, 0.25).astype(np.float16)
    got = weight_fixed(x, np.float16(0.0), 1.3).astype(np.float64)
    y = x.astype(np.float64) / np.float64(np.float32(1.3))
    want = np.floor(np.exp(y) * 2.0 ** 40)
    # the exponential's roundings plus the float32 rounding of y (relative |y| 2^-24 in e^y)
    assert np.all(np.abs(got - want) <= np.maximum(want * (4 + 2 * np.abs(y)) * 2.0 ** -24, 1.0))
    assert np.all(got[y < -30.01] == 0)


def test_draw_is_an_integer_inverse_cdf():
    ids = np.array([3, 5, 9])
    w = np.array([1 << 38, 1 << 39, 1 << 40], np.uint64)   # masses 1/7, 2/7, 4/7
    assert draw(ids, w, 0.0) == 3 and draw(ids, w, np.nan) == 3 and draw(ids, w, -1.0) == 3
    assert draw(ids, w, 1.0) == 9 and draw(ids, w, 0.9999999) == 9
    # boundaries at 1/7 and 3/7 of the mass: u24 = floor(u 2^24) and t = floor(u24 Z / 2^24)
    b1 = (1 << 24) // 7                                   # largest u24 with t < Z/7 ... or equal
    for u24, tok in ((b1, 3), (b1 + 1, 5), (3 * (1 << 24) // 7, 5), (3 * (1 << 24) // 7 + 1, 9)):
        z = 7 << 38
        t = (u24 * z) >> 24
        want = 3 if t < (1 << 38) else (5 if t < 3 << 38 else 9)
        assert want == tok, (u24, t)
        assert draw(ids, w, u24 / float(1 << 24)) == tok


def test_penalties_closed_forms():
    x = np.array([2.0, -2.0, 1.0, -1.0, 0.0, 3.0, np.nan, -np.inf, np.inf], np.float16)
    c = np.array([1, 1, 0, 0, 2, 3, 1, 1, 1])
    got = apply_penalties(x, c, 2.0, 0.5, 0.25)
    # seen: positive / r, negative * r, then - f c - p; unseen tokens unchanged bit for bit
    want = np.array([2 / 2 - 0.5 - 0.25, -2 * 2 - 0.5 - 0.25, 1.0, -1.0, 0.0 - 1.0 - 0.25,
                     3 / 2 - 1.5 - 0.25, np.nan, -np.inf, np.inf], np.float16)
    assert np.array_equal(got.view(np.uint16)[:6], want.view(np.uint16)[:6])
    assert np.isnan(got[6]) and got[7] == -np.inf and got[8] == np.inf
    assert np.array_equal(apply_penalties(x, np.zeros(9, int), 1.3, 0.7, 0.1).view(np.uint16), x.view(np.uint16))
    # neutral parameters leave every seen logit unchanged too
    assert np.array_equal(apply_penalties(x[:6], c[:6], 1.0, 0.0, 0.0).view(np.uint16), x[:6].view(np.uint16))
    # rounding to f16 after the float32 arithmetic: 1/3 of a logit of 1
    assert apply_penalties(np.float16([1.0]), [1], 3.0, 0.0, 0.0)[0] == np.float16(np.float32(1.0) / np.float32(3.0))


def test_penalised_greedy_and_counts():
    lg = np.zeros((2, 6), np.float16)
    lg[:, 4], lg[:, 2] = 5.0, 4.5
    counts = np.zeros((2, 6), np.int32)
    counts[0, 4] = 1                                      # row 0 already produced token 4
    tok, pen, new = sample_penalized(lg, counts, [1.0, 1.0], [0.0, 0.0], [1.0, 1.0], [0.0, 0.0], [-1, -1],
                                     [1.0, 1.0], [0.5, 0.5])
    assert tok.tolist() == [2, 4]                         # presence 1 pushes token 4 below token 2 in row 0
    assert pen[0, 4] == np.float16(4.0) and pen[1, 4] == np.float16(5.0)
    assert new[0, 4] == 1 and new[0, 2] == 1 and new[1, 4] == 1 and new.sum() == 3
