"""GPU parity of the sampler (penalties, temperature / top-k / top-p and the
inverse-CDF draw, through the C ABI) against the oracle.

Weights are 2^-40 fixed-point integers of a float32 exponential that both
sides evaluate operation by operation, and every mass and comparison is an
exact integer, so the sampled token must equal the oracle's on every row;
the penalised logits must equal the oracle's f16 values bit for bit (NaN
payloads aside) and the token counts must gain exactly the sampled tokens."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev

pytestmark = pytest.mark.gpu


def run_sample(pkv, case, with_lens=True):
    b = case.logits.shape[0]
    tokens = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    pkv.sample(dev(case.logits), dev(case.temperature), dev(case.top_k), dev(case.top_p), dev(case.uniform),
               tokens, context_lens=dev(case.lens) if with_lens else None)
    torch.cuda.synchronize()
    return tokens.cpu().numpy()


def oracle_tokens(case):
    want = oracle.sample(case.logits, case.temperature, case.top_k, case.top_p, case.uniform)
    if case.lens is not None:
        want[case.lens == 0] = -1
    return want


@pytest.mark.parametrize("batch,vocab,seed", [
    (40, 151936, 1),     # Qwen2.5 vocabulary, 16-byte row loads
    (45, 1000, 2),       # small vocabulary, 16-byte row loads
    (36, 997, 3),        # odd vocabulary: element loads, ragged per-thread chunks
    (10, 37, 4),         # fewer tokens than threads
    (12, 70001, 8),      # element loads, wave segments longer than the kept step sums
    (8, 600000, 9),      # 16-byte loads, wave segments longer than the kept step sums
])
def test_sample_parity(lib, batch, vocab, seed):
    case = inp.sampling_case(batch, vocab, seed)
    got = run_sample(lib, case)
    want = oracle_tokens(case)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(int(b), int(got[b]), int(want[b])) for b in bad[:8]]


def test_sample_without_lens_and_uniform_edges(lib):
    """No length array (every row active); a uniform of 0 (or NaN, or
    negative) takes the first kept token of non-zero weight; values of 1 or
    more count as 1 - 2^-24."""
    case = inp.sampling_case(24, 5000, 5, masked_rows=False)
    case.temperature[:] = 0.8
    case.top_k[:] = np.where(np.arange(24) % 2, 40, -1)
    case.top_p[:] = 1.0
    case.uniform[:] = np.array([0.0, 0.99999994, np.nan, -0.5, 1.0, 7.0], np.float32)[np.arange(24) % 6]
    got = run_sample(lib, case, with_lens=False)
    case.lens = None
    assert np.array_equal(got, oracle_tokens(case))
    for b in range(24):
        if b % 6 in (0, 2, 3):
            ids, w = oracle.candidates(case.logits[b], 0.8, int(case.top_k[b]), 1.0)
            assert got[b] == ids[np.nonzero(w > 0)[0][0]], b


def test_sample_degenerate_rows(lib):
    """Rows with no finite logit (token 0 when sampling), NaN before -inf at
    temperature 0 (the -inf wins), a +inf logit (never kept when sampling,
    the greedy winner), all-equal logits (ties kept at both thresholds) and a
    single finite logit among -inf: the sampled token equals the oracle's."""
    V = 1000
    rng = np.random.default_rng(31)
    rows, params = [], []
    def add(row, t, k, p, u):
        rows.append(np.asarray(row, np.float16))
        params.append((t, k, p, u))
    ninf = np.full(V, -np.inf)
    nan = np.full(V, np.nan)
    lead_nan = ninf.copy(); lead_nan[0] = np.nan
    pinf = rng.standard_normal(V); pinf[[3, 400]] = np.inf; pinf[7] = np.nan
    one = ninf.copy(); one[500] = 1.25
    flat = np.full(V, 1.5)
    for t in (0.0, 0.7):
        add(ninf, t, -1, 1.0, 0.3)
        add(nan, t, 5, 0.9, 0.3)
        add(lead_nan, t, -1, 0.5, 0.6)
        add(pinf, t, -1, 1.0, 0.4)
        add(pinf, t, 10, 0.8, 0.9)
        add(one, t, 5, 0.2, 0.99)
        add(flat, t, 3, 0.5, 0.73)
        add(flat, t, -1, 0.0, 0.11)
    lg = np.stack(rows)
    t, k, p, u = (np.array(c, dt) for c, dt in zip(zip(*params), (np.float32, np.int32, np.float32, np.float32)))
    case = inp.SamplingCase(lg, t, k, p, u, np.ones(len(rows), np.int32))
    got = run_sample(lib, case)
    want = oracle_tokens(case)
    assert want[:3].tolist() == [0, 0, 1] and want[8:11].tolist() == [0, 0, 0]
    assert np.array_equal(got, want), list(zip(got.tolist(), want.tolist()))


def test_sample_distribution_matches_softmax(lib):
    """One small row repeated with evenly spaced uniforms: the token counts
    follow softmax(z) restricted to the top-k / top-p set."""
    rng = np.random.default_rng(6)
    n, vocab = 4096, 24
    row = (rng.standard_normal(vocab) * 1.5).astype(np.float16)
    case = inp.SamplingCase(np.tile(row, (n, 1)), np.full(n, 1.2, np.float32), np.full(n, 10, np.int32),
                            np.full(n, 0.8, np.float32), ((np.arange(n) + 0.5) / n).astype(np.float32),
                            np.ones(n, np.int32))
    got = run_sample(lib, case)
    assert np.array_equal(got, oracle_tokens(case))
    ids, w = oracle.candidates(row, 1.2, 10, 0.8)
    w = w.astype(np.float64)
    counts = np.bincount(got, minlength=vocab)
    assert counts.sum() == n and set(np.nonzero(counts)[0]) <= set(ids.tolist())
    assert np.max(np.abs(counts[ids] / n - w / w.sum())) <= 2.0 / n


def _same_f16(a, b):
    """Bit-equal f16 arrays, NaN payloads aside."""
    a, b = np.asarray(a), np.asarray(b)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint16) == b.view(np.uint16))))


@pytest.mark.parametrize("batch,vocab,seed", [(40, 151936, 11), (33, 997, 12)])
def test_sample_penalized_parity_over_steps(lib, batch, vocab, seed):
    """Four sampling steps in a row on fresh logits, the counts carried over on
    the device: penalised logits, tokens and counts equal the oracle's."""
    counts, rep, freq, pres = inp.penalty_case(batch, vocab, seed)
    counts_d = dev(counts)
    rep_d, freq_d, pres_d = dev(rep), dev(freq), dev(pres)
    for step in range(4):
        case = inp.sampling_case(batch, vocab, seed * 10 + step)
        logits_d = dev(case.logits)
        tokens = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
        lib.sample_penalized(logits_d, dev(case.temperature), dev(case.top_k), dev(case.top_p), rep_d, freq_d,
                             pres_d, dev(case.uniform), counts_d, tokens, context_lens=dev(case.lens))
        torch.cuda.synchronize()
        active = case.lens > 0
        tok_w, pen_w, counts_w = oracle.sample_penalized(case.logits, counts, rep, freq, pres, case.temperature,
                                                         case.top_k, case.top_p, case.uniform)
        tok_w[~active] = -1
        counts_w[~active] = counts[~active]           # inactive rows: no penalty, no count
        pen_w[~active] = case.logits[~active]
        got_tok = tokens.cpu().numpy()
        assert np.array_equal(got_tok, tok_w), (step, np.nonzero(got_tok != tok_w)[0][:8])
        assert _same_f16(logits_d.cpu().numpy(), pen_w), step
        got_counts = counts_d.cpu().numpy()
        assert np.array_equal(got_counts, counts_w), step
        counts = got_counts


def test_sample_host_errors(lib):
    x = torch.zeros(2, 8, dtype=torch.float16, device="cuda")
    f = torch.zeros(2, dtype=torch.float32, device="cuda")
    i = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        lib.sample(x.float(), f, i, f, f, i)
    with pytest.raises(lib.PkvError, match="batch and vocab"):
        lib.sample(x[:, :0], f, i, f, f, i)
    c = torch.zeros(2, 8, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="counts"):
        lib.sample_penalized(x, f, i, f, f, f, f, f, c[:, :4], i)
