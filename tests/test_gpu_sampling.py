"""GPU parity of the sampler (temperature / top-k / top-p and the inverse-CDF
draw, through the C ABI) against the oracle.

The kernel sums weights in float32 and the oracle in float64, so the two may
pick neighbouring tokens when the caller's uniform lands within rounding of a
boundary of the cumulative mass, or when top_p * Z lands within rounding of
the mass at a candidate threshold.  Each row therefore checks:
  * greedy rows (temperature 0), top-k = 1 rows and inactive rows: exact;
  * otherwise, when top_p * Z is at least 1e-4 Z away from the masses on both
    sides of tau: the token is one the oracle keeps, and u * Z' falls inside
    that token's interval of the oracle's cumulative mass, widened by 3e-5 Z'
    (so the token is the oracle's whenever u is farther than that from the
    interval's ends);
  * when top_p * Z is that close to a boundary: the token is kept by the
    oracle at top_p + 1e-3.
The count of rows that must equal the oracle exactly keeps the test from
passing on the loose checks alone."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev

pytestmark = pytest.mark.gpu

DRAW_TOL = 3e-5
TOP_P_MARGIN = 1e-4


def run_sample(pkv, case, with_lens=True):
    b = case.logits.shape[0]
    tokens = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    pkv.sample(dev(case.logits), dev(case.temperature), dev(case.top_k), dev(case.top_p), dev(case.uniform),
               tokens, context_lens=dev(case.lens) if with_lens else None)
    torch.cuda.synchronize()
    return tokens.cpu().numpy()


def top_p_margin(logits, t, k, p):
    """Distance (relative to Z) of top_p * Z from the nearest mass the
    threshold search compares it with; inf when top-p is off."""
    if not p < 1.0:
        return np.inf
    _, w = oracle.candidates(logits, t, k, 1.0)
    vals = np.sort(w)[::-1]
    cum = np.cumsum(vals)
    z = cum[-1]
    return np.min(np.abs(cum - p * z)) / z


def check_rows(case, got):
    exact = 0
    for b in range(case.logits.shape[0]):
        lg, t, k, p, u = (case.logits[b], float(case.temperature[b]), int(case.top_k[b]),
                          float(case.top_p[b]), float(case.uniform[b]))
        if case.lens is not None and case.lens[b] == 0:
            assert got[b] == -1, b
            continue
        want = oracle.sample_row(lg, t, k, p, u)
        if t == 0.0 or k == 1:
            assert got[b] == want, (b, t, k, got[b], want)
            exact += 1
            continue
        if top_p_margin(lg, t, k, p) < TOP_P_MARGIN:
            wide, _ = oracle.candidates(lg, t, k, min(1.0, p + 1e-3))
            assert got[b] in wide, (b, got[b])
            continue
        ids, w = oracle.candidates(lg, t, k, p)
        assert got[b] in ids, (b, t, k, p, got[b], want)
        j = int(np.searchsorted(ids, got[b]))
        cum = np.cumsum(w)
        zk = cum[-1]
        lo = cum[j - 1] if j > 0 else 0.0
        assert lo - DRAW_TOL * zk <= u * zk <= cum[j] + DRAW_TOL * zk, (b, got[b], want, u, lo / zk, cum[j] / zk)
        exact += int(got[b] == want)
    return exact


@pytest.mark.parametrize("batch,vocab,seed", [
    (40, 151936, 1),     # Qwen2.5 vocabulary, 16-byte row loads
    (45, 1000, 2),       # small vocabulary, 16-byte row loads
    (36, 997, 3),        # odd vocabulary: element loads, ragged per-thread chunks
    (10, 37, 4),         # fewer tokens than threads
    (12, 70001, 8),      # element loads, wave segments longer than the kept step sums
])
def test_sample_parity(lib, batch, vocab, seed):
    case = inp.sampling_case(batch, vocab, seed)
    got = run_sample(lib, case)
    exact = check_rows(case, got)
    active = int((case.lens > 0).sum())
    assert exact >= 0.8 * active, (exact, active)


def test_sample_without_lens_and_uniform_edges(lib):
    """No length array (every row active); a uniform of 0 takes the first kept
    token, one just below 1 a token at the far end of the kept mass."""
    case = inp.sampling_case(24, 5000, 5, masked_rows=False)
    case.temperature[:] = 0.8
    case.top_k[:] = np.where(np.arange(24) % 2, 40, -1)
    case.top_p[:] = 1.0
    case.uniform[:] = np.where(np.arange(24) % 3 == 0, 0.0, np.float32(0.99999994))
    got = run_sample(lib, case, with_lens=False)
    for b in range(0, 24, 3):
        ids, _ = oracle.candidates(case.logits[b], 0.8, int(case.top_k[b]), 1.0)
        assert got[b] == ids[0], b
    case.lens = None
    check_rows(case, got)


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
    ids, w = oracle.candidates(row, 1.2, 10, 0.8)
    counts = np.bincount(got, minlength=vocab)
    assert counts.sum() == n and set(np.nonzero(counts)[0]) <= set(ids.tolist())
    assert np.max(np.abs(counts[ids] / n - w / w.sum())) <= 2.0 / n


def test_sample_host_errors(lib):
    x = torch.zeros(2, 8, dtype=torch.float16, device="cuda")
    f = torch.zeros(2, dtype=torch.float32, device="cuda")
    i = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        lib.sample(x.float(), f, i, f, f, i)
    with pytest.raises(lib.PkvError, match="batch and vocab"):
        lib.sample(x[:, :0], f, i, f, f, i)
