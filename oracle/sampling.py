"""Sampling of the next token from one row of logits: temperature, top-k,
top-p and a draw with a uniform number passed in by the caller.

The zingnex.cn article (section 支持的参数) lists the request parameters:
temperature (default 1.0, 0 decodes greedily), top_p (default 1.0, nucleus
threshold) and top_k (default -1, disabled).  The rvLLM post (section "CUDA
그래프 리플레이") keeps sampling outside the captured forward pass.  The pages
give no formula; the reading taken here, step by step:

  1. temperature == 0: the greedy token (lowest index of the largest logit).
  2. z = logits / temperature (float32 logits widened).
  3. top_k > 0: keep every token whose z is at least the k-th largest z
     (counted with multiplicity; ties at the boundary are all kept).
  4. w = exp(z - max z) over the kept tokens; Z = sum w.
  5. top_p < 1: keep every token whose w is at least tau, where tau is the
     largest weight such that the kept tokens with w >= tau carry at least
     top_p * Z (ties at tau all kept).
  6. The draw: with the kept mass Z', the first kept token in index order
     whose running sum of w exceeds u * Z' (u in [0, 1), one per row); if
     rounding leaves none, the last kept token.

Test infrastructure only (see the package docstring).
"""
import numpy as np


def candidates(logits, temperature, top_k, top_p):
    """Kept token ids (ascending) and their weights w for one row (fp64)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64) / float(temperature)
    keep = np.isfinite(z)
    if top_k > 0 and top_k < keep.sum():
        kth = np.sort(z[keep])[::-1][top_k - 1]
        keep &= z >= kth
    m = z[keep].max()
    w = np.where(keep, np.exp(np.where(keep, z - m, 0.0)), 0.0)
    if top_p < 1.0:
        total = w.sum()
        vals = np.sort(w[keep])[::-1]
        cum = np.cumsum(vals)
        # The first position whose running mass reaches top_p * Z holds tau:
        # every larger value ends its run of ties earlier, below the target,
        # and the mass of w >= tau (its ties included) is at least cum there.
        i = np.nonzero(cum >= top_p * total)[0]
        tau = vals[i[0] if i.size else -1]
        keep &= w >= tau
    ids = np.nonzero(keep)[0]
    return ids, w[ids]


def sample_row(logits, temperature, top_k, top_p, u):
    """The sampled token id for one row (steps 1-6 of the module docstring)."""
    x = np.asarray(logits, dtype=np.float32)
    if temperature == 0.0:
        finite = np.where(np.isnan(x), -np.inf, x)
        return int(np.flatnonzero(finite == finite.max())[0])
    ids, w = candidates(x, temperature, top_k, top_p)
    cum = np.cumsum(w)
    hit = np.nonzero(cum > u * cum[-1])[0]
    return int(ids[hit[0]] if hit.size else ids[-1])


def sample(logits, temperature, top_k, top_p, u):
    """sample_row for every row of [B, V] logits with per-row parameters."""
    return np.array([sample_row(logits[b], temperature[b], top_k[b], top_p[b], u[b])
                     for b in range(logits.shape[0])], dtype=np.int32)
