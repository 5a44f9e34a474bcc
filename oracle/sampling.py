"""Sampling of the next token from one row of logits: penalties, temperature,
top-k, top-p and a draw with a uniform number passed in by the caller.

The zingnex.cn article lists the request parameters (section 支持的参数):
temperature (default 1.0, 0 decodes greedily), top_p (default 1.0, nucleus
threshold) and top_k (default -1, disabled); its CPU-operation table (section
CPU操作优化) names repetition, frequency and presence penalties, applied
together.  The rvLLM post (section "CUDA 그래프 리플레이") keeps sampling
outside the captured forward pass.  The pages give no formula; the reading
taken here, step by step:

  0. Penalties, from the row's token counts c (how many times each token was
     already sampled for this row): for every token with c > 0, in float32,
         x = x / r if x > 0 else x * r      (repetition penalty r; 1 = off)
         x = (x - f * c) - p                (frequency f, presence p; 0 = off)
     and the result is rounded to f16, like the logits it replaces.
  1. temperature <= 0: the greedy token (lowest index among the largest
     logits, a NaN never winning; 0 for a row of NaNs only).
  2. Each finite logit x gets an integer weight W(x) = floor(2^40 E(y)) with
     y = (x - m) * (1 / T) in float32 (m = the largest finite logit) and E the
     float32 exponential of ``exp_f32`` below, so every mass and every
     comparison of the draw is an exact integer computation (a token decision
     taken in one stated precision on both sides).
  3. top_k > 0: keep every finite token whose logit is at least the k-th
     largest (counted with multiplicity; ties at the boundary all kept).
  4. top_p < 1: with M(t) the summed W of the kept tokens whose logit is >= t,
     target = ceil(max(top_p, 0) * M(-inf)) in float64, keep the tokens whose
     logit is >= the largest logit value t with M(t) >= target (ties kept;
     target 0 keeps the largest logit and its ties).
  5. The draw: with Z the summed W of the kept tokens and
     u24 = floor(u * 2^24) (u clamped to [0, 1)), the first kept token in
     index order whose running sum of W exceeds floor(u24 * Z / 2^24).
A row whose logits are all non-finite gets token 0.

Test infrastructure only (see the package docstring).
"""
import numpy as np

F32 = np.float32
TWO40 = 1 << 40

# float32 constants of the exponential (Cody-Waite split of ln 2, Taylor
# coefficients 1/k!)
_L2E = F32(1.4426950408889634)
_LN2_HI = F32(0.693359375)
_LN2_LO = F32(-2.12194440e-4)
_COEF = [F32(1.0 / 5040.0), F32(1.0 / 720.0), F32(1.0 / 120.0), F32(1.0 / 24.0), F32(1.0 / 6.0), F32(0.5),
         F32(1.0), F32(1.0)]


def exp_f32(y):
    """e^y for float32 y <= 0, evaluated in float32 with one rounding per
    operation: n = floor(y log2(e) + 1/2); r = (y - n c1) - n c2 with
    c1 + c2 = ln 2 (c1 exact in 9 bits); e^r by its degree-7 Taylor polynomial
    in Horner form; the result 2^n e^r.  Returns float32 (0 for y < -30)."""
    y = np.asarray(y, dtype=F32)
    small = ~(y >= F32(-30.0))
    y = np.where(small, F32(0.0), y)
    n = np.floor(y * _L2E + F32(0.5))
    r = (y - n * _LN2_HI) - n * _LN2_LO
    p = _COEF[0]
    for c in _COEF[1:]:
        p = p * r + c
    out = np.ldexp(p, n.astype(np.int32)).astype(F32)
    return np.where(small, F32(0.0), out)


def weight_fixed(x, m, temperature):
    """W(x) = floor(2^40 exp_f32((x - m) * (1 / T))) (uint64) for f16 logits
    x <= m; every value is at most 2^40, so sums over a row stay exact in
    uint64."""
    with np.errstate(over="ignore", invalid="ignore"):
        inv_t = F32(1.0) / F32(temperature)
        d = np.asarray(x, dtype=F32) - F32(m)
        y = np.where(d == F32(0.0), F32(0.0), d * inv_t)   # the maximum has weight 1 even when 1/T overflows
        e = exp_f32(y)
    q = np.ldexp(e, 40)                       # exact scaling
    return np.floor(q).astype(np.uint64)


def apply_penalties(logits, counts, repetition, frequency, presence):
    """Step 0 for one row: f16 logits and int counts -> penalised f16 logits."""
    x = np.asarray(logits, dtype=np.float16).astype(F32)
    c = np.asarray(counts, dtype=np.int64)
    seen = c > 0
    r, f, p = F32(repetition), F32(frequency), F32(presence)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.where(x > 0, x / r, x * r)
        y = (y - f * c.astype(F32)) - p
    out = np.where(seen, y, x)
    return out.astype(np.float16)


def _key_order(x16):
    """Logit values as float32 (order of the f16 logits; -0 == +0)."""
    return np.asarray(x16, dtype=np.float16).astype(F32)


def candidates(logits, temperature, top_k, top_p):
    """Kept token ids (ascending) and their integer weights W (uint64) for one
    row of f16 logits (steps 2-4)."""
    x = _key_order(logits)
    keep = np.isfinite(x)
    if not keep.any():
        return np.zeros(0, np.int64), np.zeros(0, np.uint64)
    m = x[keep].max()
    if top_k > 0 and top_k < keep.sum():
        kth = np.sort(x[keep])[::-1][top_k - 1]
        keep &= x >= kth
    w = np.zeros(x.shape, dtype=np.uint64)
    w[keep] = weight_fixed(x[keep], m, temperature)
    if top_p < 1.0:
        frac = max(float(F32(top_p)), 0.0)
        total = int(w[keep].sum(dtype=np.uint64))
        target = int(np.ceil(np.float64(frac) * np.float64(total))) if frac > 0 else 0
        # the kept tokens' mass per distinct logit value, from the largest value down
        vals, inv = np.unique(x[keep], return_inverse=True)
        mass = np.zeros(vals.shape, np.uint64)
        np.add.at(mass, inv, w[keep])
        run = np.cumsum(mass[::-1], dtype=np.uint64)      # mass at or above each value
        i = np.nonzero(run >= np.uint64(target))[0]
        t = vals[::-1][i[0] if i.size else -1]
        keep &= x >= t
    ids = np.nonzero(keep)[0]
    return ids, w[ids]


def draw(ids, w, u):
    """Step 5: the first id whose running sum of W exceeds floor(u24 Z / 2^24)."""
    u = float(u)
    u = 0.0 if not (u > 0.0) else min(u, float(np.nextafter(F32(1.0), F32(0.0))))
    u24 = int(np.floor(np.float64(F32(u)) * (1 << 24)))
    run = np.cumsum(np.asarray(w, dtype=np.uint64), dtype=np.uint64)
    z = int(run[-1])
    t = (u24 * z) >> 24
    j = int(np.searchsorted(run, np.uint64(t), side="right"))   # first running sum > t
    assert j < len(ids), "the running sum always passes floor(u24 Z / 2^24) < Z"
    return int(ids[j])


def sample_row(logits, temperature, top_k, top_p, u):
    """The sampled token id for one row of f16 logits (steps 1-5)."""
    x = _key_order(logits)
    if not (float(temperature) > 0.0):
        # the greedy token: lowest index among the largest logits, a NaN never
        # winning (-inf beats NaN); 0 when every logit is NaN
        valid = ~np.isnan(x)
        if not valid.any():
            return 0
        return int(np.flatnonzero(valid & (x == x[valid].max()))[0])
    ids, w = candidates(logits, temperature, top_k, top_p)
    if ids.size == 0:
        return 0
    return draw(ids, w, u)


def sample(logits, temperature, top_k, top_p, u):
    """sample_row for every row of [B, V] f16 logits with per-row parameters."""
    return np.array([sample_row(logits[b], temperature[b], top_k[b], top_p[b], u[b])
                     for b in range(logits.shape[0])], dtype=np.int32)


def sample_penalized(logits, counts, repetition, frequency, presence, temperature, top_k, top_p, u):
    """Steps 0-5 for every row; returns (tokens, penalised logits, counts after
    adding each row's sampled token)."""
    pen = np.stack([apply_penalties(logits[b], counts[b], repetition[b], frequency[b], presence[b])
                    for b in range(logits.shape[0])])
    tok = sample(pen, temperature, top_k, top_p, u)
    new_counts = np.array(counts, dtype=np.int32, copy=True)
    new_counts[np.arange(len(tok)), tok] += 1
    return tok, pen, new_counts
