"""Seeded synthetic inputs for the paged-KV GQA decode step.

This module only draws random numbers and lays them out; it holds none of the
decode arithmetic.  Both the oracle tests and the HIP path are fed from here,
so the two sides see identical arrays.

Recipe (all draws from numpy.random.default_rng(seed), PCG64, in fp32 and
rounded to f16 with round-to-nearest-even):

* context lengths: ``uniform`` -> integers in [lo, hi] inclusive;
  ``loguniform`` -> floor(exp(U(ln lo, ln(hi + 1)))), clipped to [lo, hi].
* block tables: each row needs ceil(c / 16) blocks; the pool holds
  ceil(1.25 * sum) blocks; a random permutation of the pool ids is dealt to the
  rows in order.  Table entries past a row's blocks are -1.
* K / V pools: N(0, 1) for every slot that holds a cached token; every other
  slot (tail of a row's last block, blocks no row owns) is NaN (f16) or the
  E4M3 NaN code 0x7F (fp8), so a kernel that reads outside the valid context
  poisons its output.
* fp8 pools: N(0, 1) values are quantised per tensor with scale s = amax / 448
  (torch's float32 -> float8_e4m3fn cast, round to nearest even); the decoded
  value of a code is code_value * s.
* weights: every matrix, the embedding and the QKV bias ~ N(0, 0.02); RMSNorm
  gains are 1 (the usual initialisation) unless ``norm_jitter`` asks for
  1 + N(0, 0.1), which unit tests use to catch indexing mistakes.
"""
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
F16 = np.float16
E4M3_NAN = 0x7F


@dataclass(frozen=True)
class Shape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6


# Workloads: model shapes of the Qwen2.5-1.5B / 7B decoders and the two
# attention-only cases (sizes as the workload descriptions state them).
TINY = Shape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, vocab=512, n_layers=1)
QWEN15 = Shape(hidden=1536, n_q_heads=12, n_kv_heads=2, head_dim=128, ffn=8960, vocab=151936, n_layers=28)
QWEN7 = Shape(hidden=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, ffn=18944, vocab=152064, n_layers=28)


@dataclass(frozen=True)
class AttnWorkload:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_lo: int
    ctx_hi: int
    dist: str = "uniform"
    kv_dtype: str = "f16"
    seed: int = 1002


ATTN15 = AttnWorkload(64, 12, 2, 128, 128, 2048, "uniform", "f16", 1002)
FP8LONG = AttnWorkload(32, 28, 4, 128, 1024, 32768, "loguniform", "fp8", 1005)


def context_lengths(rng, batch, lo, hi, dist="uniform"):
    if dist == "uniform":
        c = rng.integers(lo, hi + 1, size=batch)
    elif dist == "loguniform":
        c = np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi + 1), size=batch)))
        c = np.clip(c, lo, hi)
    else:
        raise ValueError(dist)
    return c.astype(np.int32)


def deal_block_tables(rng, ctx_lens, max_context=None, pool_factor=1.25, min_blocks=0):
    """Random physical block ids for every row.

    Returns (block_tables [B, stride] int32 with -1 padding, num_blocks).
    stride = ceil(max_context / 16) (max_context defaults to max(ctx_lens)).
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    need = (ctx_lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    if max_context is None:
        max_context = int(ctx_lens.max()) if ctx_lens.size else 1
    stride = max(1, (max_context + BLOCK_SIZE - 1) // BLOCK_SIZE)
    total = int(need.sum())
    num_blocks = max(int(np.ceil(pool_factor * total)), total, min_blocks, 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((len(ctx_lens), stride), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, num_blocks


def valid_slot_masks(block_tables, ctx_lens, num_blocks):
    """Boolean [num_blocks, 16]: True where a slot holds a token of some row."""
    m = np.zeros((num_blocks, BLOCK_SIZE), dtype=bool)
    for b, c in enumerate(np.asarray(ctx_lens)):
        c = int(c)
        for t in range(0, c, BLOCK_SIZE):
            n = min(BLOCK_SIZE, c - t)
            m[block_tables[b, t // BLOCK_SIZE], :n] = True
    return m


def random_pools(rng, num_blocks, n_kv_heads, head_dim, valid):
    """K and V [NB, Hkv, 16, D] f16 (token-major blocks), N(0,1) in valid slots,
    NaN elsewhere.  V is drawn in [NB, Hkv, D, 16] order and transposed (the
    draw order of the first recipe, kept so that seeded values stay the same)."""
    k = rng.standard_normal((num_blocks, n_kv_heads, BLOCK_SIZE, head_dim), dtype=np.float32).astype(F16)
    v = rng.standard_normal((num_blocks, n_kv_heads, head_dim, BLOCK_SIZE), dtype=np.float32).astype(F16)
    v = np.ascontiguousarray(v.transpose(0, 1, 3, 2))
    mask = np.broadcast_to((~valid)[:, None, :, None], k.shape)
    k[mask] = np.nan
    v[mask] = np.nan
    return k, v


def quantize_e4m3(x, amax=None):
    """f32 -> (E4M3 codes uint8, scale) with scale = amax / 448, torch's RNE cast."""
    import torch
    x = np.asarray(x, dtype=np.float32)
    if amax is None:
        finite = x[np.isfinite(x)]
        amax = float(np.abs(finite).max()) if finite.size else 1.0
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = torch.from_numpy(np.nan_to_num(x / scale, nan=0.0)).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[~np.isfinite(x)] = E4M3_NAN
    return codes, float(scale)


@dataclass
class AttnCase:
    q: np.ndarray            # [B, Hq, D] f16
    k_pool: np.ndarray       # [NB, Hkv, 16, D] f16 or uint8
    v_pool: np.ndarray       # [NB, Hkv, 16, D] f16 or uint8
    block_tables: np.ndarray  # [B, stride] int32
    ctx_lens: np.ndarray     # [B] int32
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    num_blocks: int = 0
    max_context: int = 0
    extra: dict = field(default_factory=dict)


def attention_case(batch, n_q_heads, n_kv_heads, head_dim, ctx_lo, ctx_hi, seed,
                   dist="uniform", kv_dtype="f16", ctx_lens=None, max_context=None):
    """One paged-attention input set (q, pools, tables, lengths) as described above."""
    rng = np.random.default_rng(seed)
    if ctx_lens is None:
        ctx_lens = context_lengths(rng, batch, ctx_lo, ctx_hi, dist)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    if max_context is None:
        max_context = max(int(ctx_lens.max()), 1)
    bt, nb = deal_block_tables(rng, ctx_lens, max_context)
    valid = valid_slot_masks(bt, ctx_lens, nb)
    k, v = random_pools(rng, nb, n_kv_heads, head_dim, valid)
    q = rng.standard_normal((batch, n_q_heads, head_dim), dtype=np.float32).astype(F16)
    ks = vs = 1.0
    if kv_dtype == "fp8":
        k, ks = quantize_e4m3(k.astype(np.float32))
        v, vs = quantize_e4m3(v.astype(np.float32))
    return AttnCase(q=q, k_pool=k, v_pool=v, block_tables=bt, ctx_lens=ctx_lens,
                    scale=1.0 / float(np.sqrt(head_dim)), k_scale=ks, v_scale=vs,
                    num_blocks=nb, max_context=max_context)


def workload_case(w: AttnWorkload, seed=None):
    return attention_case(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_lo,
                          w.ctx_hi, w.seed if seed is None else seed, w.dist, w.kv_dtype)


def model_weights(shape: Shape, seed, bias=True, norm_jitter=False, std=0.02, n_layers=None):
    """Random-init f16 weights, [out, in] row-major; QKV rows [q | k | v], gate-up rows [gate | up]."""
    rng = np.random.default_rng(seed)
    n_layers = shape.n_layers if n_layers is None else n_layers
    h, d = shape.hidden, shape.head_dim
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * d

    def mat(*s):
        return (rng.standard_normal(s, dtype=np.float32) * np.float32(std)).astype(F16)

    def gain(n):
        if norm_jitter:
            return (1.0 + 0.1 * rng.standard_normal(n, dtype=np.float32)).astype(F16)
        return np.ones(n, dtype=F16)

    layers = []
    for _ in range(n_layers):
        layers.append({
            "w_in": gain(h),
            "w_qkv": mat(qkv, h),
            "b_qkv": mat(qkv) if bias else None,
            "w_o": mat(h, shape.n_q_heads * d),
            "w_post": gain(h),
            "w_gate_up": mat(2 * shape.ffn, h),
            "w_down": mat(h, shape.ffn),
        })
    return {
        "embed": mat(shape.vocab, h),
        "layers": layers,
        "w_final_norm": gain(h),
        "w_lm_head": mat(shape.vocab, h),
    }


def tiny_layer_case(seed=1001, batch=4, ctx_lo=1, ctx_hi=64, norm_jitter=True, bias=True,
                    shape=TINY, ctx_lens=None):
    """Inputs of one decoder-layer step at a small shape: weights, hidden [B,H]
    ~N(0,1), pools pre-filled for positions < c-1 (the slot at c-1 is left NaN:
    the layer writes it), tables, lengths."""
    rng = np.random.default_rng(seed)
    w = model_weights(shape, seed + 7, bias=bias, norm_jitter=norm_jitter, n_layers=1)
    if ctx_lens is None:
        ctx_lens = context_lengths(rng, batch, ctx_lo, ctx_hi)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    bt, nb = deal_block_tables(rng, ctx_lens)
    prefilled = np.maximum(ctx_lens - 1, 0)
    valid = valid_slot_masks(bt, prefilled, nb)
    k, v = random_pools(rng, nb, shape.n_kv_heads, shape.head_dim, valid)
    hidden = rng.standard_normal((batch, shape.hidden), dtype=np.float32).astype(F16)
    return {"weights": w, "hidden": hidden, "k_pool": k, "v_pool": v,
            "block_tables": bt, "ctx_lens": ctx_lens, "num_blocks": nb}


def prompts(rng, batch, length, vocab):
    return rng.integers(0, vocab, size=(batch, length)).astype(np.int32)


def model_weights_torch(shape: Shape, seed, device="cuda", bias=True, std=0.02, n_layers=None):
    """The same recipe as model_weights (N(0, std) matrices and bias, unit
    RMSNorm gains) drawn with torch's Philox generator on the device, for
    full-size models where host generation would dominate the run time."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n_layers = shape.n_layers if n_layers is None else n_layers
    h, d = shape.hidden, shape.head_dim
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * d

    def mat(*s):
        t = torch.empty(s, dtype=torch.float16, device=device)
        t.normal_(0.0, std, generator=g)
        return t

    def gain(n):
        return torch.ones(n, dtype=torch.float16, device=device)

    layers = []
    for _ in range(n_layers):
        layers.append({
            "w_in": gain(h), "w_qkv": mat(qkv, h), "b_qkv": mat(qkv) if bias else None,
            "w_o": mat(h, shape.n_q_heads * d), "w_post": gain(h),
            "w_gate_up": mat(2 * shape.ffn, h), "w_down": mat(h, shape.ffn),
        })
    return {"embed": mat(shape.vocab, h), "layers": layers, "w_final_norm": gain(h),
            "w_lm_head": mat(shape.vocab, h)}


def random_pools_torch(seed, num_blocks, n_kv_heads, head_dim, valid, device="cuda"):
    """The random_pools recipe (N(0, 1) in valid slots, NaN elsewhere; K and V
    [NB, Hkv, 16, D]) drawn with torch's Philox generator on the device, for
    full-size caches whose host generation would dominate a test.
    valid: bool [num_blocks, 16]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.empty(num_blocks, n_kv_heads, BLOCK_SIZE, head_dim, dtype=torch.float16, device=device)
    v = torch.empty(num_blocks, n_kv_heads, head_dim, BLOCK_SIZE, dtype=torch.float16, device=device)
    k.normal_(generator=g)
    v.normal_(generator=g)
    v = v.transpose(2, 3).contiguous()
    inval = torch.from_numpy(~np.asarray(valid, dtype=bool)).to(device)
    k.masked_fill_(inval[:, None, :, None], float("nan"))
    v.masked_fill_(inval[:, None, :, None], float("nan"))
    return k, v


class SamplingCase:
    def __init__(self, logits, temperature, top_k, top_p, uniform, lens):
        self.logits, self.temperature, self.top_k, self.top_p = logits, temperature, top_k, top_p
        self.uniform, self.lens = uniform, lens


def sampling_case(batch, vocab, seed, masked_rows=True):
    """Logits shaped like a language model's: N(0, 2^2) background plus 20
    peaked tokens (+U(4, 12)); every fourth row bans ~10% of the vocabulary
    with -inf and every eighth holds one NaN.  Per-row parameters cycle through
    temperature {0, 0.3, 0.7, 1, 1.5}, top_k {-1, 1, 5, 50, 1000, 0},
    top_p {1, 0.9, 0.5, 0, 0.99, 0.2}; uniforms U[0, 1); every ninth row is
    inactive (length 0)."""
    rng = np.random.default_rng(seed)
    lg = rng.normal(0.0, 2.0, (batch, vocab))
    for b in range(batch):
        peaks = rng.choice(vocab, size=min(20, vocab), replace=False)
        lg[b, peaks] += rng.uniform(4.0, 12.0, peaks.size)
        if masked_rows and b % 4 == 3:
            banned = rng.random(vocab) < 0.1
            banned[np.argmax(lg[b])] = False
            lg[b, banned] = -np.inf
        if masked_rows and b % 8 == 5:
            lg[b, rng.integers(vocab)] = np.nan
    temps = np.array([0.0, 0.3, 0.7, 1.0, 1.5], np.float32)
    ks = np.array([-1, 1, 5, 50, 1000, 0], np.int32)
    ps = np.array([1.0, 0.9, 0.5, 0.0, 0.99, 0.2], np.float32)
    idx = np.arange(batch)
    lens = np.where(idx % 9 == 8, 0, 1 + idx).astype(np.int32)
    return SamplingCase(lg.astype(F16), temps[idx % 5], ks[(idx // 2) % 6], ps[(idx // 3) % 6],
                        rng.random(batch).astype(np.float32), lens)


def penalty_case(batch, vocab, seed):
    """Per-row token counts (200 random tokens of each row seen 1-5 times,
    every fifth row never seen) and penalty parameters cycling over rows:
    repetition {1, 1.1, 1.3, 0.8}, frequency {0, 0.2, 0.5}, presence
    {0, 0.3, 1, 2.5}; every seventh row neutral (1, 0, 0)."""
    rng = np.random.default_rng(seed)
    counts = np.zeros((batch, vocab), np.int32)
    for b in range(batch):
        if b % 5 == 4:
            continue
        ids = rng.choice(vocab, size=min(200, vocab), replace=False)
        counts[b, ids] = rng.integers(1, 6, size=ids.size)
    idx = np.arange(batch)
    rep = np.array([1.0, 1.1, 1.3, 0.8], np.float32)[idx % 4]
    freq = np.array([0.0, 0.2, 0.5], np.float32)[idx % 3]
    pres = np.array([0.0, 0.3, 1.0, 2.5], np.float32)[(idx // 2) % 4]
    neutral = idx % 7 == 6
    rep[neutral], freq[neutral], pres[neutral] = 1.0, 0.0, 0.0
    return counts, rep, freq, pres
