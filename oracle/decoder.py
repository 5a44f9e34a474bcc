"""The decode step of a Llama/Qwen2-style decoder over a paged KV cache, written
as its plain definition (test infrastructure only; see the package docstring).

What the pages fix, and the readings taken where they are silent:

* The per-layer structure is named by the rvLLM post (discuss.pytorch.kr),
  section "퓨즈드 CUDA 커널": Add+RMSNorm+QKV, Add+RMSNorm+GateUp and
  SiLU*Mul+Down.  Reading: the pre-norm decoder layer of the Llama/Qwen2
  families listed in the post's supported-architecture table,
      a  = RMSNorm(h) * w_in
      q, k, v = split(W_qkv a + b_qkv)      (bias optional: Qwen2 has one)
      q, k = RoPE(q, pos), RoPE(k, pos)     (rotate-half form, theta from the model)
      append k, v at position pos; o = softmax(q K^T / sqrt(D)) V per query head
      h1 = h + W_o o
      m  = RMSNorm(h1) * w_post
      g, u = split(W_gu m)                  (rows: gate first, then up)
      h2 = h1 + W_down (silu(g) * u)
  The "Add" in the fused names is the residual add, folded here into a single
  hidden state h that is stored in f16 between layers.
* The KV cache is paged with a per-sequence block table (section
  "PagedAttention과 FlashAttention-3" of the same post; aitrends.kr glossary
  entry on PagedAttention: fixed-size pages).  Layout (the plain one; block
  size BS = 16):
      K pool of a layer: [num_blocks, Hkv, BS, D]  (token-major inside a block)
      V pool of a layer: [num_blocks, Hkv, BS, D]  (the same)
  Token t of sequence b lives in physical block block_table[b][t // BS], slot
  t % BS.
* GQA: query head h reads KV head h // (Hq / Hkv) (contiguous groups), which is
  what lets a kernel read each KV head once per group (same section).
* context_lens[b] counts the cached tokens including the one being decoded, so
  the new token sits at pos = context_lens[b] - 1 and attention covers
  positions [0, context_lens[b]).  A row with context length 0 is inactive: no
  append, attention output 0.
* Block tables and context lengths are the per-step metadata named in section
  "CUDA 그래프 리플레이"; sampling is outside the forward, and the benchmark
  decodes greedily (H100 section: greedy decoding) -> greedy_argmax.
* Rounding points (reading of "pure f16 end to end" in the post's
  introduction, with fp32 or wider accumulation): the hidden state after every
  residual add, q and k after RoPE, v, the attention output and the logits are
  rounded to f16 (round to nearest even); everything else stays in ``acc``.
"""
from dataclasses import dataclass

import numpy as np

from .fp8 import e4m3_decode, e4m3_quantize

F16 = np.float16


@dataclass(frozen=True)
class ModelConfig:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    block_size: int = 16

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


# ---------------------------------------------------------------- elementwise

def rmsnorm(x, w, eps, acc=np.float64):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=acc)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + acc(eps)) * np.asarray(w, dtype=acc)


def silu(x, acc=np.float64):
    """SiLU (swish): x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=acc)
    return x / (acc(1) + np.exp(-x))


def rope_angles(pos, head_dim, theta):
    """Rotation angles pos * theta^(-2i/D), i < D/2, in float64.

    pos may be a scalar or an array; the result has a trailing axis of D/2.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, theta, acc=np.float64):
    """Rotary embedding in rotate-half form on the last axis (length D).

    With x1 = x[..., :D/2], x2 = x[..., D/2:] and angle a_i:
        out[..., i]       = x1_i cos a_i - x2_i sin a_i
        out[..., i + D/2] = x2_i cos a_i + x1_i sin a_i
    ``pos`` broadcasts against x's leading axes (one position per row).
    """
    x = np.asarray(x, dtype=acc)
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)
    # one position per leading row: insert axes so ang broadcasts over heads
    while ang.ndim < x.ndim:
        ang = ang[..., None, :]
    c = np.cos(ang).astype(acc)
    s = np.sin(ang).astype(acc)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------- paged KV

def _kv_values(pool, scale, acc):
    """Pool contents as real numbers: f16 as is, uint8 as E4M3 codes * scale."""
    if pool.dtype == np.uint8:
        return e4m3_decode(pool, acc) * acc(scale)
    return pool.astype(acc)


def gather_sequence(k_pool, v_pool, block_row, ctx_len, block_size):
    """Token-by-token gather of one sequence's K and V through its block table.

    Returns K [c, Hkv, D] and V [c, Hkv, D] in the pools' storage dtype.
    """
    t = np.arange(ctx_len)
    blocks = np.asarray(block_row)[t // block_size]
    slots = t % block_size
    k = k_pool[blocks, :, slots, :]          # [c, Hkv, D]
    v = v_pool[blocks, :, slots, :]          # [c, Hkv, D]
    return k, v


def paged_attention(q, k_pool, v_pool, block_row, ctx_len, scale, *,
                    k_scale=1.0, v_scale=1.0, acc=np.float64, return_weights=False):
    """Decode attention of one sequence over its paged KV.

    q: [Hq, D]; pools in the layout of the module docstring (f16, or uint8 E4M3
    codes with per-tensor scales k_scale / v_scale).  For query head h
    (KV head g = h // G):
        s_t = scale * <q_h, K_{t,g}>,  t < ctx_len
        p   = softmax(s)
        o_h = sum_t p_t V_{t,g}
    Returns o [Hq, D] in ``acc`` (and lse [Hq], p [Hq, c] when asked).
    A context length of 0 gives o = 0 (inactive row).
    """
    q = np.asarray(q)
    hq, d = q.shape
    hkv = k_pool.shape[1]
    bs = k_pool.shape[2]
    grp = hq // hkv
    if ctx_len == 0:
        o = np.zeros((hq, d), dtype=acc)
        if return_weights:
            return o, np.full(hq, -np.inf, dtype=acc), np.zeros((hq, 0), dtype=acc)
        return o
    kc, vc = gather_sequence(k_pool, v_pool, block_row, ctx_len, bs)
    kr = _kv_values(kc, k_scale, acc)
    vr = _kv_values(vc, v_scale, acc)
    qa = q.astype(acc)
    o = np.empty((hq, d), dtype=acc)
    lse = np.empty(hq, dtype=acc)
    probs = np.empty((hq, ctx_len), dtype=acc)
    for h in range(hq):
        g = h // grp
        s = (kr[:, g, :] @ qa[h]) * acc(scale)           # [c]
        m = np.max(s)
        e = np.exp(s - m)
        z = np.sum(e)
        p = e / z
        o[h] = p @ vr[:, g, :]
        lse[h] = m + np.log(z)
        probs[h] = p
    if return_weights:
        return o, lse, probs
    return o


def paged_attention_batch(q, k_pool, v_pool, block_tables, ctx_lens, scale, *,
                          k_scale=1.0, v_scale=1.0, acc=np.float64):
    """paged_attention for every row b; returns (o [B,Hq,D] f16, lse [B,Hq] acc)."""
    b_n = q.shape[0]
    out = np.zeros(q.shape, dtype=F16)
    lse = np.full(q.shape[:2], -np.inf, dtype=acc)
    for b in range(b_n):
        c = int(ctx_lens[b])
        if c == 0:
            continue
        o, l, _ = paged_attention(q[b], k_pool, v_pool, block_tables[b], c, scale,
                                  k_scale=k_scale, v_scale=v_scale, acc=acc,
                                  return_weights=True)
        out[b] = o.astype(F16)
        lse[b] = l
    return out, lse


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, ctx_lens, k_scale=None, v_scale=None):
    """Store each active row's new K/V (f16 [B, Hkv, D]) at pos = ctx_len - 1.

    E4M3 pools (uint8) store the codes of the f16 values under the layer's
    per-tensor scales (e4m3_quantize: float32 quotient, nearest-even,
    saturating), the reading taken for the quantised cache of the rvLLM post
    (section "PagedAttention과 FlashAttention-3")."""
    bs = k_pool.shape[2]
    if k_pool.dtype == np.uint8:
        k_new = e4m3_quantize(k_new, k_scale)
        v_new = e4m3_quantize(v_new, v_scale)
    for b in range(k_new.shape[0]):
        c = int(ctx_lens[b])
        if c == 0:
            continue
        pos = c - 1
        blk = int(block_tables[b][pos // bs])
        k_pool[blk, :, pos % bs, :] = k_new[b]
        v_pool[blk, :, pos % bs, :] = v_new[b]


# ---------------------------------------------------------------- one layer

def _linear(x, w, acc, bias=None):
    """y = x W^T (+ b) with W stored [out, in]; x [..., in].  W may be given
    as f16 or already widened to ``acc`` (exact: every f16 is an fp32 value);
    a widened W is used without a copy."""
    y = np.asarray(x, dtype=acc) @ np.asarray(w, dtype=acc).T
    if bias is not None:
        y = y + np.asarray(bias, dtype=acc)
    return y


def _layer(cfg, lw, h, k_pool, v_pool, block_tables, ctx_lens, acc, k_scale, v_scale):
    """The layer up to its last product: returns h1 = f16(h + W_o o) (the
    hidden state after the attention sub-block) and W_d (silu(g) * u) in
    `acc` precision, not rounded."""
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    b_n = h.shape[0]
    lens = np.asarray(ctx_lens, dtype=np.int64)
    pos = np.maximum(lens - 1, 0)

    a = rmsnorm(h, lw["w_in"], cfg.rms_eps, acc)
    qkv = _linear(a, lw["w_qkv"], acc, lw.get("b_qkv"))
    q = qkv[:, : hq * d].reshape(b_n, hq, d)
    k = qkv[:, hq * d:(hq + hkv) * d].reshape(b_n, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(b_n, hkv, d)
    q = rope(q, pos, cfg.rope_theta, acc).astype(F16)
    k = rope(k, pos, cfg.rope_theta, acc).astype(F16)
    v = v.astype(F16)
    kv_append(k_pool, v_pool, k, v, block_tables, lens, k_scale, v_scale)

    if k_pool.dtype == np.uint8:
        o, _ = paged_attention_batch(q, k_pool, v_pool, block_tables, lens, 1.0 / np.sqrt(d),
                                     k_scale=k_scale, v_scale=v_scale, acc=acc)
    else:
        o, _ = paged_attention_batch(q, k_pool, v_pool, block_tables, lens, 1.0 / np.sqrt(d), acc=acc)
    h1 = (np.asarray(h, dtype=acc) + _linear(o.reshape(b_n, hq * d), lw["w_o"], acc)).astype(F16)

    m = rmsnorm(h1, lw["w_post"], cfg.rms_eps, acc)
    gu = _linear(m, lw["w_gate_up"], acc)
    act = silu(gu[:, : cfg.ffn], acc) * gu[:, cfg.ffn:]
    return h1, _linear(act, lw["w_down"], acc)


def decode_layer(cfg, lw, h, k_pool, v_pool, block_tables, ctx_lens, acc=np.float64, k_scale=None,
                 v_scale=None):
    """One decoder layer for a batch of single-token rows.

    h: [B, H] f16 hidden state; the pools are this layer's and are updated in
    place by the append (E4M3 pools with this layer's k_scale / v_scale).
    Returns the new hidden state [B, H] f16.
    """
    h1, down = _layer(cfg, lw, h, k_pool, v_pool, block_tables, ctx_lens, acc, k_scale, v_scale)
    return (np.asarray(h1, dtype=acc) + down).astype(F16)


def decode_layer_xr(cfg, lw, x, r, k_pool, v_pool, block_tables, ctx_lens, acc=np.float64, k_scale=None,
                    v_scale=None):
    """The same layer in the (x, residual) form of the fused "Add + RMSNorm"
    kernels (rvLLM post, section "퓨즈드 CUDA 커널": the add joins the previous
    sub-block's output to the residual stream inside the next fused op).

    x: [B, H] f16 output of the previous MLP (the embedding for layer 0), r:
    [B, H] f16 residual stream (zero for layer 0).  The layer adds x to r
    (h = f16(r + x)), runs as decode_layer on h up to the down projection, and
    returns (x', r') = (f16(W_d (silu(g) * u)), h1): the new MLP output, not
    yet added, and the residual stream after the attention sub-block.
    """
    h = (np.asarray(r, dtype=acc) + np.asarray(x, dtype=acc)).astype(F16)
    h1, down = _layer(cfg, lw, h, k_pool, v_pool, block_tables, ctx_lens, acc, k_scale, v_scale)
    return down.astype(F16), h1


def embed_rows(embed, tokens):
    """The embedding rows of the tokens, f16 [B, H] (reading R25): a token id
    outside [0, V), such as the -1 the greedy argmax gives an inactive row,
    embeds as a zero row."""
    e = np.asarray(embed)
    t = np.asarray(tokens, dtype=np.int64)
    ok = (t >= 0) & (t < e.shape[0])
    h = e[np.where(ok, t, 0)].astype(F16)
    h[~ok] = 0
    return h


def decode_step(cfg, weights, k_pools, v_pools, tokens, block_tables, ctx_lens,
                acc=np.float64, k_scales=None, v_scales=None):
    """Embedding -> every layer -> final RMSNorm -> LM head.

    weights: {"embed" [V,H], "layers": [layer dicts], "w_final_norm" [H],
    "w_lm_head" [V,H]} (f16).  k_pools / v_pools: per-layer pools, updated in
    place (E4M3 pools take per-layer k_scales / v_scales).  Returns
    (logits [B, V] f16, final hidden [B, H] f16).
    """
    h = embed_rows(weights["embed"], tokens)
    for li, lw in enumerate(weights["layers"]):
        ks = None if k_scales is None else k_scales[li]
        vs = None if v_scales is None else v_scales[li]
        h = decode_layer(cfg, lw, h, k_pools[li], v_pools[li], block_tables, ctx_lens, acc, ks, vs)
    n = rmsnorm(h, weights["w_final_norm"], cfg.rms_eps, acc)
    logits = _linear(n, weights["w_lm_head"], acc).astype(F16)
    return logits, h


def prefill(cfg, weights, k_pools, v_pools, tokens, seq_starts, prior_lens, block_tables,
            acc=np.float64, k_scales=None, v_scales=None):
    """Batched, chunked prefill over the paged cache.

    Sequence s brings the new tokens tokens[seq_starts[s]:seq_starts[s+1]] at
    positions prior_lens[s], prior_lens[s] + 1, ... (prior_lens[s] tokens are
    already cached).  Reading of the multi-token causal step (the post's
    "PagedAttention과 FlashAttention-3" section names causal multi-token
    attention over the same cache): in every layer the k and v of all new
    tokens are appended first, and new token j of sequence s then attends over
    positions [0, prior_lens[s] + j] of its own sequence.  That is the decode
    layer applied to each new token as a row of its own, with context length
    prior_lens[s] + j + 1 and its sequence's block-table row.  Returns (logits
    [S, V] f16 of each sequence's last new token, hidden [T, H] f16 of every
    new token).  The pools are updated in place.
    """
    starts = np.asarray(seq_starts, dtype=np.int64)
    n_seq = starts.shape[0] - 1
    seq_of = np.repeat(np.arange(n_seq), np.diff(starts))
    j = np.arange(starts[-1]) - starts[seq_of]
    lens = (np.asarray(prior_lens, dtype=np.int64)[seq_of] + j + 1).astype(np.int32)
    rows_bt = np.asarray(block_tables)[seq_of]
    h = embed_rows(weights["embed"], tokens)
    for li, lw in enumerate(weights["layers"]):
        ks = None if k_scales is None else k_scales[li]
        vs = None if v_scales is None else v_scales[li]
        h = decode_layer(cfg, lw, h, k_pools[li], v_pools[li], rows_bt, lens, acc, ks, vs)
    n = rmsnorm(h[starts[1:] - 1], weights["w_final_norm"], cfg.rms_eps, acc)
    logits = _linear(n, weights["w_lm_head"], acc).astype(F16)
    return logits, h


def greedy_argmax(logits):
    """Greedy token per row (reading R10): the lowest index among the largest
    f16 logits, a NaN never winning (so -inf beats NaN); 0 for a row of NaNs
    only."""
    x = np.asarray(logits, dtype=np.float64)
    nan = np.isnan(x)
    xm = np.where(nan, -np.inf, x)
    hit = (xm == xm.max(axis=-1, keepdims=True)) & ~nan
    return np.where(hit.any(axis=-1), np.argmax(hit, axis=-1), 0).astype(np.int32)


# ---------------------------------------------------------------- full sequence

def causal_forward(cfg, weights, tokens, acc=np.float64):
    """Textbook full-sequence forward of one sequence with contiguous K/V and a
    causal mask (no paging, all positions at once).

    Used to pin the incremental paged decode: feeding the same tokens one at a
    time through decode_step must give the same per-position logits.
    Returns (logits [T, V] f16, per-layer K [T, Hkv, D] f16, V [T, Hkv, D] f16).
    """
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    grp = hq // hkv
    tok = np.asarray(tokens, dtype=np.int64)
    t_n = tok.shape[0]
    pos = np.arange(t_n)
    h = embed_rows(weights["embed"], tok)
    ks, vs = [], []
    mask = np.tril(np.ones((t_n, t_n), dtype=bool))
    for lw in weights["layers"]:
        a = rmsnorm(h, lw["w_in"], cfg.rms_eps, acc)
        qkv = _linear(a, lw["w_qkv"], acc, lw.get("b_qkv"))
        q = rope(qkv[:, : hq * d].reshape(t_n, hq, d), pos, cfg.rope_theta, acc).astype(F16)
        k = rope(qkv[:, hq * d:(hq + hkv) * d].reshape(t_n, hkv, d), pos,
                 cfg.rope_theta, acc).astype(F16)
        v = qkv[:, (hq + hkv) * d:].reshape(t_n, hkv, d).astype(F16)
        ks.append(k)
        vs.append(v)
        # repeat each KV head for its group of query heads
        kr = np.repeat(k.astype(acc), grp, axis=1)      # [T, Hq, D]
        vr = np.repeat(v.astype(acc), grp, axis=1)
        s = np.einsum("thd,uhd->htu", q.astype(acc), kr) / np.sqrt(acc(d))
        s = np.where(mask[None], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        o = np.einsum("htu,uhd->thd", p, vr).astype(F16)
        h1 = (h.astype(acc) + _linear(o.reshape(t_n, hq * d), lw["w_o"], acc)).astype(F16)
        m = rmsnorm(h1, lw["w_post"], cfg.rms_eps, acc)
        gu = _linear(m, lw["w_gate_up"], acc)
        act = silu(gu[:, : cfg.ffn], acc) * gu[:, cfg.ffn:]
        h = (h1.astype(acc) + _linear(act, lw["w_down"], acc)).astype(F16)
    n = rmsnorm(h, weights["w_final_norm"], cfg.rms_eps, acc)
    logits = _linear(n, weights["w_lm_head"], acc).astype(F16)
    return logits, ks, vs
