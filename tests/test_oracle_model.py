"""Pins for the oracle's decoder layer and decode step (oracle/decoder.py).

* incremental paged decode == the oracle's own full-sequence causal forward
  (contiguous K/V, causal mask: a different evaluation order);
* the causal forward == a textbook implementation built from torch.nn.functional
  primitives (rms_norm, linear, scaled_dot_product_attention with GQA, silu) and
  a complex-number RoPE;
* rows are independent (batch composition does not change a row);
* the append writes exactly the slot at pos = ctx - 1 and nothing else;
* greedy argmax takes the lowest index on ties;
* the (x, residual) form of the layer: with W_o = 0 its residual is exactly
  the f16 sum r + x, with W_d = 0 its x' is exactly zero and its residual the
  plain layer's output on h = f16(r + x), and in general f16(r' + x') is the
  plain layer's output up to the one extra rounding of x';
* prefill of several prompts at once == the textbook causal forward of each
  prompt (last logits and every cached K and V), and prefill in two chunks ==
  prefill in one == token-by-token decode.
The end-to-end logits of a random-weight model are otherwise parity unpinned
(the pages print no logits or tokens).
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import ModelConfig, decode_step, causal_forward, decode_layer, decode_layer_xr, embed_rows, greedy_argmax, prefill
import pkv_inputs as inp

SHAPE = inp.Shape(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=160, vocab=300, n_layers=2)
CFG = ModelConfig(SHAPE.hidden, SHAPE.n_q_heads, SHAPE.n_kv_heads, SHAPE.head_dim, SHAPE.ffn,
                  SHAPE.vocab, SHAPE.n_layers)
BS = 16


def _weights(seed=21, std=0.08):
    return inp.model_weights(SHAPE, seed, bias=True, norm_jitter=True, std=std)


def _run_incremental(w, tokens_bt, rng, extra_blocks=3):
    """Decode all positions of every row one token at a time; returns logits [B, T, V]."""
    b_n, t_n = tokens_bt.shape
    need = (t_n + BS - 1) // BS
    nb = b_n * need + extra_blocks
    perm = rng.permutation(nb)
    bt = perm[: b_n * need].reshape(b_n, need).astype(np.int32)
    kp = [np.full((nb, CFG.n_kv_heads, BS, CFG.head_dim), np.nan, np.float16) for _ in range(CFG.n_layers)]
    vp = [np.full((nb, CFG.n_kv_heads, BS, CFG.head_dim), np.nan, np.float16) for _ in range(CFG.n_layers)]
    out = []
    for t in range(t_n):
        lens = np.full(b_n, t + 1, np.int32)
        lg, _ = decode_step(CFG, w, kp, vp, tokens_bt[:, t], bt, lens)
        out.append(lg)
    return np.stack(out, axis=1), kp, vp, bt


def test_incremental_decode_equals_causal_forward():
    w = _weights()
    rng = np.random.default_rng(22)
    toks = rng.integers(0, SHAPE.vocab, size=(1, 37)).astype(np.int32)
    inc, kp, vp, bt = _run_incremental(w, toks, rng)
    full, ks, vs = causal_forward(CFG, w, toks[0])
    np.testing.assert_allclose(inc[0].astype(np.float64), full.astype(np.float64), atol=4e-3, rtol=4e-3)
    # cached K of layer 1 equals the contiguous K of the full forward
    t = np.arange(37)
    kc = kp[1][bt[0][t // BS], :, t % BS, :]
    np.testing.assert_allclose(kc.astype(np.float64), ks[1].astype(np.float64), atol=2e-3, rtol=2e-3)


def _rope_c(x, pos, theta):
    d = x.shape[-1]
    z = torch.complex(x[..., : d // 2], x[..., d // 2:])
    freq = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None].to(torch.float64) * freq[None]
    z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_textbook(w, tokens):
    """Llama/Qwen2 pre-norm decoder from torch.nn.functional, fp64, f16 at the same
    storage points as the oracle (hidden after each add, q/k/v, attention output, logits)."""
    f16 = lambda x: x.to(torch.float16).to(torch.float64)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    hq, hkv, d = CFG.n_q_heads, CFG.n_kv_heads, CFG.head_dim
    tok = torch.from_numpy(tokens.astype(np.int64))
    pos = torch.arange(len(tokens))
    h = T(w["embed"])[tok]
    for lw in w["layers"]:
        a = F.rms_norm(h, (CFG.hidden,), T(lw["w_in"]), eps=CFG.rms_eps)
        qkv = F.linear(a, T(lw["w_qkv"]), T(lw["b_qkv"]))
        q = f16(_rope_c(qkv[:, : hq * d].view(-1, hq, d), pos, CFG.rope_theta))
        k = f16(_rope_c(qkv[:, hq * d:(hq + hkv) * d].view(-1, hkv, d), pos, CFG.rope_theta))
        v = f16(qkv[:, (hq + hkv) * d:].view(-1, hkv, d))
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None].contiguous(),
                                           v.transpose(0, 1)[None].contiguous(), is_causal=True, enable_gqa=True)
        o = f16(o[0].transpose(0, 1).reshape(len(tokens), hq * d))
        h = f16(h + F.linear(o, T(lw["w_o"])))
        m = F.rms_norm(h, (CFG.hidden,), T(lw["w_post"]), eps=CFG.rms_eps)
        gu = F.linear(m, T(lw["w_gate_up"]))
        act = F.silu(gu[:, : CFG.ffn]) * gu[:, CFG.ffn:]
        h = f16(h + F.linear(act, T(lw["w_down"])))
    n = F.rms_norm(h, (CFG.hidden,), T(w["w_final_norm"]), eps=CFG.rms_eps)
    return f16(F.linear(n, T(w["w_lm_head"]))).numpy()


def test_causal_forward_vs_torch_textbook():
    w = _weights(31)
    toks = np.random.default_rng(32).integers(0, SHAPE.vocab, size=29).astype(np.int32)
    full, _, _ = causal_forward(CFG, w, toks)
    ref = _torch_textbook(w, toks)
    # a one-ulp f16 flip of a cached K/V element (different summation order in
    # fp64) reaches every later position through attention, so compare within a
    # few f16 ulps rather than bit for bit; a wrong term moves logits by ~0.1-1.
    np.testing.assert_allclose(full.astype(np.float64), ref, atol=4e-3, rtol=4e-3)
    assert np.array_equal(full[:8].astype(np.float64), ref[:8])


def test_rows_are_independent():
    w = _weights(41)
    rng = np.random.default_rng(42)
    toks = rng.integers(0, SHAPE.vocab, size=(3, 18)).astype(np.int32)
    both, *_ = _run_incremental(w, toks, np.random.default_rng(1))
    for b in range(3):
        one, *_ = _run_incremental(w, toks[b:b + 1], np.random.default_rng(2 + b))
        np.testing.assert_allclose(both[b].astype(np.float64), one[0].astype(np.float64), atol=2e-3, rtol=2e-3)


def test_layer_append_touches_only_its_slot():
    case = inp.tiny_layer_case(seed=51, shape=inp.Shape(128, 4, 2, 32, 96, 64, 1))
    cfg = ModelConfig(128, 4, 2, 32, 96, 64, 1)
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    h = decode_layer(cfg, case["weights"]["layers"][0], case["hidden"], kp, vp,
                     case["block_tables"], case["ctx_lens"])
    assert h.dtype == np.float16 and np.all(np.isfinite(h))
    changed_k = ~((kp == case["k_pool"]) | (np.isnan(kp) & np.isnan(case["k_pool"])))
    expect = np.zeros_like(changed_k)
    for b, c in enumerate(case["ctx_lens"]):
        if c > 0:
            expect[case["block_tables"][b][(c - 1) // BS], :, (c - 1) % BS, :] = True
    assert np.array_equal(changed_k, expect)
    assert not np.any(np.isnan(kp[expect]))


def test_embed_rows_out_of_range_ids_are_zero_rows():
    """Reading R25 by hand: ids outside [0, V) embed as zero rows."""
    table = np.arange(12, dtype=np.float16).reshape(4, 3)  # V = 4, H = 3
    got = embed_rows(table, [-1, 0, 4, 2, 3, -7])
    want = np.array([[0, 0, 0], [0, 1, 2], [0, 0, 0], [6, 7, 8], [9, 10, 11], [0, 0, 0]], np.float16)
    assert got.dtype == np.float16 and np.array_equal(got, want)


def test_argmax_lowest_index_on_ties():
    lg = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-5, -4, -4.5, -4]], np.float16)
    assert greedy_argmax(lg).tolist() == [1, 0, 1]


def _empty_pools(nb):
    kp = [np.full((nb, CFG.n_kv_heads, BS, CFG.head_dim), np.nan, np.float16) for _ in range(CFG.n_layers)]
    vp = [np.full((nb, CFG.n_kv_heads, BS, CFG.head_dim), np.nan, np.float16) for _ in range(CFG.n_layers)]
    return kp, vp


def test_prefill_equals_causal_forward():
    """Three prompts of different lengths in one prefill from an empty cache:
    each sequence's last logits and every cached K and V equal the textbook
    causal forward of that prompt alone."""
    w = _weights(61)
    rng = np.random.default_rng(62)
    lens = [23, 1, 37]
    prompts = [rng.integers(0, SHAPE.vocab, size=n).astype(np.int32) for n in lens]
    need = [(n + BS - 1) // BS for n in lens]
    nb = sum(need) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((3, max(need)), -1, np.int32)
    off = 0
    for s, k in enumerate(need):
        bt[s, :k] = perm[off:off + k]
        off += k
    kp, vp = _empty_pools(nb)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    logits, h = prefill(CFG, w, kp, vp, np.concatenate(prompts), starts, [0, 0, 0], bt)
    assert logits.shape == (3, SHAPE.vocab) and h.shape == (sum(lens), SHAPE.hidden)
    for s, toks in enumerate(prompts):
        full, ks, vs = causal_forward(CFG, w, toks)
        np.testing.assert_allclose(logits[s].astype(np.float64), full[-1].astype(np.float64),
                                   atol=4e-3, rtol=4e-3)
        t = np.arange(lens[s])
        for li in range(CFG.n_layers):
            np.testing.assert_allclose(kp[li][bt[s][t // BS], :, t % BS, :].astype(np.float64),
                                       ks[li].astype(np.float64), atol=2e-3, rtol=2e-3)
            np.testing.assert_allclose(vp[li][bt[s][t // BS], :, t % BS, :].astype(np.float64),
                                       vs[li].astype(np.float64), atol=2e-3, rtol=2e-3)


def test_prefill_in_chunks_equals_one_chunk_and_decode():
    """The same prompts prefilled whole, in two chunks (the second continuing
    from a cached prefix), and token by token through the decode step give the
    same last logits and the same cache."""
    w = _weights(63)
    rng = np.random.default_rng(64)
    toks = rng.integers(0, SHAPE.vocab, size=(2, 29)).astype(np.int32)
    nb = 2 * 2 + 1
    bt = rng.permutation(nb)[:4].reshape(2, 2).astype(np.int32)
    kp1, vp1 = _empty_pools(nb)
    whole, _ = prefill(CFG, w, kp1, vp1, toks.reshape(-1), [0, 29, 58], [0, 0], bt)
    kp2, vp2 = _empty_pools(nb)
    cut = [11, 20]
    first = np.concatenate([toks[0, :cut[0]], toks[1, :cut[1]]])
    prefill(CFG, w, kp2, vp2, first, [0, cut[0], cut[0] + cut[1]], [0, 0], bt)
    rest = np.concatenate([toks[0, cut[0]:], toks[1, cut[1]:]])
    second, _ = prefill(CFG, w, kp2, vp2, rest, [0, 29 - cut[0], 58 - cut[0] - cut[1]], cut, bt)
    np.testing.assert_allclose(second.astype(np.float64), whole.astype(np.float64), atol=2e-3, rtol=2e-3)
    inc, kp3, vp3, bt3 = _run_incremental(w, toks, np.random.default_rng(65))
    np.testing.assert_allclose(inc[:, -1].astype(np.float64), whole.astype(np.float64), atol=4e-3, rtol=4e-3)
    t = np.arange(29)
    for li in range(CFG.n_layers):
        for b in range(2):
            a = kp1[li][bt[b][t // BS], :, t % BS, :].astype(np.float64)
            np.testing.assert_allclose(kp2[li][bt[b][t // BS], :, t % BS, :].astype(np.float64), a,
                                       atol=2e-3, rtol=2e-3)
            np.testing.assert_allclose(kp3[li][bt3[b][t // BS], :, t % BS, :].astype(np.float64), a,
                                       atol=2e-3, rtol=2e-3)


def test_layer_xr_form_pins():
    shape = inp.Shape(128, 4, 2, 32, 96, 64, 1)
    cfg = ModelConfig(128, 4, 2, 32, 96, 64, 1)
    case = inp.tiny_layer_case(seed=57, batch=5, ctx_lo=1, ctx_hi=40, shape=shape)
    rng = np.random.default_rng(58)
    x = (rng.standard_normal(case["hidden"].shape) * 0.5).astype(np.float16)
    r = case["hidden"]
    h = (r.astype(np.float64) + x.astype(np.float64)).astype(np.float16)
    lw = case["weights"]["layers"][0]

    def run(lw, form):
        kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
        if form == "xr":
            return decode_layer_xr(cfg, lw, x, r, kp, vp, case["block_tables"], case["ctx_lens"]), kp
        return decode_layer(cfg, lw, h, kp, vp, case["block_tables"], case["ctx_lens"]), kp

    # W_o = 0: the attention sub-block adds nothing, r' is the input sum itself
    (x1, r1), _ = run(dict(lw, w_o=np.zeros_like(lw["w_o"])), "xr")
    assert np.array_equal(r1.view(np.uint16), h.view(np.uint16))
    # W_d = 0: x' is zero and r' is the plain layer's output on h
    lw0 = dict(lw, w_down=np.zeros_like(lw["w_down"]))
    (x2, r2), k_xr = run(lw0, "xr")
    h2, k_plain = run(lw0, "plain")
    assert not np.any(x2.astype(np.float32)) and np.array_equal(r2.view(np.uint16), h2.view(np.uint16))
    assert np.array_equal(np.nan_to_num(k_xr), np.nan_to_num(k_plain))
    # in general: r' + x' (one more f16 rounding of x') is the plain layer's output
    (x3, r3), _ = run(lw, "xr")
    h3, _ = run(lw, "plain")
    s = (r3.astype(np.float64) + x3.astype(np.float64)).astype(np.float16)
    # f16(x') is off by half an ulp of x', and each final rounding by half an
    # ulp of the sum (x' can be larger than the sum when r' and x' cancel)
    ulp = lambda a: np.spacing(np.abs(a).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(s.astype(np.float64) - h3.astype(np.float64)) <= ulp(h3) + 0.5 * ulp(x3) + 1e-7)
    assert np.any(x3.astype(np.float32))

