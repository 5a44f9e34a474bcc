"""GPU parity of the batched, chunked prefill (through the C ABI) against the
oracle's prefill: the logits of each sequence's last new token, the K and V
appended for every new token (parity bar) and every other cache byte
untouched (bit-exact).  Cached prefixes (prior_lens > 0) hold N(0, 1) values;
unwritten slots hold NaN, so a read outside a token's causal range poisons its
output."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import (ATOL, RTOL, dev, assert_parity, weights_to_device, oracle_config, k_to_lib, k_from_lib,
                      v_to_lib, v_from_lib)
from test_gpu_model import MID

pytestmark = pytest.mark.gpu
BS = 16


def prefill_case(shape, new_lens, prior_lens, seed, spare_blocks=3):
    rng = np.random.default_rng(seed)
    w = inp.model_weights(shape, seed, bias=True, norm_jitter=True)
    totals = [p + n for p, n in zip(prior_lens, new_lens)]
    need = [(t + BS - 1) // BS for t in totals]
    nb = sum(need) + spare_blocks
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(new_lens), max(need)), -1, np.int32)
    off = 0
    for s, k in enumerate(need):
        bt[s, :k] = perm[off:off + k]
        off += k
    kp, vp = [], []
    for _ in range(shape.n_layers):
        k = np.full((nb, shape.n_kv_heads, BS, shape.head_dim), np.nan, np.float16)
        v = np.full((nb, shape.n_kv_heads, BS, shape.head_dim), np.nan, np.float16)
        for s, p in enumerate(prior_lens):
            t = np.arange(p)
            k[bt[s][t // BS], :, t % BS, :] = rng.standard_normal((p, shape.n_kv_heads, shape.head_dim))
            v[bt[s][t // BS], :, t % BS, :] = rng.standard_normal((p, shape.n_kv_heads, shape.head_dim))
        kp.append(k)
        vp.append(v)
    tokens = rng.integers(0, shape.vocab, size=sum(new_lens)).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    return dict(weights=w, k=kp, v=vp, bt=bt, tokens=tokens, starts=starts,
                prior=np.asarray(prior_lens, np.int32), nb=nb, max_context=max(totals))


def run_prefill_gpu(pkv, shape, case, max_context=None, model=None, weights=None):
    model = model or pkv.Model(shape, weights or weights_to_device(case["weights"]), max_positions=4096)
    if "k_scales" in case:
        cache = pkv.KVCache(shape.n_layers, case["nb"], shape.n_kv_heads, shape.head_dim, dtype=pkv.KV_FP8_E4M3,
                            k_scales=case["k_scales"], v_scales=case["v_scales"])
    else:
        cache = pkv.KVCache(shape.n_layers, case["nb"], shape.n_kv_heads, shape.head_dim)
    for li in range(shape.n_layers):
        k, v = cache.layer(li)
        k.copy_(torch.from_numpy(k_to_lib(case["k"][li])))
        v.copy_(torch.from_numpy(v_to_lib(case["v"][li])))
    mc = max_context or case["max_context"]
    bt = case["bt"]
    if bt.shape[1] * BS < mc:
        bt = np.concatenate([bt, np.full((bt.shape[0], (mc + BS - 1) // BS - bt.shape[1]), -1, np.int32)], axis=1)
    n_seq = len(case["prior"])
    logits = torch.empty(n_seq, shape.vocab, dtype=torch.float16, device="cuda")
    ws = torch.empty(pkv.prefill_workspace_bytes(model, cache, len(case["tokens"]), n_seq, mc),
                     dtype=torch.uint8, device="cuda")
    pkv.prefill(model, cache, dev(case["tokens"]), dev(case["starts"]), dev(case["prior"]), dev(bt), mc, logits, ws)
    torch.cuda.synchronize()
    ks = [k_from_lib(cache.layer(li)[0].cpu().numpy()) for li in range(shape.n_layers)]
    vs = [v_from_lib(cache.layer(li)[1].cpu().numpy()) for li in range(shape.n_layers)]
    return logits.cpu().numpy(), ks, vs


def run_prefill_oracle(shape, case):
    kp = [k.copy() for k in case["k"]]
    vp = [v.copy() for v in case["v"]]
    logits, _ = oracle.prefill(oracle_config(shape), case["weights"], kp, vp, case["tokens"], case["starts"],
                               case["prior"], case["bt"], k_scales=case.get("k_scales"),
                               v_scales=case.get("v_scales"))
    return logits, kp, vp


def check_cache(case, shape, gk, gv, rk, rv, seqs=None):
    """Appended slots within the bar; every other byte as it was."""
    n_seq = len(case["prior"])
    for li in range(shape.n_layers):
        written = np.zeros(gk[li].shape, bool)
        for s in (range(n_seq) if seqs is None else seqs):
            t = np.arange(case["prior"][s], case["prior"][s] + case["starts"][s + 1] - case["starts"][s])
            written[case["bt"][s][t // BS], :, t % BS, :] = True
        if seqs is None:
            keep = ~written
            assert np.array_equal(gk[li][keep].view(np.uint16), case["k"][li][keep].view(np.uint16))
            assert np.array_equal(gv[li][keep].view(np.uint16), case["v"][li][keep].view(np.uint16))
        assert_parity(gk[li][written], rk[li][written], f"layer {li} appended K")
        assert_parity(gv[li][written], rv[li][written], f"layer {li} appended V")


@pytest.mark.parametrize("shape,new_lens,prior_lens,seed", [
    (MID, [1, 17, 40, 5], [0, 0, 0, 0], 5001),        # whole prompts, 63 tokens: MFMA projections
    (MID, [3, 9], [0, 0], 5002),                      # 12 tokens: GEMV projections
    (MID, [20, 33, 1], [30, 0, 100], 5003),           # chunks continuing cached prefixes
    (inp.TINY, [64, 7, 16], [0, 3, 16], 5004),        # D = 64; block-aligned starts and ends
])
def test_prefill_parity(lib, shape, new_lens, prior_lens, seed):
    case = prefill_case(shape, new_lens, prior_lens, seed)
    g_logits, gk, gv = run_prefill_gpu(lib, shape, case)
    r_logits, rk, rv = run_prefill_oracle(shape, case)
    assert_parity(g_logits, r_logits, "last-token logits")
    check_cache(case, shape, gk, gv, rk, rv)


def test_prefill_two_chunks_equal_one(lib):
    """A prompt prefilled in two GPU calls (the second continuing from what the
    first cached) matches the oracle's one-call prefill."""
    shape = MID
    case = prefill_case(shape, [45, 26], [0, 0], 5005)
    r_logits, rk, rv = run_prefill_oracle(shape, case)
    model = lib.Model(shape, weights_to_device(case["weights"]), max_positions=4096)
    cut = np.array([13, 26], np.int32)               # the second sequence ends with the first chunk
    first = dict(case, tokens=np.concatenate([case["tokens"][:13], case["tokens"][45:71]]),
                 starts=np.array([0, 13, 39], np.int32))
    _, k1, v1 = run_prefill_gpu(lib, shape, first, max_context=case["max_context"], model=model)
    second = dict(case, k=k1, v=v1, tokens=case["tokens"][13:45], starts=np.array([0, 32], np.int32),
                  prior=cut[:1], bt=case["bt"][:1])
    g_logits, gk, gv = run_prefill_gpu(lib, shape, second, max_context=case["max_context"], model=model)
    assert_parity(g_logits[0], r_logits[0], "chunked last-token logits")
    check_cache(case, shape, gk, gv, rk, rv, seqs=[0, 1])


def test_prefill_host_errors(lib):
    shape = MID
    case = prefill_case(shape, [4], [0], 5006)
    model = lib.Model(shape, weights_to_device(case["weights"]), max_positions=4096)
    cache = lib.KVCache(shape.n_layers, case["nb"], shape.n_kv_heads, shape.head_dim)
    logits = torch.empty(1, shape.vocab, dtype=torch.float16, device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    args = (dev(case["tokens"]), dev(case["starts"]), dev(case["prior"]))
    with pytest.raises(lib.PkvError, match="workspace too small"):
        lib.prefill(model, cache, *args, dev(case["bt"]), 4, logits, small)
    with pytest.raises(lib.PkvError, match="bt_stride"):
        lib.prefill(model, cache, *args, dev(case["bt"]), 400, logits, small)
    with pytest.raises(ValueError):
        lib.prefill(model, cache, args[0], args[1][:1], args[2], dev(case["bt"]), 4, logits, small)


def test_prefill_workspace_bytes_long_prompt(lib):
    """The prefill workspace holds no decode-attention partials: for one
    32768-token prompt at the 7B layer shape it stays within the per-token
    buffers (hidden, q, o, FFN activation, block-table copies: ~2.3 GB), where
    sizing the decode partials for 32768 rows needed ~30 GB more."""
    shape = inp.QWEN7
    one = torch.zeros(16, dtype=torch.float16, device="cuda")   # never read: only sizes are asked for
    lw = {k: one for k in ("w_in", "w_qkv", "b_qkv", "w_o", "w_post", "w_gate_up", "w_down")}
    w = {"embed": one, "w_final_norm": one, "w_lm_head": one, "layers": [lw]}
    model = lib.Model(inp.Shape(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                                shape.vocab, 1), w, max_positions=32768)
    cache = lib.KVCache(1, 16, shape.n_kv_heads, shape.head_dim)
    n = lib.prefill_workspace_bytes(model, cache, 32768, 1, 32768)
    per_token = 2 * (shape.hidden + 2 * shape.n_q_heads * shape.head_dim + shape.ffn) + 4 * (1 + 32768 // 16)
    assert 32768 * per_token <= n < 32768 * per_token + (1 << 30), n


def test_prefill_full_shape_sampled_sequences(lib):
    """Qwen2.5-1.5B layer shape (one layer, a 16-token vocabulary: the layer
    does not depend on it), 256 prompts of 128 tokens in one call (32768 new
    tokens, the bench's prompt fill); four sampled sequences (prefill keeps
    sequences independent) against the oracle, logits and appended K / V."""
    from test_gpu_fullsize import _layer_shape
    shape = _layer_shape(inp.QWEN15)
    case = prefill_case(shape, [128] * 256, [0] * 256, 5007)
    g_logits, gk, gv = run_prefill_gpu(lib, shape, case)
    seqs = np.random.default_rng(5008).choice(256, size=4, replace=False)
    sub = dict(case, tokens=np.concatenate([case["tokens"][128 * s:128 * (s + 1)] for s in seqs]),
               starts=np.arange(0, 129 * 4, 128)[:5].astype(np.int32), prior=case["prior"][seqs],
               bt=case["bt"][seqs])
    r_logits, rk, rv = run_prefill_oracle(shape, sub)
    assert_parity(g_logits[seqs], r_logits, "full-shape last-token logits")
    check_cache(sub, shape, gk, gv, rk, rv, seqs=range(4))


def test_prefill_fp8_cache(lib):
    """One layer over an E4M3 cache (cached prefixes quantised with scale
    amax/448, NaN slots as the NaN code): logits within 3x the parity bar,
    appended codes within the bar plus one code step, every other byte
    identical (the quantiser itself is pinned bit-exact by the append tests)."""
    shape = inp.Shape(MID.hidden, MID.n_q_heads, MID.n_kv_heads, MID.head_dim, MID.ffn, MID.vocab, 1)
    case = prefill_case(shape, [20, 33, 1], [30, 0, 100], 5009)
    kq, ks = inp.quantize_e4m3(case["k"][0].astype(np.float32))
    vq, vs = inp.quantize_e4m3(case["v"][0].astype(np.float32))
    case = dict(case, k=[kq], v=[vq], k_scales=[ks], v_scales=[vs])
    g_logits, gk, gv = run_prefill_gpu(lib, shape, case)
    r_logits, rk, rv = run_prefill_oracle(shape, case)
    assert_parity(g_logits, r_logits, "fp8-cache last-token logits", atol=3 * ATOL, rtol=3 * RTOL)
    written = np.zeros(kq.shape, bool)
    for s_ in range(3):
        t = np.arange(case["prior"][s_], case["prior"][s_] + case["starts"][s_ + 1] - case["starts"][s_])
        written[case["bt"][s_][t // BS], :, t % BS, :] = True
    for got, ref, orig, sc, m in ((gk[0], rk[0], kq, ks, written), (gv[0], rv[0], vq, vs, written)):
        assert np.array_equal(got[~m], orig[~m])
        dg = oracle.e4m3_decode(got[m]) * sc
        dr = oracle.e4m3_decode(ref[m]) * sc
        assert np.all(np.abs(dg - dr) <= ATOL + RTOL * np.abs(dr) + np.abs(dr) / 8 + sc * 2.0 ** -9)


@pytest.mark.parametrize("shape,new_lens,prior_lens,seed", [
    # 7B head grouping (G = 7: chunks of 16 query rows straddle tokens unevenly)
    (inp.Shape(512, 14, 2, 128, 1024, 500, 1), [37, 5, 64], [0, 21, 90], 5010),
    # MHA (G = 1: 16 tokens of one head per chunk)
    (inp.Shape(512, 4, 4, 128, 1024, 500, 1), [50, 3], [16, 7], 5011),
    # long prompts: up to 63 pages per chunk, many rescaled page groups
    (inp.Shape(512, 12, 2, 128, 1024, 500, 1), [700, 260], [300, 0], 5012),
    # 1100 new tokens with FFN 16040: the gate/up projection on 256 x 256 tiles,
    # partial in both the last row tile and the last column tile
    (inp.Shape(256, 4, 2, 64, 16040, 500, 1), [600, 500], [0, 40], 5013),
])
def test_prefill_group_sizes_and_long_prompts(lib, shape, new_lens, prior_lens, seed):
    case = prefill_case(shape, new_lens, prior_lens, seed)
    g_logits, gk, gv = run_prefill_gpu(lib, shape, case)
    r_logits, rk, rv = run_prefill_oracle(shape, case)
    assert_parity(g_logits, r_logits, "last-token logits")
    check_cache(case, shape, gk, gv, rk, rv)
