"""GPU parity of the FP8 E4M3 KV cache end to end (through the C ABI) against
the oracle: the quantising append (bit-exact codes), one decoder layer and
greedy decode steps over an fp8 cache (rvLLM post, section
"PagedAttention과 FlashAttention-3": FP8 E4M3 KV; the quantisation rule is the
oracle's e4m3_quantize).

Quantisation turns an ulp of difference before rounding into a whole code
step (up to 1/8 relative) after it.  So the quantiser and the cache indexing
are checked bit-exact on identical inputs; in a model, appended values are
held to the parity bar plus one code step, each decode step is compared over
the same cache history (the oracle continues from the GPU's codes), its
logits are held to three times the f16 bar, and greedy tokens must agree on
>= 99% of rows (ties within the f16 bar accepted)."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import (ATOL, RTOL, assert_parity, dev, k_from_lib, k_to_lib, load_case_into_cache, oracle_config,
                      tie_aware_agree, v_from_lib, v_to_lib, weights_to_device)

pytestmark = pytest.mark.gpu

FP8_ATOL, FP8_RTOL = 3 * ATOL, 3 * RTOL

MID = inp.Shape(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, ffn=1408, vocab=1000, n_layers=2)


def _append(lib, cache, k, v, bt, lens, layer=0):
    lib.kv_append(cache, layer, dev(k), dev(v), dev(bt), dev(lens))
    torch.cuda.synchronize()
    gk, gv = cache.layer(layer)
    return k_from_lib(gk.cpu().numpy()), v_from_lib(gv.cpu().numpy())


def test_kv_append_fp8_bit_exact(lib):
    case = inp.attention_case(9, 4, 2, 128, 1, 200, seed=31, kv_dtype="fp8",
                              ctx_lens=[1, 16, 17, 32, 33, 100, 0, 200, 2])
    cache = load_case_into_cache(lib, case)
    rng = np.random.default_rng(32)
    k = (rng.standard_normal((9, 2, 128)) * 2).astype(np.float16)
    v = (rng.standard_normal((9, 2, 128)) * 2).astype(np.float16)
    k[0, 0, :4] = [1e4, -1e4, 0.0, -0.0]          # saturation and signed zero
    gk, gv = _append(lib, cache, k, v, case.block_tables, case.ctx_lens)
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.kv_append(kp, vp, k, v, case.block_tables, case.ctx_lens, case.k_scale, case.v_scale)
    assert np.array_equal(gk, kp) and np.array_equal(gv, vp)


def test_kv_append_fp8_rounding_edges(lib):
    """Unit scales: every exact midpoint between adjacent codes (ties go to the
    even code), subnormals, the saturation boundary and infinities."""
    t = oracle.e4m3_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float16)
    assert np.array_equal(mids.astype(np.float64), (t[:-1] + t[1:]) / 2)   # exact in f16
    edge = np.array([448, 456, 464, 480, 1e4, np.inf, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6 - 2.0 ** -11],
                    np.float16)
    vals = np.concatenate([mids, -mids, t.astype(np.float16), edge, -edge])
    d = 128
    n_rows = (vals.size + 2 * d - 1) // (2 * d)
    vals = np.concatenate([vals, np.zeros(n_rows * 2 * d - vals.size, np.float16)])
    k = vals.reshape(n_rows, 2, d)
    v = k[::-1].copy()
    lens = np.arange(1, n_rows + 1, dtype=np.int32) * 3
    rng = np.random.default_rng(33)
    bt, nb = inp.deal_block_tables(rng, lens)
    cache = lib.KVCache(1, nb, 2, d, dtype=lib.KV_FP8_E4M3, k_scales=[1.0], v_scales=[1.0])
    gk0, gv0 = cache.layer(0)
    gk0.fill_(0x55)
    gv0.fill_(0x55)
    gk, gv = _append(lib, cache, k, v, bt, lens)
    kp = np.full(gk.shape, 0x55, np.uint8)
    vp = np.full(gv.shape, 0x55, np.uint8)
    oracle.kv_append(kp, vp, k, v, bt, lens, 1.0, 1.0)
    assert np.array_equal(gk, kp) and np.array_equal(gv, vp)


def _fp8_pools(k, v):
    """Quantise a case's f16 pools (NaN slots to the NaN code) with scale amax/448."""
    kq, ks = inp.quantize_e4m3(k.astype(np.float32))
    vq, vs = inp.quantize_e4m3(v.astype(np.float32))
    return kq, vq, ks, vs


@pytest.mark.parametrize("batch,seed,hi", [(3, 1101, 300), (40, 1102, 200)])
def test_decode_layer_fp8(lib, batch, seed, hi):
    case = inp.tiny_layer_case(seed=seed, batch=batch, ctx_lo=1, ctx_hi=hi, shape=MID)
    kq, vq, ks, vs = _fp8_pools(case["k_pool"], case["v_pool"])
    w = weights_to_device(case["weights"])
    model = lib.Model(MID, w, max_positions=4096)
    cache = lib.KVCache(1, case["num_blocks"], MID.n_kv_heads, MID.head_dim, dtype=lib.KV_FP8_E4M3,
                        k_scales=[ks], v_scales=[vs])
    gk, gv = cache.layer(0)
    gk.copy_(torch.from_numpy(k_to_lib(kq)))
    gv.copy_(torch.from_numpy(v_to_lib(vq)))
    mc = int(case["ctx_lens"].max())
    hidden = dev(case["hidden"])
    ws = torch.empty(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    lib.decode_layer(model, cache, 0, hidden, dev(case["block_tables"]), dev(case["ctx_lens"]), mc, ws)
    torch.cuda.synchronize()
    rk, rv = kq.copy(), vq.copy()
    rh = oracle.decode_layer(oracle_config(MID, 1), case["weights"]["layers"][0], case["hidden"], rk, rv,
                             case["block_tables"], case["ctx_lens"], k_scale=ks, v_scale=vs)
    assert_parity(hidden.cpu().numpy(), rh, "hidden after an fp8-cache layer")
    # appended slots: indexing bit-exact (every other byte untouched); values
    # within the parity bar plus one code step.  The f16 k and v entering the
    # quantiser differ between the two sides by the projection's rounding
    # (the kernel applies the norm gain in f16), so near zero a code can sit
    # a few steps away; the quantiser itself is pinned bit-exact above.
    ck, cv = k_from_lib(gk.cpu().numpy()), v_from_lib(gv.cpu().numpy())
    kmask = np.zeros(kq.shape, bool)
    for b, c in enumerate(case["ctx_lens"]):
        if c > 0:
            kmask[case["block_tables"][b][(c - 1) // 16], :, (c - 1) % 16, :] = True
    for got, ref, orig, sc, m in ((ck, rk, kq, ks, kmask), (cv, rv, vq, vs, kmask)):
        assert np.array_equal(got[~m], orig[~m])
        assert (got[m] == ref[m]).mean() > 0.95
        dg = oracle.e4m3_decode(got[m]) * sc
        dr = oracle.e4m3_decode(ref[m]) * sc
        assert np.all(np.abs(dg - dr) <= ATOL + RTOL * np.abs(dr) + np.abs(dr) / 8 + sc * 2.0 ** -9)


def _check_appended(got, ref, orig_mask, sc):
    """Appended slots (mask) within the parity bar plus one code step; every
    other byte identical."""
    assert np.array_equal(got[~orig_mask], ref[~orig_mask])
    dg = oracle.e4m3_decode(got[orig_mask]) * sc
    dr = oracle.e4m3_decode(ref[orig_mask]) * sc
    assert np.all(np.abs(dg - dr) <= ATOL + RTOL * np.abs(dr) + np.abs(dr) / 8 + sc * 2.0 ** -9)


def test_decode_steps_fp8_cache_greedy(lib):
    """Decode steps over an fp8 cache.  After every step the GPU cache is
    compared with the oracle's (untouched bytes identical, appended codes
    within the bar) and the oracle continues from the GPU's codes, so each
    step's logits are compared over the same history and only that step's
    own quantisation can differ."""
    shape, batch, mc, n_layers = MID, 5, 64, MID.n_layers
    w = inp.model_weights(shape, 2101, bias=True, norm_jitter=True, std=0.05)
    model = lib.Model(shape, weights_to_device(w), max_positions=mc)
    stride = (mc + 15) // 16
    nb = batch * stride + 7
    ks, vs = [0.02, 0.03], [0.01, 0.015]
    cache = lib.KVCache(n_layers, nb, shape.n_kv_heads, shape.head_dim, dtype=lib.KV_FP8_E4M3,
                        k_scales=ks, v_scales=vs)
    for layer in range(n_layers):
        for t_ in cache.layer(layer):
            t_.fill_(0x7F)
    rng = np.random.default_rng(2102)
    bt = rng.permutation(nb).astype(np.int32)[: batch * stride].reshape(batch, stride)
    prompts = rng.integers(0, shape.vocab, size=(batch, 16)).astype(np.int32)
    lens = np.zeros(batch, np.int32)
    ws = torch.empty(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device="cuda")
    kp = [np.full((nb, shape.n_kv_heads, 16, shape.head_dim), 0x7F, np.uint8) for _ in range(n_layers)]
    vp = [np.full((nb, shape.n_kv_heads, 16, shape.head_dim), 0x7F, np.uint8) for _ in range(n_layers)]
    cfg = oracle_config(shape)
    agree = total = 0
    worst = 0.0
    tok = prompts[:, 0]
    for t in range(24):
        lens += 1
        lib.decode_step(model, cache, dev(tok), dev(bt), dev(lens), mc, logits, ws)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        rl, _ = oracle.decode_step(cfg, w, kp, vp, tok, bt, lens, k_scales=ks, v_scales=vs)
        err = np.abs(lg.astype(np.float64) - rl.astype(np.float64))
        worst = max(worst, float(err.max()))
        assert np.all(err <= FP8_ATOL + FP8_RTOL * np.abs(rl.astype(np.float64))), (t, float(err.max()))
        kmask = np.zeros(kp[0].shape, bool)
        for b, c in enumerate(lens):
            kmask[bt[b][(c - 1) // 16], :, (c - 1) % 16, :] = True
        for layer in range(n_layers):
            gk, gv = cache.layer(layer)
            gk, gv = k_from_lib(gk.cpu().numpy()), v_from_lib(gv.cpu().numpy())
            _check_appended(gk, kp[layer], kmask, ks[layer])
            _check_appended(gv, vp[layer], kmask, vs[layer])
            kp[layer][...] = gk
            vp[layer][...] = gv
        g_tok = lg.argmax(-1)
        assert np.all(tie_aware_agree(g_tok, rl))
        agree += int(np.sum(g_tok == oracle.greedy_argmax(rl)))
        total += batch
        tok = prompts[:, t + 1] if t + 1 < prompts.shape[1] else g_tok.astype(np.int32)
    print(f"fp8-cache decode steps: max abs logit error {worst:.4f}, greedy agreement {agree / total:.4f}")
    assert agree / total >= 0.99
