"""GPU parity of the decoder layer, the decode step, greedy argmax and graph
replay (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev, assert_parity, weights_to_device, oracle_config, k_to_lib, k_from_lib, v_to_lib, v_from_lib

pytestmark = pytest.mark.gpu

MID = inp.Shape(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, ffn=1408, vocab=1000, n_layers=2)
# FFN wide enough that the down projection spreads a row over a whole workgroup
WIDE = inp.Shape(hidden=512, n_q_heads=12, n_kv_heads=2, head_dim=128, ffn=4096, vocab=1000, n_layers=2)


def _layer_case(shape, batch, seed, lo=1, hi=64):
    return inp.tiny_layer_case(seed=seed, batch=batch, ctx_lo=lo, ctx_hi=hi, shape=shape)


def _layer_rig(pkv, shape, case, max_context=None):
    """Model, cache (case pools loaded), tables, lengths, max context and workspace."""
    w = weights_to_device(case["weights"])
    model = pkv.Model(shape, w, max_positions=4096)
    cache = pkv.KVCache(1, case["num_blocks"], shape.n_kv_heads, shape.head_dim)
    k, v = cache.layer(0)
    k.copy_(torch.from_numpy(k_to_lib(case["k_pool"])))
    v.copy_(torch.from_numpy(v_to_lib(case["v_pool"])))
    b = case["hidden"].shape[0]
    mc = max_context or int(case["ctx_lens"].max())
    bt = case["block_tables"]
    if bt.shape[1] * 16 < mc:
        bt = np.concatenate([bt, np.full((b, (mc + 15) // 16 - bt.shape[1]), -1, np.int32)], axis=1)
    ws = torch.empty(pkv.step_workspace_bytes(model, cache, b, mc), dtype=torch.uint8, device="cuda")
    return model, cache, dev(bt), dev(case["ctx_lens"]), mc, ws, w


def _run_layer_gpu(pkv, shape, case, max_context=None):
    w = weights_to_device(case["weights"])
    model = pkv.Model(shape, w, max_positions=4096)
    nb = case["num_blocks"]
    cache = pkv.KVCache(1, nb, shape.n_kv_heads, shape.head_dim)
    k, v = cache.layer(0)
    k.copy_(torch.from_numpy(k_to_lib(case["k_pool"])))
    v.copy_(torch.from_numpy(v_to_lib(case["v_pool"])))
    b = case["hidden"].shape[0]
    mc = max_context or int(case["ctx_lens"].max())
    bt = case["block_tables"]
    if bt.shape[1] * 16 < mc:
        bt = np.concatenate([bt, np.full((b, (mc + 15) // 16 - bt.shape[1]), -1, np.int32)], axis=1)
    hidden = dev(case["hidden"])
    ws = torch.empty(pkv.step_workspace_bytes(model, cache, b, mc), dtype=torch.uint8, device="cuda")
    pkv.decode_layer(model, cache, 0, hidden, dev(bt), dev(case["ctx_lens"]), mc, ws)
    torch.cuda.synchronize()
    return hidden.cpu().numpy(), k_from_lib(k.cpu().numpy()), v_from_lib(v.cpu().numpy())


def _oracle_layer(shape, case):
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    h = oracle.decode_layer(oracle_config(shape, 1), case["weights"]["layers"][0], case["hidden"], kp, vp,
                            case["block_tables"], case["ctx_lens"])
    return h, kp, vp


@pytest.mark.parametrize("shape,batch,seed,hi", [
    (inp.TINY, 4, 1001, 64),       # the one-layer workload (GEMV path)
    (inp.TINY, 40, 1011, 64),      # MFMA path, ragged last M tile
    (MID, 3, 1021, 300),           # D = 128, G = 6
    (MID, 70, 1031, 200),          # MFMA path at D = 128
    (MID, 1, 1051, 300),           # GEMV batch buckets 1, 2, 16 and 32
    (MID, 2, 1061, 300),
    (MID, 12, 1071, 100),
    (MID, 31, 1081, 100),
    (WIDE, 2, 1091, 100),          # 256 lanes per row, cross-wave reduction
])
def test_decode_layer_parity(lib, shape, batch, seed, hi):
    case = _layer_case(shape, batch, seed, hi=hi)
    h, k, v = _run_layer_gpu(lib, shape, case)
    rh, rk, rv = _oracle_layer(shape, case)
    assert_parity(h, rh, "hidden after layer")
    # cache: appended slots within the parity bar, every other byte untouched
    changed = np.zeros(rk.shape, bool)
    for b, c in enumerate(case["ctx_lens"]):
        changed[case["block_tables"][b][(c - 1) // 16], :, (c - 1) % 16, :] = True
    keep = ~changed
    assert np.array_equal(k[keep].view(np.uint16), case["k_pool"][keep].view(np.uint16))
    assert_parity(k[changed], rk[changed], "appended K")
    assert np.array_equal(v[keep].view(np.uint16), case["v_pool"][keep].view(np.uint16))
    assert_parity(v[changed], rv[changed], "appended V")


@pytest.mark.parametrize("shape,batch,seed,hi", [
    (inp.TINY, 4, 1301, 64),       # GEMV path
    (MID, 3, 1302, 300),           # D = 128, several partitions
    (MID, 70, 1303, 200),          # MFMA path
    (WIDE, 2, 1304, 100),          # down projection over a whole workgroup per row
])
def test_decode_layer_xr_parity(lib, shape, batch, seed, hi):
    """The (x, residual) form: residual after the attention sub-block and the
    MLP output (not yet added) against the oracle's, each within the bar, and
    the cache's appended slots as for the plain layer."""
    case = _layer_case(shape, batch, seed, hi=hi)
    rng = np.random.default_rng(seed + 5)
    x = (rng.standard_normal(case["hidden"].shape) * 0.5).astype(np.float16)
    r = case["hidden"]
    model, cache, bt, lens, mc, ws, _w = _layer_rig(lib, shape, case)
    xd, rd = dev(x), dev(r)
    lib.decode_layer_xr(model, cache, 0, xd, rd, bt, lens, mc, ws)
    torch.cuda.synchronize()
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    ox, orr = oracle.decode_layer_xr(oracle_config(shape, 1), case["weights"]["layers"][0], x, r, kp, vp,
                                     case["block_tables"], case["ctx_lens"])
    assert_parity(rd.cpu().numpy(), orr, "residual after the attention sub-block")
    assert_parity(xd.cpu().numpy(), ox, "MLP output")
    k, v = cache.layer(0)
    changed = np.zeros(kp.shape, bool)
    for b, c in enumerate(case["ctx_lens"]):
        changed[case["block_tables"][b][(c - 1) // 16], :, (c - 1) % 16, :] = True
    assert_parity(k_from_lib(k.cpu().numpy())[changed], kp[changed], "appended K")
    assert_parity(v_from_lib(v.cpu().numpy())[changed], vp[changed], "appended V")


def test_decode_layer_xr_chain_equals_plain_chain(lib):
    """Two layers in (x, residual) form from (embedding-like x, zero residual)
    end at f16(residual + x), which matches two plain layers on h = x within
    the bar; x and residual must be distinct buffers."""
    shape = MID
    case = _layer_case(shape, 6, 1311, hi=200)
    model, cache, bt, lens, mc, ws, _w = _layer_rig(lib, shape, case)
    x = dev(case["hidden"])
    r = torch.zeros_like(x)
    for _ in range(2):
        lib.decode_layer_xr(model, cache, 0, x, r, bt, lens, mc, ws)
    final = (r.float() + x.float()).half().cpu().numpy()
    model2, cache2, bt2, lens2, mc2, ws2, _w2 = _layer_rig(lib, shape, case)
    h = dev(case["hidden"])
    for _ in range(2):
        lib.decode_layer(model2, cache2, 0, h, bt2, lens2, mc2, ws2)
    torch.cuda.synchronize()
    assert_parity(final, h.cpu().numpy(), "two layers, (x, residual) form against plain")
    with pytest.raises(lib.PkvError):
        lib.decode_layer_xr(model, cache, 0, x, x, bt, lens, mc, ws)


def test_decode_layer_without_bias_and_unit_gains(lib):
    case = inp.tiny_layer_case(seed=1041, batch=5, bias=False, norm_jitter=False, shape=MID)
    h, _, _ = _run_layer_gpu(lib, MID, case)
    rh, _, _ = _oracle_layer(MID, case)
    assert_parity(h, rh, "no-bias layer")


class StepRig:
    """A small model decoding several rows through the GPU step and the oracle."""

    def __init__(self, pkv, shape, batch, seed, prompt_len, max_context):
        self.pkv, self.shape, self.batch = pkv, shape, batch
        self.w = inp.model_weights(shape, seed, bias=True, norm_jitter=True, std=0.05)
        self.model = pkv.Model(shape, weights_to_device(self.w), max_positions=max_context)
        self.mc = max_context
        stride = (max_context + 15) // 16
        self.nb = batch * stride + 7
        self.cache = pkv.KVCache(shape.n_layers, self.nb, shape.n_kv_heads, shape.head_dim)
        rng = np.random.default_rng(seed + 1)
        perm = rng.permutation(self.nb).astype(np.int32)
        self.bt = perm[: batch * stride].reshape(batch, stride)
        self.prompts = rng.integers(0, shape.vocab, size=(batch, prompt_len)).astype(np.int32)
        self.lens = np.zeros(batch, np.int32)
        self.ws = torch.empty(pkv.step_workspace_bytes(self.model, self.cache, batch, max_context),
                              dtype=torch.uint8, device="cuda")
        self.logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device="cuda")
        self.hidden = torch.empty(batch, shape.hidden, dtype=torch.float16, device="cuda")
        self.kp = [np.full((self.nb, shape.n_kv_heads, 16, shape.head_dim), np.nan, np.float16)
                   for _ in range(shape.n_layers)]
        self.vp = [np.full((self.nb, shape.n_kv_heads, 16, shape.head_dim), np.nan, np.float16)
                   for _ in range(shape.n_layers)]
        self.cfg = oracle_config(shape)
        self.d_bt = dev(self.bt)

    def gpu_step(self, tokens):
        self.lens += 1
        self.pkv.decode_step(self.model, self.cache, dev(tokens), self.d_bt, dev(self.lens), self.mc,
                             self.logits, self.ws, hidden_out=self.hidden)
        torch.cuda.synchronize()
        return self.logits.cpu().numpy(), self.hidden.cpu().numpy()

    def oracle_step(self, tokens):
        return oracle.decode_step(self.cfg, self.w, self.kp, self.vp, tokens, self.bt, self.lens)


@pytest.mark.parametrize("batch", [3, 33])
def test_decode_step_parity_and_greedy(lib, batch):
    rig = StepRig(lib, MID, batch, seed=2001, prompt_len=20, max_context=64)
    agree = total = 0
    tok = rig.prompts[:, 0]
    for t in range(30):
        lg, hd = rig.gpu_step(tok)
        rl, rh = rig.oracle_step(tok)
        assert_parity(lg, rl, f"logits step {t}")
        assert_parity(hd, rh, f"hidden step {t}")
        g_tok = lg.argmax(-1)
        agree += int(np.sum(g_tok == oracle.greedy_argmax(rl)))
        total += batch
        # teacher forcing: both sides get the prompt, then the GPU's own tokens
        tok = rig.prompts[:, t + 1] if t + 1 < rig.prompts.shape[1] else g_tok.astype(np.int32)
    assert agree / total >= 0.99


def test_decode_step_out_of_range_tokens_embed_as_zero(lib):
    """Token ids outside [0, V) (the -1 the argmax gives an inactive row, the
    vocabulary size itself, a large negative id) embed as zero rows on both
    sides (reading R25); the other rows are unaffected."""
    rig = StepRig(lib, MID, 5, seed=2011, prompt_len=4, max_context=32)
    for t in range(3):
        tok = rig.prompts[:, t].astype(np.int32).copy()
        tok[1], tok[3], tok[4] = -1, MID.vocab + t, -(1 << 20)
        lg, hd = rig.gpu_step(tok)
        rl, rh = rig.oracle_step(tok)
        assert_parity(lg, rl, f"logits step {t}")
        assert_parity(hd, rh, f"hidden step {t}")


@pytest.mark.parametrize("vocab", [151936, 152064, 163840, 163848, 1000, 999])
def test_argmax_kernel(lib, vocab):
    # vocab 163840 fills exactly one round of loads per thread, 163848 needs a
    # second round for one vector, 999 takes the unaligned (scalar) path
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((7, vocab)).astype(np.float16)
    lg[1, [5, 77, vocab - 3]] = 30.0       # ties: lowest index wins
    lg[2, :] = -1.0
    lg[3, 100] = np.nan
    lg[4, vocab - 1] = 40.0                # the row's very last logit
    lg[5, [vocab - 1, vocab - 9]] = 35.0   # a tie inside the last vector and the one before
    # NaN never wins: -inf beats a leading NaN, a row of NaNs gives 0, +inf wins
    extra = np.full((4, vocab), -np.inf, np.float16)
    extra[0, 0] = np.nan
    extra[1, :] = np.nan
    extra[2, :] = rng.standard_normal(vocab).astype(np.float16)
    extra[2, [0, vocab // 2]] = np.nan
    extra[2, vocab - 2] = np.inf
    extra[3, [1, 2]] = np.nan
    lg = np.concatenate([lg, extra])
    out = torch.empty(lg.shape[0], dtype=torch.int32, device="cuda")
    lib.argmax(dev(lg), out)
    torch.cuda.synchronize()
    want = oracle.greedy_argmax(lg)
    assert want[7:].tolist() == [1, 0, vocab - 2, 0]
    assert out.cpu().numpy().tolist() == want.tolist()


def test_graph_replay_matches_eager_and_sees_new_metadata(lib):
    """Capture one step, then replay it with rewritten tokens / lengths: every
    replay equals the eager step on the same metadata, bit for bit."""
    shape = MID
    batch, mc = 5, 64
    eager = StepRig(lib, shape, batch, seed=3001, prompt_len=12, max_context=mc)
    graph_rig = StepRig(lib, shape, batch, seed=3001, prompt_len=12, max_context=mc)
    toks = dev(graph_rig.prompts[:, 0])
    lens = dev(graph_rig.lens)
    g = lib.Graph(graph_rig.model, graph_rig.cache, toks, graph_rig.d_bt, lens, mc, graph_rig.logits,
                  graph_rig.ws, hidden_out=graph_rig.hidden)
    for t in range(12):
        graph_rig.lens += 1
        # metadata for this step written on the replay stream, then replay there
        toks.copy_(torch.from_numpy(graph_rig.prompts[:, t]))
        lens.copy_(torch.from_numpy(graph_rig.lens))
        g.replay()
        torch.cuda.synchronize()
        gl = graph_rig.logits.cpu().numpy()
        el, _ = eager.gpu_step(eager.prompts[:, t])
        assert np.array_equal(gl.view(np.uint16), el.view(np.uint16)), t
    g.close()


def test_long_context_layer_in_worklist_form(lib):
    """40 rows x 2 KV heads with contexts of 600-4096 tokens: the layer's
    attention runs in work-list form (long rows over a grid of several
    rounds).  The layer matches the oracle, and the direct grid of the same
    partitions (hook off) gives the same bits."""
    rng = np.random.default_rng(4101)
    lens = inp.context_lengths(rng, 40, 600, 4096, "loguniform")
    lens[7] = 4096
    case = inp.tiny_layer_case(seed=4102, batch=40, shape=MID, ctx_lens=lens)
    rh, _, _ = _oracle_layer(MID, case)
    outs = []
    try:
        for enable in (True, False):
            lib.debug_attn_worklist(enable)
            h, _, _ = _run_layer_gpu(lib, MID, case)
            outs.append(h)
    finally:
        lib.debug_attn_worklist(True)
    assert_parity(outs[0], rh, "long-context layer (work-list form)")
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))


def test_graph_replay_with_worklist_attention_matches_eager(lib):
    """A captured step whose attention runs in work-list form (24 rows x 2 KV
    heads, contexts up to 8000 over a random pre-filled cache): four replays
    with advancing lengths equal the eager steps bit for bit, and so does the
    eager step on the direct grid (hook off)."""
    shape = MID
    batch, mc = 24, 8192
    rng = np.random.default_rng(4201)
    w = inp.model_weights(shape, 4202, bias=True, norm_jitter=True, std=0.05)
    model = lib.Model(shape, weights_to_device(w), max_positions=mc)
    stride = mc // 16
    nb = batch * stride + 5
    cache = lib.KVCache(shape.n_layers, nb, shape.n_kv_heads, shape.head_dim)
    g = torch.Generator(device="cuda")
    g.manual_seed(4203)
    for layer in range(shape.n_layers):
        for t in cache.layer(layer):
            t.normal_(generator=g)
    bt = dev(rng.permutation(nb)[: batch * stride].astype(np.int32).reshape(batch, stride))
    lens_h = inp.context_lengths(rng, batch, 600, 7990, "loguniform")
    toks_h = rng.integers(0, shape.vocab, size=(5, batch)).astype(np.int32)
    ws = torch.empty(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device="cuda")
    toks, lens = dev(toks_h[0]), dev(lens_h)
    graph = lib.Graph(model, cache, toks, bt, lens, mc, logits, ws)
    try:
        for t in range(4):
            lens_h = lens_h + 1
            toks.copy_(torch.from_numpy(toks_h[t]))
            lens.copy_(torch.from_numpy(lens_h))
            runs = []
            for mode in ("eager", "direct", "graph"):
                lib.debug_attn_worklist(mode != "direct")
                if mode == "graph":
                    graph.replay()
                else:
                    lib.decode_step(model, cache, toks, bt, lens, mc, logits, ws)
                torch.cuda.synchronize()
                runs.append(logits.cpu().numpy().copy())
            assert np.all(np.isfinite(runs[0]))
            for r in runs[1:]:
                assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16)), t
    finally:
        lib.debug_attn_worklist(True)
        graph.close()


def test_graph_set_buckets_with_inactive_rows(lib):
    """Buckets 1/4/8 over shared buffers: 3 active rows run in bucket 4, then 6
    in bucket 8 (rows 3-5 join); active rows match the oracle, padding rows get
    token -1 and never touch the cache."""
    shape, mc, buckets = MID, 64, [1, 4, 8]
    w = inp.model_weights(shape, 4001, bias=True, norm_jitter=True, std=0.05)
    model = lib.Model(shape, weights_to_device(w), max_positions=mc)
    stride = (mc + 15) // 16
    nb = 8 * stride + 7
    cache = lib.KVCache(shape.n_layers, nb, shape.n_kv_heads, shape.head_dim)
    for layer in range(shape.n_layers):
        for t_ in cache.layer(layer):
            t_.zero_()
    rng = np.random.default_rng(4002)
    bt = rng.permutation(nb).astype(np.int32)[: 8 * stride].reshape(8, stride)
    prompts = rng.integers(0, shape.vocab, size=(8, 12)).astype(np.int32)
    lens = np.zeros(8, np.int32)
    tok_d = torch.zeros(8, dtype=torch.int32, device="cuda")
    lens_d = torch.zeros(8, dtype=torch.int32, device="cuda")
    logits = torch.empty(8, shape.vocab, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(lib.step_workspace_bytes(model, cache, b, mc) for b in buckets), dtype=torch.uint8,
                     device="cuda")
    gs = lib.GraphSet(model, cache, buckets, tok_d, dev(bt), lens_d, mc, logits, ws)
    kp = [np.full((nb, shape.n_kv_heads, 16, shape.head_dim), np.nan, np.float16) for _ in range(shape.n_layers)]
    vp = [np.full((nb, shape.n_kv_heads, 16, shape.head_dim), np.nan, np.float16) for _ in range(shape.n_layers)]
    cfg = oracle_config(shape)
    out = torch.empty(8, dtype=torch.int32, device="cuda")
    for phase, n in ((0, 3), (1, 6)):
        for t in range(6):
            lens[:n] += 1
            tok = prompts[:n, 6 * phase + t]
            host_tok = np.zeros(8, np.int32)
            host_tok[:n] = tok
            tok_d.copy_(torch.from_numpy(host_tok))
            lens_d.copy_(torch.from_numpy(lens))
            bk = gs.replay(n)
            assert bk == (4 if n == 3 else 8)
            lib.argmax(logits[:bk], out[:bk], context_lens=lens_d[:bk])
            torch.cuda.synchronize()
            rl, _ = oracle.decode_step(cfg, w, kp, vp, tok, bt[:n], lens[:n])
            assert_parity(logits[:n].cpu().numpy(), rl, f"bucket {bk}, step {t}")
            got = out[:bk].cpu().numpy()
            assert np.all(got[n:] == -1)
            assert lens_d[n:bk].cpu().numpy().tolist() == [0] * (bk - n)
    # rows 6 and 7 were never active: their blocks are still zero
    for layer in range(shape.n_layers):
        k, v = cache.layer(layer)
        k, v = k.cpu().numpy(), v.cpu().numpy()
        for b in (6, 7):
            assert not k[bt[b]].any() and not v[bt[b]].any()
    gs.close()


@pytest.mark.parametrize("shape,batch,seed,hi", [(MID, 3, 1101, 300), (MID, 70, 1102, 200),
                                                 (inp.Shape(1536, 12, 2, 128, 8960, 16, 1), 256, 1103, 700)])
def test_layer_ops_in_order_equal_decode_layer(lib, shape, batch, seed, hi):
    """pkv_layer_op for QKV, ATTN, O, GATE_UP, DOWN in order gives the hidden
    state and cache of pkv_decode_layer bit for bit (1.5B layer at batch 256:
    split-K and the 128 x 160 gate/up tiles of the bench)."""
    case = _layer_case(shape, batch, seed, hi=hi)
    h_ref, k_ref, v_ref = _run_layer_gpu(lib, shape, case)
    w = weights_to_device(case["weights"])
    model = lib.Model(shape, w, max_positions=4096)
    cache = lib.KVCache(1, case["num_blocks"], shape.n_kv_heads, shape.head_dim)
    k, v = cache.layer(0)
    k.copy_(torch.from_numpy(k_to_lib(case["k_pool"])))
    v.copy_(torch.from_numpy(v_to_lib(case["v_pool"])))
    mc = int(case["ctx_lens"].max())
    hidden = dev(case["hidden"])
    ws = torch.zeros(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    bt, lens = dev(case["block_tables"]), dev(case["ctx_lens"])
    for op in (lib.OP_QKV, lib.OP_ATTN, lib.OP_O, lib.OP_GATE_UP, lib.OP_DOWN):
        lib.layer_op(model, cache, 0, op, hidden, bt, lens, mc, ws)
    torch.cuda.synchronize()
    assert np.array_equal(hidden.cpu().numpy().view(np.uint16), h_ref.view(np.uint16))
    assert np.array_equal(k_from_lib(k.cpu().numpy()).view(np.uint16), k_ref.view(np.uint16))
    assert np.array_equal(v_from_lib(v.cpu().numpy()).view(np.uint16), v_ref.view(np.uint16))
    with pytest.raises(lib.PkvError, match="op must be"):
        lib.layer_op(model, cache, 0, 7, hidden, bt, lens, mc, ws)
