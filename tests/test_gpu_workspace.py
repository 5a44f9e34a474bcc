"""Workspace poisoning and determinism (through the C ABI):

* canaries: every call that takes a workspace is given exactly the size its
  *_workspace_bytes call returns, between two 4 KB canary regions; after the
  call both canaries are unchanged (decode step and graph replay, prefill,
  standalone attention at the attn15 workload);
* determinism of the cross-workgroup merges (split-K GEMM partial tiles,
  attention partitions merged by the last workgroup to arrive): 100 attn15
  calls cycling over four workspaces, and 30 replays of a one-layer 1.5B-shape
  decode step on unchanged inputs, all bit-identical to the first call; the
  loops stop at the first mismatch."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev, load_case_into_cache, assert_parity, weights_to_device, oracle_config
from test_gpu_model import MID

pytestmark = pytest.mark.gpu

CANARY = 4096


def _guarded(nbytes, zero=False):
    """A buffer of nbytes between two canary regions (offsets stay 256-byte aligned)."""
    buf = torch.full((CANARY + nbytes + CANARY,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = buf[CANARY:CANARY + nbytes]
    if zero:
        ws.zero_()
    return buf, ws


def _canaries_intact(buf):
    head, tail = buf[:CANARY], buf[-CANARY:]
    return bool((head == 0xA5).all().item()) and bool((tail == 0xA5).all().item())


def test_attention_workspace_canaries_attn15(lib):
    case = inp.workload_case(inp.ATTN15)
    cache = load_case_into_cache(lib, case)
    b, hq, _ = case.q.shape
    need = lib.attn_workspace_bytes(cache, b, hq, case.max_context)
    buf, ws = _guarded(need, zero=True)
    q = dev(case.q)
    out = torch.empty_like(q)
    lib.paged_attn_decode(cache, 0, q, out, dev(case.block_tables), dev(case.ctx_lens), case.max_context,
                          case.scale, ws)
    torch.cuda.synchronize()
    assert _canaries_intact(buf)
    ref, _ = oracle.paged_attention_batch(case.q, case.k_pool, case.v_pool, case.block_tables, case.ctx_lens,
                                          case.scale)
    assert_parity(out.cpu().numpy(), ref, "attn15 with an exactly sized workspace")


def _step_rig(lib, shape, batch, mc, seed, n_layers=None):
    w = inp.model_weights(shape, seed, bias=True, norm_jitter=True, n_layers=n_layers)
    model = lib.Model(shape, weights_to_device(w), max_positions=max(mc, 64))
    stride = (mc + 15) // 16
    nb = batch * stride + 5
    n_l = shape.n_layers if n_layers is None else n_layers
    cache = lib.KVCache(n_l, nb, shape.n_kv_heads, shape.head_dim)
    for layer in range(n_l):
        for t in cache.layer(layer):
            t.normal_()
    rng = np.random.default_rng(seed + 1)
    bt = rng.permutation(nb).astype(np.int32)[: batch * stride].reshape(batch, stride)
    lens = rng.integers(1, mc + 1, size=batch).astype(np.int32)
    tok = rng.integers(0, shape.vocab, size=batch).astype(np.int32)
    return model, cache, bt, lens, tok


def test_decode_step_and_graph_workspace_canaries(lib):
    shape, batch, mc = MID, 33, 300
    model, cache, bt, lens, tok = _step_rig(lib, shape, batch, mc, 7001)
    need = lib.step_workspace_bytes(model, cache, batch, mc)
    buf, ws = _guarded(need)
    logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device="cuda")
    lib.decode_step(model, cache, dev(tok), dev(bt), dev(lens), mc, logits, ws)
    torch.cuda.synchronize()
    assert _canaries_intact(buf)
    g = lib.Graph(model, cache, dev(tok), dev(bt), dev(lens), mc, logits, ws)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    assert _canaries_intact(buf)
    assert torch.isfinite(logits.float()).all().item()
    g.close()


def test_prefill_workspace_canaries(lib):
    shape = MID
    w = inp.model_weights(shape, 7101, bias=True, norm_jitter=True)
    model = lib.Model(shape, weights_to_device(w), max_positions=4096)
    new = [37, 128, 5, 70]
    mc = 200
    stride = (mc + 15) // 16
    nb = len(new) * stride + 3
    cache = lib.KVCache(shape.n_layers, nb, shape.n_kv_heads, shape.head_dim)
    rng = np.random.default_rng(7102)
    bt = rng.permutation(nb).astype(np.int32)[: len(new) * stride].reshape(len(new), stride)
    tokens = rng.integers(0, shape.vocab, size=sum(new)).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    need = lib.prefill_workspace_bytes(model, cache, sum(new), len(new), mc)
    buf, ws = _guarded(need)
    logits = torch.empty(len(new), shape.vocab, dtype=torch.float16, device="cuda")
    lib.prefill(model, cache, dev(tokens), dev(starts), dev(np.zeros(len(new), np.int32)), dev(bt), mc, logits, ws)
    torch.cuda.synchronize()
    assert _canaries_intact(buf)
    assert torch.isfinite(logits.float()).all().item()


def test_attention_merge_is_deterministic_over_100_calls(lib):
    case = inp.workload_case(inp.ATTN15)
    cache = load_case_into_cache(lib, case)
    b, hq, _ = case.q.shape
    need = lib.attn_workspace_bytes(cache, b, hq, case.max_context)
    wss = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in range(4)]
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.ctx_lens)
    first = torch.empty_like(q)
    lib.paged_attn_decode(cache, 0, q, first, bt, lens, case.max_context, case.scale, wss[0])
    out = torch.empty_like(q)
    for i in range(1, 100):
        lib.paged_attn_decode(cache, 0, q, out, bt, lens, case.max_context, case.scale, wss[i % 4])
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"call {i} differs"
    for w_ in wss:
        assert not w_[: max(256, need // 64 // 256 * 256)].any().item()


def test_split_k_decode_step_is_deterministic_over_30_replays(lib):
    """One 1.5B-shape layer at batch 64 (split-K O and down projections) and a
    small vocabulary: 30 replays on unchanged metadata (the append rewrites the
    same slot with the same values) give bit-identical logits."""
    shape = inp.Shape(1536, 12, 2, 128, 8960, 4096, 1)
    batch, mc = 64, 200
    model, cache, bt, lens, tok = _step_rig(lib, shape, batch, mc, 7201, n_layers=1)
    ws = torch.empty(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device="cuda")
    g = lib.Graph(model, cache, dev(tok), dev(bt), dev(lens), mc, logits, ws)
    g.replay()
    torch.cuda.synchronize()
    first = logits.clone()
    for i in range(1, 30):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits.view(torch.int16), first.view(torch.int16)), f"replay {i} differs"
    g.close()
