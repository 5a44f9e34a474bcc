"""Caller errors in the per-call metadata stay inside the caller's buffers
(through the C ABI): block ids outside the pool among the entries a call uses,
and context lengths above max_context.  The kernels' own bounds checks drop
an append whose slot has no valid block and read block 0 in place of an
invalid one, so every access stays inside the pool, the tables and the
workspace.  Rows whose metadata is valid give the same bits as in a call
without the bad rows, and the cache changes only where valid rows append."""
import numpy as np
import pytest
import torch

import pkv_inputs as inp
from gpu_util import dev, k_to_lib, v_to_lib, k_from_lib, v_from_lib, weights_to_device
from test_gpu_model import MID

pytestmark = pytest.mark.gpu


def _spoil(bt, lens, nb, mc, r_append, r_read, r_long):
    """Bad metadata on three rows: the new token's block id -1 (its append and
    that block's read), a read block id past the pool, a length above max_context."""
    bt, lens = bt.copy(), lens.copy()
    assert lens[r_append] >= 1 and lens[r_read] > 16, "the case must give these rows room"
    bt[r_append, (lens[r_append] - 1) // 16] = -1
    bt[r_read, 0] = nb + 7
    lens[r_long] = mc + 40
    assert (mc + 39) // 16 >= bt.shape[1], "the long row's slot lies past the table"
    return bt, lens


def _append_slots(bt, lens, rows):
    return [(int(bt[r, (lens[r] - 1) // 16]), int((lens[r] - 1) % 16)) for r in rows if lens[r] > 0]


@pytest.mark.parametrize("batch,seed", [(6, 4101), (40, 4102)])   # GEMV and MFMA epilogues
def test_decode_layer_with_bad_rows(lib, batch, seed):
    case = inp.tiny_layer_case(seed=seed, batch=batch, ctx_lo=20, ctx_hi=300, shape=MID)
    nb, bt, lens = case["num_blocks"], case["block_tables"], case["ctx_lens"]
    mc = int(lens.max())
    assert bt.shape[1] == (mc + 15) // 16
    bad = (1, 3, 4)
    bt_bad, lens_bad = _spoil(bt, lens, nb, mc, *bad)
    w = weights_to_device(case["weights"])
    model = lib.Model(MID, w, max_positions=4096)
    cache = lib.KVCache(1, nb, MID.n_kv_heads, MID.head_dim)
    ws = torch.empty(lib.step_workspace_bytes(model, cache, batch, mc), dtype=torch.uint8, device="cuda")
    k, v = cache.layer(0)
    outs = {}
    for name, (t, c) in (("clean", (bt, lens)), ("bad", (bt_bad, lens_bad))):
        k.copy_(torch.from_numpy(k_to_lib(case["k_pool"])))
        v.copy_(torch.from_numpy(v_to_lib(case["v_pool"])))
        hidden = dev(case["hidden"])
        lib.decode_layer(model, cache, 0, hidden, dev(t), dev(c), mc, ws)
        torch.cuda.synchronize()
        outs[name] = (hidden.cpu().numpy(), k_from_lib(k.cpu().numpy()), v_from_lib(v.cpu().numpy()))
    good = [b for b in range(batch) if b not in bad]
    assert np.array_equal(outs["bad"][0][good].view(np.uint16), outs["clean"][0][good].view(np.uint16))
    # the cache: as in the clean call, except that the appends of the row
    # with the invalid block id and of the over-long row were dropped
    for i, pool in ((1, case["k_pool"]), (2, case["v_pool"])):
        want = outs["clean"][i].copy()
        for blk, slot in _append_slots(bt, lens, (bad[0], bad[2])):
            want[blk, :, slot, :] = pool[blk, :, slot, :]
        assert np.array_equal(outs["bad"][i].view(np.uint16), want.view(np.uint16))


def test_standalone_attention_and_append_with_bad_rows(lib):
    case = inp.attention_case(7, 12, 2, 128, 20, 300, seed=4103)
    nb, bt, lens = case.num_blocks, case.block_tables, case.ctx_lens
    mc = case.max_context
    bad = (0, 2, 5)
    bt_bad, lens_bad = _spoil(bt, lens, nb, mc, *bad)
    cache = lib.KVCache(1, nb, 2, 128)
    k, v = cache.layer(0)
    k0, v0 = torch.from_numpy(k_to_lib(case.k_pool)), torch.from_numpy(v_to_lib(case.v_pool))
    ws = lib.attn_workspace(cache, 7, 12, mc)
    q = dev(case.q)
    region = max(256, ws.numel() // 64 // 256 * 256)
    outs = {}
    for name, (t, c) in (("clean", (bt, lens)), ("bad", (bt_bad, lens_bad))):
        k.copy_(k0)
        v.copy_(v0)
        out = torch.empty_like(q)
        lib.paged_attn_decode(cache, 0, q, out, dev(t), dev(c), mc, case.scale, ws)
        torch.cuda.synchronize()
        assert not ws[:region].any().item(), f"{name}: arrival counters left set"
        # the standalone append of one token per row, into the same tables
        kn = dev(np.full((7, 2, 128), 0.5, np.float16))
        vn = dev(np.full((7, 2, 128), -0.25, np.float16))
        lib.kv_append(cache, 0, kn, vn, dev(t), dev(c))
        torch.cuda.synchronize()
        outs[name] = (out.cpu().numpy(), k_from_lib(k.cpu().numpy()), v_from_lib(v.cpu().numpy()))
    good = [b for b in range(7) if b not in bad]
    assert np.array_equal(outs["bad"][0][good].view(np.uint16), outs["clean"][0][good].view(np.uint16))
    for i, pool in ((1, case.k_pool), (2, case.v_pool)):
        want = outs["clean"][i].copy()
        for blk, slot in _append_slots(bt, lens, (bad[0], bad[2])):
            want[blk, :, slot, :] = pool[blk, :, slot, :]
        assert np.array_equal(outs["bad"][i].view(np.uint16), want.view(np.uint16))
