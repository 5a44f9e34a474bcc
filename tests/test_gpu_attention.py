"""GPU parity of paged GQA decode attention and the KV append (through the C ABI)
against the oracle, plus bit-exact addressing checks."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev, load_case_into_cache, assert_parity, k_from_lib, v_from_lib

pytestmark = pytest.mark.gpu


def run_attention(pkv, case, max_context=None, cache=None, with_lse=True, ws=None):
    cache = load_case_into_cache(pkv, case, cache=cache)
    mc = max_context or case.max_context
    b, hq, d = case.q.shape
    q = dev(case.q)
    out = torch.empty_like(q)
    lse = torch.empty(b, hq, dtype=torch.float32, device="cuda") if with_lse else None
    if ws is None:
        ws = pkv.attn_workspace(cache, b, hq, mc)
    bt = case.block_tables
    if bt.shape[1] * 16 < mc:
        bt = np.concatenate([bt, np.full((b, (mc + 15) // 16 - bt.shape[1]), -1, np.int32)], axis=1)
    pkv.paged_attn_decode(cache, 0, q, out, dev(bt), dev(case.ctx_lens), mc, case.scale, ws, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def oracle_attention(case):
    return oracle.paged_attention_batch(case.q, case.k_pool, case.v_pool, case.block_tables, case.ctx_lens,
                                        case.scale, k_scale=case.k_scale, v_scale=case.v_scale)


@pytest.mark.parametrize("b,hq,hkv,d,lo,hi,seed", [
    (4, 4, 2, 64, 1, 64, 1001),        # one-layer workload shape
    (7, 12, 2, 128, 1, 700, 3),        # ragged, several partitions
    (5, 28, 4, 128, 1, 300, 4),        # 7B head shape, G = 7
    (3, 16, 1, 64, 1, 2100, 5),        # G = 16, one KV head
    (6, 8, 8, 128, 1, 90, 6),          # MHA (G = 1)
    (9, 12, 2, 128, 900, 2000, 7),     # 18 pairs x 2 partitions dealt to the XCDs, last round partly empty
    (9, 12, 2, 128, 1, 4000, 9),       # the same with up to 4 partitions per pair
    (24, 28, 4, 128, 500, 1000, 10),   # 96 rows of at most 1024 tokens: 256-token partitions, merged
    (130, 28, 4, 128, 500, 760, 11),   # 520 rows of at most 768 tokens: one 8-wave partition per row
])
def test_attention_parity_f16(lib, b, hq, hkv, d, lo, hi, seed):
    case = inp.attention_case(b, hq, hkv, d, lo, hi, seed)
    out, lse = run_attention(lib, case)
    ref, ref_lse = oracle_attention(case)
    assert_parity(out, ref, "attention out")
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-4, atol=1e-4)


def test_attention_parity_attn15_full_size(lib):
    """Qwen2.5-1.5B layer shape, batch 64, contexts U[128, 2048], shuffled pool."""
    case = inp.workload_case(inp.ATTN15)
    out, lse = run_attention(lib, case)
    ref, ref_lse = oracle_attention(case)
    err = assert_parity(out, ref, "attn15")
    assert err < 5e-3
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-4, atol=1e-4)


def test_attention_parity_fp8_ragged(lib):
    case = inp.attention_case(6, 28, 4, 128, 1, 3000, seed=8, dist="loguniform", kv_dtype="fp8")
    out, _ = run_attention(lib, case)
    ref, _ = oracle_attention(case)
    assert_parity(out, ref, "fp8 attention")


def test_attention_parity_fp8long_full_size(lib):
    """7B layer shape, fp8 E4M3 KV, batch 32, contexts log-uniform in [1024, 32768]."""
    case = inp.workload_case(inp.FP8LONG)
    out, lse = run_attention(lib, case)
    ref, ref_lse = oracle_attention(case)
    assert_parity(out, ref, "fp8long")
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-4, atol=1e-4)


def test_fp8_all_codes_decode_exactly(lib):
    """Single-token contexts make out = V exactly: all 256 E4M3 codes through the kernel."""
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    kp = np.full((2, 1, 16, 128), 0x38, np.uint8)      # K = 1.0 everywhere
    vp = np.full((2, 1, 16, 128), 0x7F, np.uint8)      # NaN outside slot 0
    vp[:, 0, 0, :] = codes
    case = inp.AttnCase(q=np.ones((2, 1, 128), np.float16), k_pool=kp, v_pool=vp,
                        block_tables=np.array([[0], [1]], np.int32), ctx_lens=np.array([1, 1], np.int32),
                        scale=0.125, k_scale=1.0, v_scale=1.0, num_blocks=2, max_context=1)
    out, _ = run_attention(lib, case, with_lse=False)
    want = oracle.e4m3_decode(codes).astype(np.float16)
    got = out[:, 0, :]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    # bit-exact except the sign of zero: code 0x80 (-0) leaves the fp32
    # accumulator (which starts at +0) as +0
    nz = ~nan & (want != 0)
    assert np.array_equal(got[nz].view(np.uint16), want[nz].view(np.uint16))
    assert np.all(got[~nan & (want == 0)] == 0)


def test_one_hot_probe_bit_exact(lib):
    """q = 64 e_0 and K_t[0] = 64 only at t*: out = V_{t*} bit for bit, for every page."""
    rng = np.random.default_rng(9)
    b, d = 6, 128
    lens = np.array([1, 16, 17, 250, 1000, 2047], np.int32)
    case = inp.attention_case(b, 2, 1, d, 1, 1, seed=10, ctx_lens=lens)
    k = np.nan_to_num(case.k_pool, nan=0.0).copy()
    k[..., 0] = 0
    tstar = np.array([rng.integers(0, c) for c in lens])
    for i in range(b):
        blk = case.block_tables[i][tstar[i] // 16]
        k[blk, 0, tstar[i] % 16, 0] = 64
    case.k_pool = np.where(np.isnan(case.k_pool), case.k_pool, k).astype(np.float16)
    case.q = np.zeros_like(case.q)
    case.q[:, :, 0] = 64
    out, _ = run_attention(lib, case, with_lse=False)
    for i in range(b):
        blk = case.block_tables[i][tstar[i] // 16]
        want = case.v_pool[blk, 0, tstar[i] % 16, :]
        assert np.array_equal(out[i, 0].view(np.uint16), want.view(np.uint16)), i
        assert np.array_equal(out[i, 1].view(np.uint16), want.view(np.uint16)), i


def test_block_permutation_invariance_bit_exact(lib):
    """The same tokens under two different physical block assignments give identical bits."""
    case = inp.attention_case(5, 12, 2, 128, 1, 600, seed=11)
    out1, _ = run_attention(lib, case)
    rng = np.random.default_rng(12)
    perm = rng.permutation(case.num_blocks).astype(np.int32)      # old id -> new id
    k2 = np.empty_like(case.k_pool)
    v2 = np.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    bt2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    case2 = inp.AttnCase(case.q, k2, v2, bt2, case.ctx_lens, case.scale, num_blocks=case.num_blocks,
                         max_context=case.max_context)
    out2, _ = run_attention(lib, case2)
    assert np.array_equal(out1.view(np.uint16), out2.view(np.uint16))


def test_split_plan_invariance(lib):
    """A larger max_context changes the partitioning; results agree within 1e-3."""
    case = inp.attention_case(4, 12, 2, 128, 300, 900, seed=13)
    a, _ = run_attention(lib, case)
    b, _ = run_attention(lib, case, max_context=32768)
    np.testing.assert_allclose(a.astype(np.float64), b.astype(np.float64), atol=1e-3, rtol=1e-3)


def test_workspace_reused_across_calls(lib):
    """One workspace for consecutive calls of different shapes: the arrival
    counters at its head are back to zero after every call, and every call
    matches the oracle."""
    big = inp.attention_case(7, 12, 2, 128, 300, 2100, seed=18)
    small = inp.attention_case(3, 12, 2, 128, 1, 1500, seed=19)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    for case in (big, small, big):
        out, _ = run_attention(lib, case, ws=ws)
        ref, _ = oracle_attention(case)
        assert_parity(out, ref, "workspace reuse")
        assert not ws[:_counter_region(ws.numel())].any().item()


def _counter_region(ws_bytes):
    """Leading bytes of a standalone attention workspace that hold the arrival
    counters (include/pkv.h: W / 64 in whole 256-byte units, at least 256)."""
    return max(256, ws_bytes // 64 // 256 * 256)


def test_workspace_small_batch_then_large_batch(lib):
    """A batch-3 call whose rows span several partitions writes partial results,
    then a batch-64 call (the attn15 workload) on the same workspace: the large
    call's counters must not read the small call's partials.  Every call
    matches the oracle and leaves the whole counter region zero."""
    small = inp.attention_case(3, 12, 2, 128, 900, 1500, seed=21)
    big = inp.workload_case(inp.ATTN15)
    cache = load_case_into_cache(lib, big)
    need = max(lib.attn_workspace_bytes(cache, 3, 12, small.max_context),
               lib.attn_workspace_bytes(cache, 64, 12, big.max_context))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    region = _counter_region(need)
    for case in (small, big, small, big):
        out, _ = run_attention(lib, case, ws=ws)
        ref, _ = oracle_attention(case)
        assert_parity(out, ref, f"batch {case.q.shape[0]} after reuse")
        assert not ws[:region].any().item()


def test_merge_by_first_partition_equals_last_arriver_merge(lib):
    """attn15 runs the 8-wave plan (about half its rows in two partitions).
    There the first partition of a row keeps its partial on chip, waits for
    the others and merges; with a zero wait it publishes at once and the last
    partition to arrive merges instead (the fallback path).  Both give the
    same bits (output and log-sum-exp), match the oracle and leave the
    counter region zero."""
    case = inp.workload_case(inp.ATTN15)
    cache = load_case_into_cache(lib, case)
    ws = lib.attn_workspace(cache, 64, 12, case.max_context)
    region = _counter_region(ws.numel())
    runs = []
    try:
        for ticks in (10000, 0, 10000, 0):
            lib.debug_attn_merge_wait(ticks)
            runs.append(run_attention(lib, case, cache=cache, ws=ws))
            assert not ws[:region].any().item(), f"counters left set (wait {ticks})"
    finally:
        lib.debug_attn_merge_wait(10000)
    ref, _ = oracle_attention(case)
    assert_parity(runs[0][0], ref, "merge by the first partition")
    for out, lse in runs[1:]:
        assert np.array_equal(out.view(np.uint16), runs[0][0].view(np.uint16))
        assert np.array_equal(lse.view(np.uint32), runs[0][1].view(np.uint32))


@pytest.mark.parametrize("kv_dtype", ["f16", "fp8"])
def test_worklist_form_equals_direct_grid(lib, kv_dtype):
    """40 rows x 4 KV heads with log-uniform contexts up to 8192 (and three
    inactive rows) need more workgroups than the device holds at once, so
    the call runs in work-list form (only the partitions inside each row's
    context, longest rows first).  The direct grid of every partition (hook
    off) gives the same bits, both match the oracle, and the counter region
    (arrival counters, item and exit counts) is zero after every call."""
    rng = np.random.default_rng(31)
    lens = inp.context_lengths(rng, 40, 1, 8192, "loguniform")
    lens[[3, 17, 38]] = 0
    lens[5] = 8192
    case = inp.attention_case(40, 28, 4, 128, 1, 8192, seed=32, kv_dtype=kv_dtype, ctx_lens=lens)
    cache = load_case_into_cache(lib, case)
    ws = lib.attn_workspace(cache, 40, 28, case.max_context)
    region = _counter_region(ws.numel())
    runs = []
    try:
        for enable in (True, False, True):
            lib.debug_attn_worklist(enable)
            runs.append(run_attention(lib, case, cache=cache, ws=ws))
            assert not ws[:region].any().item(), f"counters left set (work list {enable})"
    finally:
        lib.debug_attn_worklist(True)
    ref, ref_lse = oracle_attention(case)
    assert_parity(runs[0][0], ref, f"work-list form ({kv_dtype})")
    assert np.all(runs[0][0][[3, 17, 38]] == 0) and np.all(np.isneginf(runs[0][1][[3, 17, 38]]))
    for out, lse in runs[1:]:
        assert np.array_equal(out.view(np.uint16), runs[0][0].view(np.uint16))
        assert np.array_equal(lse.view(np.uint32), runs[0][1].view(np.uint32))


def test_inactive_rows(lib):
    case = inp.attention_case(4, 4, 2, 64, 1, 40, seed=14, ctx_lens=[0, 5, 0, 33])
    out, lse = run_attention(lib, case)
    assert np.all(out[[0, 2]] == 0) and np.all(np.isneginf(lse[[0, 2]]))
    ref, _ = oracle_attention(case)
    assert_parity(out, ref, "inactive rows")


def test_kv_append_bit_exact(lib):
    case = inp.attention_case(9, 4, 2, 128, 1, 200, seed=15, ctx_lens=[1, 16, 17, 32, 33, 100, 0, 200, 2])
    cache = load_case_into_cache(lib, case)
    rng = np.random.default_rng(16)
    k = rng.standard_normal((9, 2, 128)).astype(np.float16)
    v = rng.standard_normal((9, 2, 128)).astype(np.float16)
    lib.kv_append(cache, 0, dev(k), dev(v), dev(case.block_tables), dev(case.ctx_lens))
    torch.cuda.synchronize()
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.kv_append(kp, vp, k, v, case.block_tables, case.ctx_lens)
    gk, gv = cache.layer(0)
    assert np.array_equal(k_from_lib(gk.cpu().numpy()).view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(v_from_lib(gv.cpu().numpy()).view(np.uint16), vp.view(np.uint16))


def test_host_errors_enqueue_nothing(lib):
    case = inp.attention_case(2, 4, 2, 64, 1, 40, seed=17)
    cache = load_case_into_cache(lib, case)
    q = dev(case.q)
    out = torch.empty_like(q)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.PkvError, match="workspace too small"):
        lib.paged_attn_decode(cache, 0, q, out, dev(case.block_tables), dev(case.ctx_lens), 40, 0.1, small)
    with pytest.raises(lib.PkvError, match="bt_stride"):
        lib.paged_attn_decode(cache, 0, q, out, dev(case.block_tables), dev(case.ctx_lens), 4000, 0.1, small)
