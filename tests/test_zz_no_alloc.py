"""The allocation-free attention entry point (pkv_paged_attn_decode_noalloc,
static per-GPU scratch) against the workspace entry point it mirrors, through
the C ABI: two calls in a row, the second with a smaller input, each equal to
pkv_paged_attn_decode bit for bit and within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import pkv_inputs as inp
from gpu_util import dev, load_case_into_cache, assert_parity

pytestmark = pytest.mark.gpu


def _pad(bt, b, mc):
    if bt.shape[1] * 16 < mc:
        bt = np.concatenate([bt, np.full((b, (mc + 15) // 16 - bt.shape[1]), -1, np.int32)], axis=1)
    return bt


def _both(lib, case):
    print(f"noalloc case: batch {case.q.shape[0]}, heads {case.q.shape[1]}, max_context {case.max_context}",
          flush=True)
    cache = load_case_into_cache(lib, case)
    b, hq, _ = case.q.shape
    mc = case.max_context
    q = dev(case.q)
    bt, lens = dev(_pad(case.block_tables, b, mc)), dev(case.ctx_lens)
    out_ws, out_na = torch.empty_like(q), torch.full_like(q, float("nan"))
    lse_ws = torch.empty(b, hq, dtype=torch.float32, device="cuda")
    lse_na = torch.full_like(lse_ws, float("nan"))
    ws = lib.attn_workspace(cache, b, hq, mc)
    lib.paged_attn_decode(cache, 0, q, out_ws, bt, lens, mc, case.scale, ws, lse=lse_ws)
    lib.paged_attn_decode_noalloc(cache, 0, q, out_na, bt, lens, mc, case.scale, lse=lse_na)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy(), out_na.cpu().numpy(), lse_ws.cpu().numpy(), lse_na.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls(lib):
    big = inp.workload_case(inp.ATTN15)                        # batch 64, rows of 1-2 partitions
    small = inp.attention_case(5, 12, 2, 128, 600, 2500, seed=31)   # smaller, up to 3 partitions
    for case in (big, small):
        o_ws, o_na, l_ws, l_na = _both(lib, case)
        assert np.array_equal(o_na.view(np.uint16), o_ws.view(np.uint16))
        assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32))
        ref, _ = oracle.paged_attention_batch(case.q, case.k_pool, case.v_pool, case.block_tables,
                                              case.ctx_lens, case.scale)
        assert_parity(o_na, ref, "noalloc attention")


def test_noalloc_rejects_shapes_beyond_the_scratch(lib):
    case = inp.attention_case(2, 28, 4, 128, 16, 32, seed=32)
    cache = load_case_into_cache(lib, case)
    q = torch.zeros(256, 28, 128, dtype=torch.float16, device="cuda")
    bt = torch.zeros(256, 2048, dtype=torch.int32, device="cuda")
    lens = torch.ones(256, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.PkvError, match="scratch"):
        lib.paged_attn_decode_noalloc(cache, 0, q, torch.empty_like(q), bt, lens, 32768, 0.088)
