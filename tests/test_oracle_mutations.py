"""The pins catch plausible mistakes: each case plants one mistake in a copy of
an oracle function (on the CPU) and checks that an independent pin rejects it."""
import numpy as np
import pytest
import torch

import oracle.decoder as dec
import sys, os
sys.path.insert(0, os.path.dirname(__file__))
import test_oracle_model as tm


_orig_rope = dec.rope


def _rope_wrong_sign(x, pos, theta, acc=np.float64):
    # rotation by -angle instead of +angle
    return _orig_rope(x, -np.asarray(pos), theta, acc)


def _silu_wrong(x, acc=np.float64):
    return np.asarray(x, acc) / (1 + np.exp(np.asarray(x, acc)))


def _rms_no_mean(x, w, eps, acc=np.float64):
    x = np.asarray(x, acc)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, acc)


def _gather_wrong_v(k_pool, v_pool, block_row, ctx_len, block_size):
    k, v = _orig_gather(k_pool, v_pool, block_row, ctx_len, block_size)
    return k, v[::-1]          # tokens of V reversed


_orig_gather = dec.gather_sequence


def _paged_wrong_group(q, k_pool, v_pool, block_row, ctx_len, scale, **kw):
    # head h reads KV head h % Hkv instead of h // G
    hq, hkv = q.shape[0], k_pool.shape[1]
    perm = np.array([(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)])
    res = _orig_paged(q[perm], k_pool, v_pool, block_row, ctx_len, scale, **kw)
    if isinstance(res, tuple):
        return tuple(r[np.argsort(perm)] if r.ndim and r.shape[0] == hq else r for r in res)
    return res[np.argsort(perm)]


_orig_paged = dec.paged_attention


@pytest.mark.parametrize("name,fn", [
    ("rope", _rope_wrong_sign), ("silu", _silu_wrong), ("rmsnorm", _rms_no_mean),
    ("gather_sequence", _gather_wrong_v), ("paged_attention", _paged_wrong_group),
])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(dec, name, fn)
    w = tm._weights(31)
    toks = np.random.default_rng(32).integers(0, tm.SHAPE.vocab, size=29).astype(np.int32)
    full, _, _ = dec.causal_forward(tm.CFG, w, toks)
    inc, *_ = tm._run_incremental(w, toks[None], np.random.default_rng(3))
    ref = tm._torch_textbook(w, toks)
    bad_full = not np.allclose(full.astype(np.float64), ref, atol=4e-3, rtol=4e-3)
    bad_inc = not np.allclose(inc[0].astype(np.float64), ref, atol=4e-3, rtol=4e-3)
    assert bad_full or bad_inc
