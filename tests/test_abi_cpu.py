"""CPU tests of the C ABI: the library loads, exports every function that
include/pkv.h declares, and its host-only logic (sizes, argument checks, block
allocator, metadata validation) behaves as documented.  No GPU work is issued."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import paged_kv_gqa_05_amd as pkv
from paged_kv_gqa_05_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pkv.h")
FAKE_DEV = 0x10000000  # host-only calls never dereference device memory


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 20
    lib = C.CDLL(_abi.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(_abi.SIGNATURES), set(names) ^ set(_abi.SIGNATURES)


def _desc(**kw):
    d = dict(num_layers=2, num_blocks=10, block_size=16, num_kv_heads=2, head_dim=128, dtype=0)
    d.update(kw)
    return _abi.CacheDesc(**d)


def test_cache_bytes_and_layout():
    lib = pkv.lib()
    n = C.c_size_t()
    assert lib.pkv_cache_bytes(C.byref(_desc()), C.byref(n)) == 0
    assert n.value == 2 * 2 * 10 * 2 * 16 * 128 * 2
    assert lib.pkv_cache_bytes(C.byref(_desc(dtype=1)), C.byref(n)) == 0
    assert n.value == 2 * 2 * 10 * 2 * 16 * 128
    h = C.c_void_p()
    assert lib.pkv_kv_cache_create(C.byref(_desc()), FAKE_DEV, 2 * 2 * 10 * 2 * 16 * 128 * 2, None, None, C.byref(h)) == 0
    k, v = C.c_void_p(), C.c_void_p()
    assert lib.pkv_kv_cache_layer(h, 1, C.byref(k), C.byref(v)) == 0
    pool = 10 * 2 * 16 * 128 * 2
    assert k.value == FAKE_DEV + 2 * pool and v.value == FAKE_DEV + 3 * pool
    ws = C.c_size_t()
    assert lib.pkv_attn_workspace_bytes(h, 64, 12, 2048, C.byref(ws)) == 0 and ws.value > 0
    assert lib.pkv_attn_workspace_bytes(h, 64, 7, 2048, C.byref(ws)) == 1        # 7 % 2 != 0
    assert lib.pkv_attn_workspace_bytes(h, 64, 34, 2048, C.byref(ws)) == 2       # 17 per group
    # the attention grid bound: batch x Hkv x ceil(max_context / 128) <= 2^30
    assert lib.pkv_attn_workspace_bytes(h, (1 << 30) // (2 * 2048), 12, 262144, C.byref(ws)) == 0
    assert lib.pkv_attn_workspace_bytes(h, (1 << 30) // (2 * 2048) + 1, 12, 262144, C.byref(ws)) == 2
    assert b"2^30" in lib.pkv_last_error()
    assert lib.pkv_attn_workspace_bytes(h, 64, 12, 262145, C.byref(ws)) == 2
    lib.pkv_kv_cache_destroy(h)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(head_dim=96), 2, "head_dim"), (dict(block_size=32), 2, "block_size"),
    (dict(num_blocks=0), 1, "num_blocks"), (dict(dtype=7), 2, "dtype"),
])
def test_cache_desc_errors(kw, status, msg):
    lib = pkv.lib()
    n = C.c_size_t()
    assert lib.pkv_cache_bytes(C.byref(_desc(**kw)), C.byref(n)) == status
    assert msg in lib.pkv_last_error().decode()


def test_cache_create_errors():
    lib = pkv.lib()
    h = C.c_void_p()
    big = 1 << 30
    assert lib.pkv_kv_cache_create(C.byref(_desc()), FAKE_DEV + 8, big, None, None, C.byref(h)) == 1
    assert lib.pkv_kv_cache_create(C.byref(_desc()), FAKE_DEV, 100, None, None, C.byref(h)) == 1
    assert "too small" in lib.pkv_last_error().decode()
    assert lib.pkv_kv_cache_create(C.byref(_desc(dtype=1)), FAKE_DEV, big, None, None, C.byref(h)) == 1
    sc = (C.c_float * 2)(1.0, 0.0)
    assert lib.pkv_kv_cache_create(C.byref(_desc(dtype=1)), FAKE_DEV, big, sc, sc, C.byref(h)) == 1


def test_allocator_ascending_shuffled_and_capacity():
    a = pkv.BlockAllocator(8)
    row = np.full(4, -1, np.int32)
    a.grow(row, 0, 20)
    assert row.tolist() == [0, 1, -1, -1] and a.free_blocks == 6
    a.grow(row, 20, 32)            # still 2 blocks: nothing new
    assert row.tolist() == [0, 1, -1, -1]
    a.grow(row, 32, 33)
    assert row.tolist() == [0, 1, 2, -1]
    before = row.copy()
    with pytest.raises(pkv.PkvError, match="row too short"):
        a.grow(row, 33, 100)
    small = pkv.BlockAllocator(2)
    r2 = np.full(8, -1, np.int32)
    with pytest.raises(pkv.PkvError) as ei:
        small.grow(r2, 0, 40)
    assert ei.value.status == 4 and small.free_blocks == 2 and np.all(r2 == -1)
    assert np.array_equal(row, before)
    a.release(row, 33)
    assert a.free_blocks == 8
    with pytest.raises(pkv.PkvError, match="not in use"):
        a.release(row, 33)
    s1, s2 = pkv.BlockAllocator(50, seed=7), pkv.BlockAllocator(50, seed=7)
    x, y = np.full(4, -1, np.int32), np.full(4, -1, np.int32)
    s1.grow(x, 0, 64)
    s2.grow(y, 0, 64)
    assert np.array_equal(x, y) and x.tolist() != [0, 1, 2, 3]
    full = np.full(50, -1, np.int32)
    pkv.BlockAllocator(50, seed=9).grow(full, 0, 800)
    assert sorted(full.tolist()) == list(range(50))


def test_allocator_random_sequences_against_a_model():
    """Random grow / release sequences over many rows: the allocator never
    hands out a block twice, frees exactly the blocks a released row held,
    reports the free count of a plain Python model, and leaves rows and its
    state unchanged on every refused request."""
    rng = np.random.default_rng(11)
    nb, rows, stride = 97, 12, 10
    a = pkv.BlockAllocator(nb, seed=5)
    bt = np.full((rows, stride), -1, np.int32)
    lens = np.zeros(rows, np.int64)
    used = set()
    for _ in range(3000):
        r = int(rng.integers(rows))
        if rng.random() < 0.7:
            new = int(lens[r] + rng.integers(0, 40))
            need = (new + 15) // 16 - (int(lens[r]) + 15) // 16
            before, free = bt[r].copy(), a.free_blocks
            if new > stride * 16 or need > nb - len(used):
                with pytest.raises(pkv.PkvError):
                    a.grow(bt[r], int(lens[r]), new)
                assert np.array_equal(bt[r], before) and a.free_blocks == free
                continue
            a.grow(bt[r], int(lens[r]), new)
            fresh = bt[r, (int(lens[r]) + 15) // 16:(new + 15) // 16].tolist()
            assert not (set(fresh) & used) and len(set(fresh)) == len(fresh)
            used |= set(fresh)
            lens[r] = new
        else:
            n = (int(lens[r]) + 15) // 16
            a.release(bt[r], int(lens[r]))
            used -= set(bt[r, :n].tolist())
            bt[r] = -1
            lens[r] = 0
        assert a.free_blocks == nb - len(used)
        assert all(0 <= x < nb for x in used)


def test_validate_metadata():
    bt = np.array([[3, 1, -1], [0, 2, -1]], np.int32)
    lens = np.array([20, 17], np.int32)
    pkv.validate_metadata(bt, lens, 4, 48)
    with pytest.raises(pkv.PkvError, match="out of range"):
        pkv.validate_metadata(bt, lens, 3, 48)
    with pytest.raises(pkv.PkvError, match="used by rows"):
        pkv.validate_metadata(np.array([[3, 1, -1], [1, 2, -1]], np.int32), lens, 4, 48)
    with pytest.raises(pkv.PkvError, match="context length"):
        pkv.validate_metadata(bt, np.array([20, 49], np.int32), 4, 48)
    with pytest.raises(pkv.PkvError, match="bt_stride"):
        pkv.validate_metadata(bt, lens, 4, 49)


def test_graph_set_argument_errors():
    lib = pkv.lib()
    out = C.c_void_p()
    for buckets in ([4, 2], [0, 4], [3, 3]):
        arr = (C.c_int32 * len(buckets))(*buckets)
        assert lib.pkv_graph_set_capture(None, None, arr, len(buckets), None, None, 1, None, 16, None, None, None, 0,
                                         None, C.byref(out)) == 1
        assert b"ascending" in lib.pkv_last_error()
    assert lib.pkv_graph_set_capture(None, None, None, 0, None, None, 1, None, 16, None, None, None, 0, None,
                                     C.byref(out)) == 1
    assert lib.pkv_graph_set_replay(None, 1, None, None) == 6


def test_sample_and_prefill_argument_errors():
    """Host checks of pkv_sample and pkv_prefill reject bad sizes and NULL
    buffers before anything is enqueued (no device is touched)."""
    lib = pkv.lib()
    for batch, vocab, msg in ((0, 10, b"batch and vocab"), (2, 0, b"batch and vocab"),
                              (2, (1 << 24) + 1, b"2^24"), (2, 10, b"NULL")):
        assert lib.pkv_sample(None, batch, vocab, None, None, None, None, None, None, None) == 1
        assert msg in lib.pkv_last_error()
    n = C.c_size_t()
    assert lib.pkv_prefill_workspace_bytes(None, None, 4, 1, 16, C.byref(n)) == 1
    assert lib.pkv_prefill(None, None, None, None, None, 1, 4, None, 1, 16, None, None, 0, None) == 1
    assert b"model / cache is NULL" in lib.pkv_last_error()


def test_stream_read_argument_errors():
    """pkv_stream_read rejects NULL pointers, sizes that are not a positive
    multiple of 16 and misaligned data on the host (nothing is enqueued)."""
    lib = pkv.lib()
    sink = C.c_void_p(FAKE_DEV)
    for data, nbytes, msg in ((None, 16, b"NULL"), (FAKE_DEV, 0, b"multiple of 16"),
                              (FAKE_DEV, 24, b"multiple of 16"), (FAKE_DEV + 8, 32, b"aligned")):
        assert lib.pkv_stream_read(data, nbytes, sink, None) == 1
        assert msg in lib.pkv_last_error()
    assert lib.pkv_stream_read(FAKE_DEV, 16, None, None) == 1


def test_handle_alive_at_interpreter_exit_is_released_quietly():
    """An object still holding a native handle when the interpreter exits is
    destroyed by __del__ while the module's globals are being cleared; that
    must not raise (Python reports such errors as 'Exception ignored')."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import paged_kv_gqa_05_amd as pkv\n"
            "a = pkv.BlockAllocator(64, seed=1)\n"
            "print('ok', a.free_blocks)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok 64"
    assert "Exception ignored" not in r.stderr and "Traceback" not in r.stderr, r.stderr
