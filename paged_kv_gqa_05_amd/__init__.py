"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every call forwards torch tensors' device addresses and the current HIP
stream to the C ABI; all arithmetic runs in the library's HIP kernels.  Import
fails loudly when libpkv.so has not been built.
"""
import ctypes as C

import torch

from . import _abi
from ._abi import CacheDesc, ModelDesc, LayerWeights, PkvError

_lib = _abi.load()

KV_F16 = 0
KV_FP8_E4M3 = 1
BLOCK_SIZE = 16


def _check(status):
    if status != 0:
        raise PkvError(status, _lib.pkv_last_error().decode())


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


def lib():
    return _lib


def _destroy(fn_name, obj):
    # also called from __del__ at interpreter exit, when the module's globals
    # may already be None (callers bind this function as a default argument)
    h = getattr(obj, "handle", None)
    if h and _lib is not None:
        getattr(_lib, fn_name)(h)
    obj.handle = None


# ------------------------------------------------------------------ KV cache

class KVCache:
    """A paged KV cache in one torch-owned device buffer (layout in pkv.h)."""

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, dtype=KV_F16,
                 k_scales=None, v_scales=None, device="cuda"):
        self.desc = CacheDesc(num_layers, num_blocks, BLOCK_SIZE, num_kv_heads, head_dim, dtype)
        n = C.c_size_t()
        _check(_lib.pkv_cache_bytes(C.byref(self.desc), C.byref(n)))
        self.nbytes = n.value
        self.mem = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        ks = vs = None
        if dtype == KV_FP8_E4M3:
            ks = (C.c_float * num_layers)(*[float(x) for x in k_scales])
            vs = (C.c_float * num_layers)(*[float(x) for x in v_scales])
        h = C.c_void_p()
        _check(_lib.pkv_kv_cache_create(C.byref(self.desc), _p(self.mem), self.nbytes, ks, vs, C.byref(h)))
        self.handle = h
        self.num_layers, self.num_blocks = num_layers, num_blocks
        self.num_kv_heads, self.head_dim, self.dtype = num_kv_heads, head_dim, dtype

    def layer(self, layer):
        """Views of one layer's pools in the library layout (include/pkv.h):
        K [NB, Hkv, D/c, 16, c] with c = 8 (f16) or 16 (fp8); V [NB, Hkv, D, 16]
        (f16) or [NB, Hkv, D/64, 4, 16, 4, 4] (fp8: dim group, token quad, dim
        in group, dim step of 16, token in quad)."""
        k, v = C.c_void_p(), C.c_void_p()
        _check(_lib.pkv_kv_cache_layer(self.handle, layer, C.byref(k), C.byref(v)))
        tdt = torch.uint8 if self.dtype == KV_FP8_E4M3 else torch.float16
        elt = 1 if self.dtype == KV_FP8_E4M3 else 2
        n = self.num_blocks * self.num_kv_heads * BLOCK_SIZE * self.head_dim * elt
        base = self.mem.data_ptr()
        kt = self.mem[k.value - base:k.value - base + n].view(tdt)
        vt = self.mem[v.value - base:v.value - base + n].view(tdt)
        nb, hkv, d = self.num_blocks, self.num_kv_heads, self.head_dim
        c = 16 if self.dtype == KV_FP8_E4M3 else 8
        if self.dtype == KV_FP8_E4M3:
            return kt.view(nb, hkv, d // c, BLOCK_SIZE, c), vt.view(nb, hkv, d // 64, 4, 16, 4, 4)
        return kt.view(nb, hkv, d // c, BLOCK_SIZE, c), vt.view(nb, hkv, d, BLOCK_SIZE)

    def close(self, _destroy=_destroy):
        _destroy("pkv_kv_cache_destroy", self)

    __del__ = close


def kv_append(cache, layer, k, v, block_tables, context_lens, stream=None):
    _need(k, torch.float16, "k")
    _need(v, torch.float16, "v")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    _check(_lib.pkv_kv_append(cache.handle, layer, _p(k), _p(v), _p(block_tables), block_tables.shape[1],
                              _p(context_lens), context_lens.shape[0], _stream(stream)))


def attn_workspace_bytes(cache, batch, num_q_heads, max_context):
    n = C.c_size_t()
    _check(_lib.pkv_attn_workspace_bytes(cache.handle, batch, num_q_heads, max_context, C.byref(n)))
    return n.value


def attn_workspace(cache, batch, num_q_heads, max_context, device="cuda"):
    """A zero-filled attention workspace (its arrival counters must start at zero)."""
    return torch.zeros(attn_workspace_bytes(cache, batch, num_q_heads, max_context), dtype=torch.uint8,
                       device=device)


def paged_attn_decode(cache, layer, q, out, block_tables, context_lens, max_context, scale,
                      workspace, lse=None, stream=None):
    _need(q, torch.float16, "q")
    _need(out, torch.float16, "out")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(_lib.pkv_paged_attn_decode(cache.handle, layer, _p(q), _p(out), _p(lse), _p(block_tables),
                                      block_tables.shape[1], _p(context_lens), q.shape[0], q.shape[1],
                                      max_context, float(scale), _p(workspace), workspace.numel(),
                                      _stream(stream)))


def debug_attn_merge_wait(ticks):
    """Testing hook (process-wide): how long, in 100 MHz wall-clock ticks, the
    first partition of a multi-partition row waits for the others before it
    publishes its partial (default 10000; 0 publishes at once)."""
    _check(_lib.pkv_debug_attn_merge_wait(int(ticks)))


def debug_attn_worklist(enable):
    """Testing hook (process-wide): whether attention calls of several rounds of
    workgroups run in work-list form (default True) or as the direct grid."""
    _check(_lib.pkv_debug_attn_worklist(int(enable)))


def paged_attn_decode_noalloc(cache, layer, q, out, block_tables, context_lens, max_context, scale, lse=None,
                              stream=None):
    """paged_attn_decode with the library's static per-GPU scratch instead of a
    workspace (allocates nothing; calls on one GPU must not overlap)."""
    _need(q, torch.float16, "q")
    _need(out, torch.float16, "out")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(_lib.pkv_paged_attn_decode_noalloc(cache.handle, layer, _p(q), _p(out), _p(lse), _p(block_tables),
                                              block_tables.shape[1], _p(context_lens), q.shape[0], q.shape[1],
                                              max_context, float(scale), _stream(stream)))


# --------------------------------------------------------------------- model

class Model:
    """Borrows f16 device weights (dict as made by pkv_inputs.model_weights, on device)."""

    def __init__(self, shape, weights, max_positions):
        self.shape = shape
        self.weights = weights  # keep the tensors alive
        self.desc = ModelDesc(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                              shape.vocab, len(weights["layers"]), max_positions,
                              float(shape.rms_eps), float(shape.rope_theta))
        arr = (LayerWeights * len(weights["layers"]))()
        for i, lw in enumerate(weights["layers"]):
            arr[i] = LayerWeights(lw["w_in"].data_ptr(), lw["w_qkv"].data_ptr(),
                                  lw["b_qkv"].data_ptr() if lw.get("b_qkv") is not None else None,
                                  lw["w_o"].data_ptr(), lw["w_post"].data_ptr(),
                                  lw["w_gate_up"].data_ptr(), lw["w_down"].data_ptr())
        h = C.c_void_p()
        _check(_lib.pkv_model_create(C.byref(self.desc), _p(weights["embed"]), arr,
                                     _p(weights["w_final_norm"]), _p(weights["w_lm_head"]), C.byref(h)))
        self.handle = h

    def set_persistent_batch1(self, enable):
        """Run batch-1 decode steps as one persistent kernel or one kernel per
        fused op (the default; both give the same bits)."""
        _check(_lib.pkv_model_set_option(self.handle, 0, 1 if enable else 0))

    def close(self, _destroy=_destroy):
        _destroy("pkv_model_destroy", self)

    __del__ = close


def step_workspace_bytes(model, cache, batch, max_context):
    n = C.c_size_t()
    _check(_lib.pkv_step_workspace_bytes(model.handle, cache.handle, batch, max_context, C.byref(n)))
    return n.value


def decode_layer(model, cache, layer, hidden, block_tables, context_lens, max_context, workspace,
                 stream=None):
    _need(hidden, torch.float16, "hidden")
    _check(_lib.pkv_decode_layer(model.handle, cache.handle, layer, _p(hidden), _p(block_tables),
                                 block_tables.shape[1], _p(context_lens), hidden.shape[0], max_context,
                                 _p(workspace), workspace.numel(), _stream(stream)))


def decode_layer_xr(model, cache, layer, x, residual, block_tables, context_lens, max_context, workspace,
                    stream=None):
    """The layer in (x, residual) form: residual = f16(residual + x), the
    layer up to the attention sub-block's residual add (left in residual),
    x = the MLP output (not yet added)."""
    _need(x, torch.float16, "x")
    _need(residual, torch.float16, "residual")
    _check(_lib.pkv_decode_layer_xr(model.handle, cache.handle, layer, _p(x), _p(residual), _p(block_tables),
                                    block_tables.shape[1], _p(context_lens), x.shape[0], max_context,
                                    _p(workspace), workspace.numel(), _stream(stream)))


OP_QKV, OP_ATTN, OP_O, OP_GATE_UP, OP_DOWN = range(5)


def layer_op(model, cache, layer, op, hidden, block_tables, context_lens, max_context, workspace, stream=None):
    """One fused op of a decoder layer (OP_QKV .. OP_DOWN; in that order they
    are decode_layer).  The workspace must start zero-filled."""
    _need(hidden, torch.float16, "hidden")
    _check(_lib.pkv_layer_op(model.handle, cache.handle, layer, int(op), _p(hidden), _p(block_tables),
                             block_tables.shape[1], _p(context_lens), hidden.shape[0], max_context,
                             _p(workspace), workspace.numel(), _stream(stream)))


def decode_step(model, cache, token_ids, block_tables, context_lens, max_context, logits, workspace,
                hidden_out=None, stream=None):
    _need(token_ids, torch.int32, "token_ids")
    _need(logits, torch.float16, "logits")
    _check(_lib.pkv_decode_step(model.handle, cache.handle, _p(token_ids), _p(block_tables),
                                block_tables.shape[1], _p(context_lens), token_ids.shape[0], max_context,
                                _p(logits), _p(hidden_out), _p(workspace), workspace.numel(),
                                _stream(stream)))


def prefill_workspace_bytes(model, cache, n_tokens, n_seqs, max_context):
    n = C.c_size_t()
    _check(_lib.pkv_prefill_workspace_bytes(model.handle, cache.handle, n_tokens, n_seqs, max_context,
                                            C.byref(n)))
    return n.value


def prefill(model, cache, token_ids, seq_starts, prior_lens, block_tables, max_context, logits, workspace,
            stream=None):
    """Prefill the new tokens of every sequence (concatenated in token_ids,
    sequence s = token_ids[seq_starts[s]:seq_starts[s+1]], continuing after
    prior_lens[s] cached tokens); logits [S, V] of each last new token."""
    for t, n in ((token_ids, "token_ids"), (seq_starts, "seq_starts"), (prior_lens, "prior_lens"),
                 (block_tables, "block_tables")):
        _need(t, torch.int32, n)
    _need(logits, torch.float16, "logits")
    n_seqs = prior_lens.shape[0]
    if seq_starts.shape[0] != n_seqs + 1 or logits.shape[0] != n_seqs or block_tables.shape[0] != n_seqs:
        raise ValueError("seq_starts must hold n_seqs + 1 offsets; logits and block_tables n_seqs rows")
    _check(_lib.pkv_prefill(model.handle, cache.handle, _p(token_ids), _p(seq_starts), _p(prior_lens), n_seqs,
                            token_ids.shape[0], _p(block_tables), block_tables.shape[1], max_context, _p(logits),
                            _p(workspace), workspace.numel(), _stream(stream)))


def argmax(logits, tokens, context_lens=None, stream=None):
    """Greedy tokens; rows whose context length is 0 (when given) get -1."""
    _need(logits, torch.float16, "logits")
    _need(tokens, torch.int32, "tokens")
    if context_lens is not None:
        _need(context_lens, torch.int32, "context_lens")
    _check(_lib.pkv_argmax(_p(logits), logits.shape[0], logits.shape[1], _p(tokens), _p(context_lens),
                           _stream(stream)))


def stream_read(data, sink, stream=None):
    """Measurement reference: one streaming read of every byte of `data` (a
    contiguous CUDA tensor, 16-byte aligned, size a multiple of 16); `sink`
    (int32 CUDA tensor) is set to 1 only if the data hold the planted fold."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous CUDA tensor")
    _need(sink, torch.int32, "sink")
    _check(_lib.pkv_stream_read(_p(data), data.numel() * data.element_size(), _p(sink), _stream(stream)))


class Graph:
    """One captured decode step; replay() launches it on the caller's stream."""

    def __init__(self, model, cache, token_ids, block_tables, context_lens, max_context, logits,
                 workspace, hidden_out=None, capture_stream=None):
        self.keep = (model, cache, token_ids, block_tables, context_lens, logits, workspace, hidden_out)
        cs = capture_stream if capture_stream is not None else torch.cuda.Stream()
        h = C.c_void_p()
        _check(_lib.pkv_graph_capture(model.handle, cache.handle, _p(token_ids), _p(block_tables),
                                      block_tables.shape[1], _p(context_lens), token_ids.shape[0],
                                      max_context, _p(logits), _p(hidden_out), _p(workspace),
                                      workspace.numel(), C.c_void_p(cs.cuda_stream), C.byref(h)))
        self.handle = h

    def replay(self, stream=None):
        _check(_lib.pkv_graph_replay(self.handle, _stream(stream)))

    def close(self, _destroy=_destroy):
        _destroy("pkv_graph_destroy", self)

    __del__ = close


def sample(logits, temperature, top_k, top_p, uniform, tokens, context_lens=None, stream=None):
    """Sampled tokens (temperature / top-k / top-p, inverse CDF with the given
    uniforms); per-row parameter tensors on the device, [batch]."""
    _need(logits, torch.float16, "logits")
    _need(temperature, torch.float32, "temperature")
    _need(top_k, torch.int32, "top_k")
    _need(top_p, torch.float32, "top_p")
    _need(uniform, torch.float32, "uniform")
    _need(tokens, torch.int32, "tokens")
    if context_lens is not None:
        _need(context_lens, torch.int32, "context_lens")
    _check(_lib.pkv_sample(_p(logits), logits.shape[0], logits.shape[1], _p(temperature), _p(top_k), _p(top_p),
                           _p(uniform), _p(tokens), _p(context_lens), _stream(stream)))


def sample_penalized(logits, temperature, top_k, top_p, repetition, frequency, presence, uniform, counts, tokens,
                     context_lens=None, stream=None):
    """sample() after repetition / frequency / presence penalties from the
    per-row token counts [batch, vocab] (int32); logits are overwritten with
    the penalised logits and counts gain each active row's sampled token."""
    _need(logits, torch.float16, "logits")
    for t, n in ((temperature, "temperature"), (top_p, "top_p"), (repetition, "repetition"),
                 (frequency, "frequency"), (presence, "presence"), (uniform, "uniform")):
        _need(t, torch.float32, n)
    for t, n in ((top_k, "top_k"), (counts, "counts"), (tokens, "tokens")):
        _need(t, torch.int32, n)
    if counts.shape != logits.shape:
        raise ValueError("counts must have the logits' shape [batch, vocab]")
    if context_lens is not None:
        _need(context_lens, torch.int32, "context_lens")
    _check(_lib.pkv_sample_penalized(_p(logits), logits.shape[0], logits.shape[1], _p(temperature), _p(top_k),
                                     _p(top_p), _p(repetition), _p(frequency), _p(presence), _p(uniform),
                                     _p(counts), _p(tokens), _p(context_lens), _stream(stream)))


class GraphSet:
    """One captured decode step per batch-size bucket over shared buffers sized
    for the largest bucket; replay(n) runs rows [0, n) in the smallest bucket
    >= n with the padding rows made inactive, and returns that bucket."""

    def __init__(self, model, cache, buckets, token_ids, block_tables, context_lens, max_context, logits,
                 workspace, hidden_out=None, capture_stream=None):
        self.keep = (model, cache, token_ids, block_tables, context_lens, logits, workspace, hidden_out)
        self.buckets = sorted(int(b) for b in buckets)
        cs = capture_stream if capture_stream is not None else torch.cuda.Stream()
        arr = (C.c_int32 * len(self.buckets))(*self.buckets)
        h = C.c_void_p()
        _check(_lib.pkv_graph_set_capture(model.handle, cache.handle, arr, len(self.buckets), _p(token_ids),
                                          _p(block_tables), block_tables.shape[1], _p(context_lens), max_context,
                                          _p(logits), _p(hidden_out), _p(workspace), workspace.numel(),
                                          C.c_void_p(cs.cuda_stream), C.byref(h)))
        self.handle = h

    def replay(self, batch, stream=None):
        bk = C.c_int(0)
        _check(_lib.pkv_graph_set_replay(self.handle, int(batch), _stream(stream), C.byref(bk)))
        return bk.value

    def close(self, _destroy=_destroy):
        _destroy("pkv_graph_set_destroy", self)

    __del__ = close


# ------------------------------------------------------------ host allocator

class BlockAllocator:
    def __init__(self, num_blocks, seed=0):
        h = C.c_void_p()
        _check(_lib.pkv_alloc_create(num_blocks, seed, C.byref(h)))
        self.handle = h

    def grow(self, row, old_len, new_len):
        """row: a writable numpy int32 array (one block-table row)."""
        ptr = row.ctypes.data_as(C.POINTER(C.c_int32))
        _check(_lib.pkv_alloc_grow(self.handle, ptr, row.shape[0], old_len, new_len))

    def release(self, row, length):
        _check(_lib.pkv_alloc_release(self.handle, row.ctypes.data_as(C.POINTER(C.c_int32)), length))

    @property
    def free_blocks(self):
        return _lib.pkv_alloc_free_blocks(self.handle)

    def close(self, _destroy=_destroy):
        _destroy("pkv_alloc_destroy", self)

    __del__ = close


def validate_metadata(block_tables, context_lens, num_blocks, max_context):
    """Host (numpy int32) metadata check; raises PkvError on a violation."""
    bt = block_tables
    _check(_lib.pkv_validate_metadata(bt.ctypes.data_as(C.POINTER(C.c_int32)), bt.shape[1],
                                      context_lens.ctypes.data_as(C.POINTER(C.c_int32)),
                                      context_lens.shape[0], num_blocks, max_context))
