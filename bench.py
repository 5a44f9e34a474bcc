"""Decode throughput of the paged-KV GQA decode step on one MI355X.

Workload (headline): the 28-layer Qwen2.5-1.5B-shaped decoder (hidden 1536,
12/2 heads, head_dim 128, FFN 8960, vocab 151936) with seeded random-init f16
weights N(0, 0.02), 256 sequences with 128-token random prompts prefilled by
teacher-forced decode steps, then greedy decode.  One timed step is the whole
hot path for one batch: the host block allocator grows block tables, the
per-step metadata (context lengths, block tables) is uploaded from pinned
staging on the stream, the captured step graph is replayed on that stream and
the greedy argmax writes the next tokens into the graph's token buffer.

Also reported (same JSON line): decode tok/s at batch 1 / 64 / 128, paged
attention alone at the 1.5B layer shape (batch 64, contexts U[128, 2048],
28 rotated pools so that every call reads HBM) and at the fp8 long-context
7B layer shape, the roofline of the dominant kernel, and the CPU oracle timed
on the host cores on a bounded sample.

    python bench.py [--gpus 1] [--steps 32] [--warmup 5]
"""
import argparse
import contextlib
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np


@contextlib.contextmanager
def no_gc():
    """A timed region with Python's cyclic garbage collector off (collected
    just before): steps are enqueued from Python, and a collection pause
    there can leave the GPU idle inside the timed region."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA, TFLOP/s
PAGES_TOKS_N256 = 40714.0  # rvLLM post, H100 1.5B table, N = 256 (other hardware)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- decode run

class DecodeRun:
    """One batch size: cache, allocator, staging ring, captured graph."""

    def __init__(self, pkv, torch, model, shape, batch, prompt_len, total_steps, seed, kv_dtype="f16"):
        self.pkv, self.torch, self.model, self.shape, self.batch = pkv, torch, model, shape, batch
        self.prompt_len = prompt_len
        self.max_context = total_steps + 1  # total_steps counts the prompt steps too
        self.stride = math.ceil(self.max_context / 16)
        need = batch * self.stride
        self.num_blocks = int(math.ceil(1.25 * need))
        if kv_dtype == "fp8":  # per-layer scales sized for |k|, |v| up to ~9
            self.cache = pkv.KVCache(shape.n_layers, self.num_blocks, shape.n_kv_heads, shape.head_dim,
                                     dtype=pkv.KV_FP8_E4M3, k_scales=[0.02] * shape.n_layers,
                                     v_scales=[0.02] * shape.n_layers)
        else:
            self.cache = pkv.KVCache(shape.n_layers, self.num_blocks, shape.n_kv_heads, shape.head_dim)
        self.alloc = pkv.BlockAllocator(self.num_blocks, seed=seed)
        rng = np.random.default_rng(seed)
        self.prompts = rng.integers(0, shape.vocab, size=(batch, prompt_len)).astype(np.int32)
        self.lens = np.zeros(batch, np.int32)
        self.bt = np.full((batch, self.stride), -1, np.int32)
        dev = "cuda"
        self.tok_d = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.lens_d = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.bt_d = torch.full((batch, self.stride), -1, dtype=torch.int32, device=dev)
        self.logits = torch.empty(batch, shape.vocab, dtype=torch.float16, device=dev)
        ws_bytes = pkv.step_workspace_bytes(model, self.cache, batch, self.max_context)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        # one pinned staging slot per step: an async copy never reads a slot
        # that a later step has already rewritten
        n_slots = total_steps + 2
        self.stage_lens = torch.empty((n_slots, batch), dtype=torch.int32).pin_memory()
        self.stage_bt = torch.empty((n_slots, batch, self.stride), dtype=torch.int32).pin_memory()
        self.stage_tok = torch.empty((n_slots, batch), dtype=torch.int32).pin_memory()
        self.slot = 0
        self.graph = pkv.Graph(model, self.cache, self.tok_d, self.bt_d, self.lens_d, self.max_context,
                               self.logits, self.ws)

    def step(self, tokens=None):
        """Grow tables, upload metadata, replay, argmax.  tokens: host ids to
        teacher-force (prompt ingestion); None = greedy from the last argmax."""
        for b in np.nonzero(self.lens % 16 == 0)[0]:
            self.alloc.grow(self.bt[b], int(self.lens[b]), int(self.lens[b]) + 1)
        self.lens += 1
        s = self.slot
        self.slot += 1
        self.stage_lens[s].numpy()[:] = self.lens
        self.stage_bt[s].numpy()[:] = self.bt
        self.lens_d.copy_(self.stage_lens[s], non_blocking=True)
        self.bt_d.copy_(self.stage_bt[s], non_blocking=True)
        if tokens is not None:
            self.stage_tok[s].numpy()[:] = tokens
            self.tok_d.copy_(self.stage_tok[s], non_blocking=True)
        self.graph.replay()
        self.pkv.argmax(self.logits, self.tok_d)

    def teacher_forced(self):
        """Prompt tokens through the decode graph, one position per step."""
        for t in range(self.prompt_len):
            self.step(self.prompts[:, t])

    def prefill(self, repeats=3):
        """All prompts in one batched prefill call (every prompt token of every
        row), then argmax of each row's last logits gives its first token.
        The call is repeated `repeats` more times (it rewrites the same cache
        slots with the same values) to time it."""
        torch, pkv = self.torch, self.pkv
        b, p = self.batch, self.prompt_len
        for r in range(b):
            self.alloc.grow(self.bt[r], 0, p)
        self.lens[:] = p
        self.bt_d.copy_(torch.from_numpy(self.bt))
        tokens = torch.from_numpy(self.prompts.reshape(-1).copy()).cuda()
        starts = torch.arange(0, (b + 1) * p, p, dtype=torch.int32, device="cuda")
        prior = torch.zeros(b, dtype=torch.int32, device="cuda")
        ws = torch.empty(pkv.prefill_workspace_bytes(self.model, self.cache, b * p, b, self.max_context),
                         dtype=torch.uint8, device="cuda")

        def call():
            pkv.prefill(self.model, self.cache, tokens, starts, prior, self.bt_d, self.max_context, self.logits, ws)

        call()
        ms = None
        if repeats:
            with no_gc():
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(repeats):
                    call()
                e1.record()
                torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / repeats
        pkv.argmax(self.logits, self.tok_d)
        torch.cuda.synchronize()
        del ws
        return ms

    def close(self):
        self.graph.close()
        self.cache.close()


OP_NAMES = ("qkv_rope_append", "attention", "o_proj_resid", "norm_gate_up_silu", "down_proj_resid")


def op_bytes_flops(shape, batch, mean_ctx, kv_elt=2):
    """Algorithmic HBM bytes and FLOPs of one launch of each fused op of one
    layer at `batch` rows: the op's weights once, its activation input and
    output, and for attention the KV of every row's context (read once per
    KV head) plus q and o."""
    h, d, f = shape.hidden, shape.head_dim, shape.ffn
    hq, hkv = shape.n_q_heads, shape.n_kv_heads
    qkv = (hq + 2 * hkv) * d
    kv = batch * mean_ctx * hkv * d * 2 * kv_elt
    return {
        "qkv_rope_append": (2 * (qkv * h + qkv + h) + batch * h * 2 + batch * hq * d * 2 + batch * 2 * hkv * d * kv_elt,
                            2 * batch * qkv * h),
        "attention": (kv + 2 * batch * hq * d * 2, 4 * batch * mean_ctx * hq * d),
        "o_proj_resid": (2 * h * hq * d + batch * hq * d * 2 + 2 * batch * h * 2, 2 * batch * h * hq * d),
        "norm_gate_up_silu": (2 * (2 * f * h + h) + batch * h * 2 + batch * f * 2, 2 * batch * 2 * f * h),
        "down_proj_resid": (2 * h * f + batch * f * 2 + 2 * batch * h * 2, 2 * batch * h * f),
    }


def time_layer_ops(pkv, torch, run, rounds=10):
    """Each fused op alone (pkv_layer_op) on the run's cache and metadata,
    cycling over every layer so that weights and KV come from HBM (28 layers
    of weights exceed the 256 MB Infinity Cache), HIP events on the stream the
    ops run on.  Returns microseconds per launch per op."""
    shape, b = run.shape, run.batch
    hidden = torch.empty(b, shape.hidden, dtype=torch.float16, device="cuda").normal_()
    ws = torch.zeros(pkv.step_workspace_bytes(run.model, run.cache, b, run.max_context), dtype=torch.uint8,
                     device="cuda")
    lens_d, bt_d = run.lens_d, run.bt_d
    for op in range(5):   # one pass in layer order fills q, o and act before the ops are timed alone
        pkv.layer_op(run.model, run.cache, 0, op, hidden, bt_d, lens_d, run.max_context, ws)
    out = {}
    stream = torch.cuda.current_stream()
    for op, name in enumerate(OP_NAMES):
        for layer in range(shape.n_layers):
            pkv.layer_op(run.model, run.cache, layer, op, hidden, bt_d, lens_d, run.max_context, ws)
        with no_gc():
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(rounds):
                for layer in range(shape.n_layers):
                    pkv.layer_op(run.model, run.cache, layer, op, hidden, bt_d, lens_d, run.max_context, ws)
            e1.record(stream)
            torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / (rounds * shape.n_layers)
        if op == 4 and not torch.isfinite(hidden).all().item():   # the residual adds keep growing hidden
            hidden.normal_()
    return out


def time_decode(pkv, torch, model, shape, batch, prompt_len, warmup, steps, seed, kv_dtype="f16",
                prompt_fill="prefill", prefill_repeats=3, ops=False, op_rounds=10):
    run = DecodeRun(pkv, torch, model, shape, batch, prompt_len, prompt_len + warmup + steps, seed, kv_dtype)
    if prompt_fill == "prefill":
        prefill_ms = run.prefill(prefill_repeats)
    else:
        run.teacher_forced()
        prefill_ms = None
    for _ in range(warmup):
        run.step()
    with no_gc():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            run.step()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    ctx_mean = float(run.lens.mean()) - steps / 2.0
    op_us = time_layer_ops(pkv, torch, run, rounds=op_rounds) if ops else None
    op_ctx = float(run.lens.mean())
    run.close()
    r = {"batch": batch, "ms_per_step": ms / steps, "tok_s": batch * steps / (ms / 1e3),
         "wall_s": wall, "mean_context": ctx_mean}
    if op_us:
        bf = op_bytes_flops(shape, batch, op_ctx, kv_elt=1 if kv_dtype == "fp8" else 2)
        r["layer_ops"] = {n: {"us_per_launch": op_us[n], "bytes": int(bf[n][0]), "flops": int(bf[n][1]),
                              "GBs": bf[n][0] / (op_us[n] * 1e-6) / 1e9,
                              "TFLOPs": bf[n][1] / (op_us[n] * 1e-6) / 1e12} for n in OP_NAMES}
        r["layer_ops_mean_context"] = op_ctx
    if prefill_ms:
        tflops = prefill_flops(shape, batch, prompt_len) / (prefill_ms / 1e3) / 1e12
        r.update({"prefill_ms": prefill_ms, "prefill_tok_s": batch * prompt_len / (prefill_ms / 1e3),
                  "prefill_tflops": tflops, "prefill_frac_of_mfma_peak": tflops / MFMA_F16_PEAK_TFLOPS})
    return r


def prefill_flops(shape, batch, prompt_len):
    """Algorithmic FLOPs of one prefill of `batch` prompts of `prompt_len`
    tokens: the projections of every token, causal attention (QK^T and PV over
    positions 0..t for token t) and the LM head of each prompt's last token."""
    h, d, f = shape.hidden, shape.head_dim, shape.ffn
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * d
    per_tok = shape.n_layers * 2 * (qkv * h + h * shape.n_q_heads * d + 2 * f * h + h * f)
    attn = shape.n_layers * 4 * shape.n_q_heads * d * (prompt_len * (prompt_len + 1) // 2)
    return batch * (prompt_len * per_tok + attn) + batch * 2 * h * shape.vocab


def step_bytes(shape, batch, mean_ctx, kv_elt=2):
    """Algorithmic HBM bytes of one decode step: weights once, the KV read for
    every row's context, the new KV written, embedding rows read, logits written
    (kv_elt: bytes per cached K/V element, 2 for f16, 1 for E4M3)."""
    h, d, f, v = shape.hidden, shape.head_dim, shape.ffn, shape.vocab
    qkv = (shape.n_q_heads + 2 * shape.n_kv_heads) * d
    per_layer_w = 2 * (h + qkv * h + qkv + h * shape.n_q_heads * d + h + 2 * f * h + h * f)
    weights = shape.n_layers * per_layer_w + 2 * (h + v * h)
    kv_tok = shape.n_layers * shape.n_kv_heads * d * 2 * kv_elt
    return weights + batch * mean_ctx * kv_tok + batch * kv_tok + batch * h * 2 + batch * v * 2


# ---------------------------------------------------------- attention alone

def time_attention(pkv, torch, w, n_pools, rounds, seed):
    """Per-call time of paged_attn_decode over n_pools rotated layer pools."""
    import pkv_inputs as inp
    rng = np.random.default_rng(w.seed)
    lens = inp.context_lengths(rng, w.batch, w.ctx_lo, w.ctx_hi, w.dist)
    mc = int(lens.max())
    bt, nb = inp.deal_block_tables(rng, lens, mc)
    fp8 = w.kv_dtype == "fp8"
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    if fp8:
        cache = pkv.KVCache(n_pools, nb, w.n_kv_heads, w.head_dim, dtype=pkv.KV_FP8_E4M3,
                            k_scales=[1.0 / 64] * n_pools, v_scales=[1.0 / 64] * n_pools)
    else:
        cache = pkv.KVCache(n_pools, nb, w.n_kv_heads, w.head_dim)
    for layer in range(n_pools):
        k, v = cache.layer(layer)
        if fp8:  # finite E4M3 codes: magnitude codes 0..0x7E, either sign
            for t in (k, v):
                t.copy_(torch.randint(0, 0x7F, t.shape, device="cuda", generator=g, dtype=torch.int32)
                        .to(torch.uint8) | (torch.randint(0, 2, t.shape, device="cuda", generator=g,
                                                          dtype=torch.int32).to(torch.uint8) << 7))
        else:
            k.normal_(generator=g)
            v.normal_(generator=g)
    q = torch.empty(w.batch, w.n_q_heads, w.head_dim, dtype=torch.float16, device="cuda").normal_(generator=g)
    out = torch.empty_like(q)
    bt_d = torch.from_numpy(bt).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    ws = pkv.attn_workspace(cache, w.batch, w.n_q_heads, mc)
    scale = 1.0 / math.sqrt(w.head_dim)

    def call(layer):
        pkv.paged_attn_decode(cache, layer, q, out, bt_d, lens_d, mc, scale, ws)

    for layer in range(n_pools):
        call(layer)
    with no_gc():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(rounds):
            for layer in range(n_pools):
                call(layer)
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (rounds * n_pools)
    elt = 1 if fp8 else 2
    kv_bytes = int(lens.sum()) * w.n_kv_heads * w.head_dim * 2 * elt
    other = 2 * q.numel() * 2 + bt.nbytes + lens.nbytes
    nbytes = kv_bytes + other
    cache.close()
    del cache, q, out, ws
    torch.cuda.empty_cache()
    # the streaming-read reference: one plain read of the same byte count per
    # call, over as many rotated buffers, timed the same way
    sr_bytes = (nbytes + 15) // 16 * 16
    bufs = torch.zeros(n_pools, sr_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(n_pools):
        pkv.stream_read(bufs[i], sink)
    with no_gc():
        torch.cuda.synchronize()
        e0.record()
        for _ in range(rounds):
            for i in range(n_pools):
                pkv.stream_read(bufs[i], sink)
        e1.record()
        torch.cuda.synchronize()
    sr_ms = e0.elapsed_time(e1) / (rounds * n_pools)
    del bufs
    torch.cuda.empty_cache()
    return {"batch": w.batch, "heads": f"{w.n_q_heads}/{w.n_kv_heads}", "head_dim": w.head_dim,
            "kv_dtype": w.kv_dtype, "sum_context": int(lens.sum()), "bytes_per_call": nbytes,
            "us_per_call": ms * 1e3, "GBs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "rotated_pools": n_pools,
            "stream_read_us_per_call": sr_ms * 1e3, "stream_read_GBs": sr_bytes / (sr_ms * 1e-3) / 1e9,
            "frac_of_stream_read": sr_ms / ms}


def time_sampling(pkv, torch, inp, batch, vocab, rounds, seed, mode):
    """Sampling after the LM head: one call over [batch, vocab] f16 logits
    shaped like a language model's (peaked rows), every row active.
    mode "mixed": temperatures 0.3-1.5 with top-k {off, 1, 5, 50, 1000} and
    top-p {1, 0.9, 0.5, 0, 0.99, 0.2} cycling over rows; "top_p": T = 0.7,
    top-p 0.9 on every row; "temperature": T = 0.7 only."""
    c = inp.sampling_case(batch, vocab, seed, masked_rows=False)
    c.lens[:] = 1
    c.temperature[c.temperature == 0] = 0.7
    if mode != "mixed":
        c.temperature[:] = 0.7
        c.top_k[:] = -1
        c.top_p[:] = 0.9 if mode == "top_p" else 1.0
    dev = lambda a: torch.from_numpy(a).cuda()
    args = [dev(x) for x in (c.logits, c.temperature, c.top_k, c.top_p, c.uniform)]
    tok = torch.empty(batch, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pkv.sample(*args, tok)
    with no_gc():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(rounds):
            pkv.sample(*args, tok)
        e1.record()
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / rounds * 1e3
    return {"batch": batch, "vocab": vocab, "mode": mode, "us_per_call": us,
            "logit_bytes": batch * vocab * 2}


ATTN_SOURCES = ("attn.hip", "attn_body.h", "coherent.h", "pkv_internal.h")
GEMM_SOURCES = ("gemm.hip", "linear.h", "linear.hip", "coherent.h", "kvstore.h", "pkv_internal.h")


def sources_sha256(files):
    """SHA-256 over the named kernel sources (in order)."""
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(here, "paged_kv_gqa_05_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(profile, files):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary under profiles/ (each counter scaled by what it reads for a device
    copy of known size), or None when the kernel's sources have changed since
    the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(here, "profiles", profile)).read()
        fields = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(("traffic_", "sources_")))
        if sources_sha256(files) != fields["sources_sha256"].strip():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def attention_traffic():
    return counted_traffic("paged_attention_attn15_counters.txt", ATTN_SOURCES)


def gate_up_traffic():
    return counted_traffic("gemm_gate_up_qwen15_b256_counters.txt", GEMM_SOURCES)


# ---------------------------------------------------------- CPU oracle leg

def host_description():
    """Host CPU as lscpu and the BLAS runtime report it."""
    import subprocess
    info = {"os_cpu_count": os.cpu_count()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k in ("Model name", "Socket(s)", "Core(s) per socket", "Thread(s) per core", "CPU(s)"):
                info[k] = v
    except Exception as e:  # no lscpu: keep what os reports
        info["lscpu_error"] = str(e)
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        info["blas"] = [{"api": p.get("internal_api"), "threads": p.get("num_threads")} for p in pools]
        info["blas_threads"] = max([p.get("num_threads", 1) for p in pools] or [1])
    except Exception:
        info["blas_threads"] = os.cpu_count()
    return info


def _host_weights(weights, layers=None):
    pick = range(len(weights["layers"])) if layers is None else layers
    return {
        "embed": weights["embed"].cpu().numpy(), "w_final_norm": weights["w_final_norm"].cpu().numpy(),
        "w_lm_head": weights["w_lm_head"].cpu().numpy(),
        "layers": [{k: (None if t is None else t.cpu().numpy()) for k, t in weights["layers"][i].items()}
                   for i in pick],
    }


def _oracle_cfg(oracle, shape, n_layers=None):
    return oracle.ModelConfig(shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                              shape.vocab, shape.n_layers if n_layers is None else n_layers, shape.rms_eps,
                              shape.rope_theta)


def cpu_baseline(torch, weights, shape, batch_sample, ctx):
    """The oracle (as it stands, default precision) running one decode step of
    the same model for the headline's rows with a pre-filled context of `ctx`
    tokens, repeated from the same state until 10 s of CPU work (at most 6)."""
    import oracle
    import pkv_inputs as inp
    host = _host_weights(weights)
    cfg = _oracle_cfg(oracle, shape)
    rng = np.random.default_rng(7)
    lens = np.full(batch_sample, ctx, np.int32)
    bt, nb = inp.deal_block_tables(rng, lens, ctx)
    valid = inp.valid_slot_masks(bt, lens - 1, nb)
    kps, vps = [], []
    for _ in range(shape.n_layers):
        k, v = inp.random_pools(rng, nb, shape.n_kv_heads, shape.head_dim, valid)
        kps.append(k)
        vps.append(v)
    toks = rng.integers(0, shape.vocab, size=batch_sample).astype(np.int32)
    reps, t0 = 0, time.perf_counter()
    while reps < 6 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        oracle.decode_step(cfg, host, kps, vps, toks, bt, lens)
        reps += 1
    dt = time.perf_counter() - t0
    hd = host_description()
    return {"value": batch_sample * reps / dt, "unit": "tok/s", "cores": int(hd["blas_threads"]), "kind": "oracle",
            "sample": f"{reps} x one oracle decode step (fp64) of the 28-layer 1.5B-shape model for "
                      f"{batch_sample} rows at context {ctx}: {dt:.1f} s",
            "host": hd}


def cpu_attention_legs():
    """The oracle's paged attention (fp64, one Python loop per row and head) on
    the seeded attn15 workload (all 64 rows) and on the first 8 of the 32 rows
    of the fp8 long-context workload; GB/s over the same algorithmic bytes as
    the GPU figures."""
    import oracle
    import pkv_inputs as inp
    legs = {}
    for name, w, rows in (("attn15", inp.ATTN15, None), ("fp8long", inp.FP8LONG, 8)):
        case = inp.workload_case(w)
        sel = slice(None) if rows is None else slice(0, rows)
        lens = case.ctx_lens[sel]
        t0 = time.perf_counter()
        oracle.paged_attention_batch(case.q[sel], case.k_pool, case.v_pool, case.block_tables[sel], lens, case.scale,
                                     k_scale=case.k_scale, v_scale=case.v_scale)
        dt = time.perf_counter() - t0
        elt = 1 if w.kv_dtype == "fp8" else 2
        nbytes = int(lens.sum()) * w.n_kv_heads * w.head_dim * 2 * elt + 2 * case.q[sel].size * 2
        legs[name] = {"s_per_call": dt, "GBs": nbytes / dt / 1e9, "rows": int(len(lens)),
                      "sample": f"one oracle call over {len(lens)} of {w.batch} rows ({int(lens.sum())} tokens)"}
        del case
    return legs


def cpu_layer_leg(torch, weights, shape, batch, ctx, name):
    """One oracle decode layer (fp64) of the model's layer 0 for `batch` rows
    at context `ctx`, plus one final norm + LM head; the step estimate is
    L x layer + head (a bounded sample of one decode step)."""
    import oracle
    import pkv_inputs as inp
    host = _host_weights(weights, layers=[0])
    cfg = _oracle_cfg(oracle, shape, 1)
    rng = np.random.default_rng(8)
    lens = np.full(batch, ctx, np.int32)
    bt, nb = inp.deal_block_tables(rng, lens, ctx)
    valid = inp.valid_slot_masks(bt, lens - 1, nb)
    k, v = inp.random_pools(rng, nb, shape.n_kv_heads, shape.head_dim, valid)
    h = rng.standard_normal((batch, shape.hidden)).astype(np.float16)
    t0 = time.perf_counter()
    oracle.decode_layer(cfg, host["layers"][0], h, k, v, bt, lens)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    n = oracle.rmsnorm(h, host["w_final_norm"], shape.rms_eps)
    (n @ host["w_lm_head"].astype(np.float64).T).astype(np.float16)
    t_head = time.perf_counter() - t0
    step = shape.n_layers * t_layer + t_head
    return {"name": name, "tok_s_estimate": batch / step, "s_per_layer": t_layer, "s_head": t_head,
            "sample": f"one oracle layer (fp64) for {batch} rows at context {ctx}, x{shape.n_layers} layers, "
                      f"+ one final norm and LM head"}


# ---------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batches", default="1,64,128,256")
    ap.add_argument("--prompt", type=int, default=128)
    ap.add_argument("--fp8-batches", default="256",
                    help="batches also timed with an E4M3 KV cache (reported beside the f16 line)")
    ap.add_argument("--attn-rounds", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-attn", action="store_true")
    ap.add_argument("--no-sample", action="store_true")
    ap.add_argument("--no-ops", action="store_true", help="skip timing the fused ops alone at the headline batch")
    ap.add_argument("--op-rounds", type=int, default=10, help="rounds over the 28 layers per fused op timed alone")
    ap.add_argument("--prompt-fill", choices=("prefill", "decode"), default="prefill",
                    help="prompts enter by one batched prefill call (timed) or one decode step per position")
    ap.add_argument("--prefill-repeats", type=int, default=3, help="timed repeats of the prefill call")
    ap.add_argument("--batches-7b", default="1,32,64,128",
                    help="batches of the 28-layer 7B-shape decode (512-token prompts), reported beside the 1.5B lines")
    ap.add_argument("--prompt-7b", type=int, default=512)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling rocprof FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_gqa_05_amd as pkv
    import pkv_inputs as inp

    torch.cuda.set_device(0)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        del src, dst
    shape = inp.QWEN15
    batches = [int(x) for x in args.batches.split(",") if x.strip()]
    head = max(batches) if batches else None
    weights = model = None
    if batches:
        log(f"generating {shape} weights on the device")
        weights = inp.model_weights_torch(shape, seed=1003)
        model = pkv.Model(shape, weights,
                          max_positions=max(4096, args.prompt + args.warmup + args.steps + 1))

    per_batch = {}
    for n in batches:
        r = time_decode(pkv, torch, model, shape, n, args.prompt, args.warmup, args.steps, seed=2003 + n,
                        prompt_fill=args.prompt_fill, prefill_repeats=args.prefill_repeats,
                        ops=(n == max(batches) and not args.no_ops), op_rounds=args.op_rounds)
        nbytes = step_bytes(shape, n, r["mean_context"])
        r["bytes_per_step"] = nbytes
        r["roofline_ms"] = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
        r["frac_of_roofline"] = r["roofline_ms"] / r["ms_per_step"]
        per_batch[n] = r
        log(f"batch {n}: {r['ms_per_step']:.3f} ms/step, {r['tok_s']:.0f} tok/s, "
            f"{100 * r['frac_of_roofline']:.1f}% of the HBM roofline")
        if "prefill_ms" in r:
            log(f"  prefill of {n} x {args.prompt} tokens: {r['prefill_ms']:.2f} ms, "
                f"{r['prefill_tok_s']:.0f} prompt tok/s, {r['prefill_tflops']:.0f} TFLOP/s")

    per_batch_fp8 = {}
    for n in ([int(x) for x in args.fp8_batches.split(",") if x.strip()] if batches else []):
        r = time_decode(pkv, torch, model, shape, n, args.prompt, args.warmup, args.steps, seed=2003 + n,
                        kv_dtype="fp8", prompt_fill=args.prompt_fill, prefill_repeats=args.prefill_repeats)
        nbytes = step_bytes(shape, n, r["mean_context"], kv_elt=1)
        r["bytes_per_step"] = nbytes
        r["roofline_ms"] = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
        r["frac_of_roofline"] = r["roofline_ms"] / r["ms_per_step"]
        per_batch_fp8[n] = r
        log(f"batch {n}, E4M3 KV cache: {r['ms_per_step']:.3f} ms/step, {r['tok_s']:.0f} tok/s")

    cpu_legs = {}
    per_batch_7b = {}
    batches_7b = [int(x) for x in args.batches_7b.split(",") if x.strip()] if batches else []
    if batches_7b:
        model.close()   # the 1.5B weights stay for the CPU baseline
        torch.cuda.empty_cache()
        shape7 = inp.QWEN7
        log(f"generating {shape7} weights on the device")
        w7 = inp.model_weights_torch(shape7, seed=1007)
        model7 = pkv.Model(shape7, w7, max_positions=max(4096, args.prompt_7b + args.warmup + args.steps + 1))
        for n in batches_7b:
            r = time_decode(pkv, torch, model7, shape7, n, args.prompt_7b, args.warmup, args.steps, seed=3007 + n,
                            prompt_fill=args.prompt_fill, prefill_repeats=1)
            nbytes = step_bytes(shape7, n, r["mean_context"])
            r["bytes_per_step"] = nbytes
            r["roofline_ms"] = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3
            r["frac_of_roofline"] = r["roofline_ms"] / r["ms_per_step"]
            per_batch_7b[n] = r
            log(f"7B batch {n}: {r['ms_per_step']:.3f} ms/step, {r['tok_s']:.0f} tok/s, "
                f"{100 * r['frac_of_roofline']:.1f}% of the HBM roofline")
        if not args.no_cpu:
            cpu_legs["full7_step"] = cpu_layer_leg(torch, w7, shape7, 8, args.prompt_7b, "7B shape, 8 rows")
            log(f"cpu oracle 7B leg: {cpu_legs['full7_step']['tok_s_estimate']:.3f} tok/s (estimate)")
        model7.close()
        del w7
        torch.cuda.empty_cache()

    attn = {}
    if not args.no_attn:
        attn["attn15"] = time_attention(pkv, torch, inp.ATTN15, 28, args.attn_rounds, seed=11)
        log(f"attn15: {attn['attn15']['us_per_call']:.2f} us/call, {attn['attn15']['GBs']:.0f} GB/s "
            f"(a streaming read of the same bytes: {attn['attn15']['stream_read_us_per_call']:.2f} us)")
        attn["fp8long"] = time_attention(pkv, torch, inp.FP8LONG, 8, args.attn_rounds, seed=12)
        log(f"fp8long: {attn['fp8long']['us_per_call']:.2f} us/call, {attn['fp8long']['GBs']:.0f} GB/s "
            f"(a streaming read of the same bytes: {attn['fp8long']['stream_read_us_per_call']:.2f} us)")

    sampling = {}
    if not args.no_sample:
        for mode in ("mixed", "top_p", "temperature"):
            r = time_sampling(pkv, torch, inp, 256, shape.vocab, 20, 13, mode)
            sampling[mode] = r
            log(f"sampling b256 {mode}: {r['us_per_call']:.1f} us/call")

    if head is None:  # profiling runs: attention only
        print(json.dumps({"attention": attn}))
        return
    h = per_batch[head]
    a = attn.get("attn15")
    roofline = roofline_attention = None
    g = (h.get("layer_ops") or {}).get("norm_gate_up_silu")
    if g:
        # the headline step's dominant kernel: its time per launch alone, weights from HBM
        roofline = {"bound": "hbm", "kernel": f"RMSNorm + gate/up projection + SiLU*mul (MFMA GEMM), 1.5B shape, "
                                              f"batch {head}: weights 2F x H f16 + hidden in + act out",
                    "achieved": round(g["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(g["GBs"] / HBM_PEAK_GBS, 4), "traffic": gate_up_traffic(),
                    "bytes_per_launch": g["bytes"], "us_per_launch": round(g["us_per_launch"], 3),
                    "flops_per_launch": g["flops"], "TFLOPs": round(g["TFLOPs"], 1),
                    "mfma_frac": round(g["TFLOPs"] / MFMA_F16_PEAK_TFLOPS, 4)}
    if a:
        roofline_attention = {"bound": "hbm", "kernel": "paged attention (split + fused merge, one kernel), "
                                                        "attn15: 1.5B layer shape, batch 64, contexts U[128, 2048]",
                              "achieved": round(a["GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(a["GBs"] / HBM_PEAK_GBS, 4), "traffic": attention_traffic(),
                              "bytes_per_launch": a["bytes_per_call"], "us_per_launch": round(a["us_per_call"], 3),
                              "stream_read_GBs": round(a["stream_read_GBs"], 1),
                              "frac_of_stream_read": round(a["frac_of_stream_read"], 4)}
    if roofline is None:
        roofline = roofline_attention
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(torch, weights, shape, head, args.prompt)
        log(f"cpu oracle: {cpu['value']:.3f} tok/s ({cpu['sample']})")
        cpu_legs.update(cpu_attention_legs())
        tiny_w = inp.model_weights_torch(inp.TINY, seed=1001)
        cpu_legs["tiny_layer"] = cpu_layer_leg(torch, tiny_w, inp.TINY, 4, 64, "tiny layer, 4 rows")
        cpu["legs"] = cpu_legs
        log("cpu oracle legs: " + ", ".join(f"{k}: {v.get('GBs', v.get('tok_s_estimate')):.3g}"
                                             for k, v in cpu_legs.items()))

    line = {
        "metric": "decode tok/s at N=1/64/128/256 + paged-attn HBM GB/s (% of 8 TB/s peak)",
        "value": round(h["tok_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(h["tok_s"] / PAGES_TOKS_N256, 3) if head == 256 else None,
        "dtype": "f16",
        "data": "synthetic: seeded random-init weights N(0,0.02), random 128-token prompts",
        "config": {"workload": f"Qwen2.5-1.5B-shape 28-layer f16 decode, batch {head}, "
                               f"{args.prompt}-token prompts, greedy, graph replay",
                   "global_batch": head, "seq_len": args.prompt + args.warmup + args.steps},
        "decode": {str(n): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                   for n, r in per_batch.items()},
        "decode_fp8_kv": {str(n): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                          for n, r in per_batch_fp8.items()},
        "decode_7b": {str(n): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                      for n, r in per_batch_7b.items()},
        "attention": attn,
        "sampling": sampling,
        "roofline": roofline,
        "roofline_attention": roofline_attention,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
