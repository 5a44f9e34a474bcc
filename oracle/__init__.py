"""Plain CPU oracle for the batched f16 paged-KV GQA decode step.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
definition that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (``paged_kv_gqa_05_amd``) never does, and this
package imports nothing from it.

Sources (cited by page title and section; the pages print no equations, no
model dimensions and no worked example, so every formula below is the plain
Llama/Qwen2 reading of what the pages name):

* rvLLM post on discuss.pytorch.kr ("rvLLM 소개"), sections
  "퓨즈드 CUDA 커널" (the three fused per-layer ops: Add+RMSNorm+QKV,
  Add+RMSNorm+GateUp, SiLU*Mul+Down), "PagedAttention과 FlashAttention-3"
  (block-table paged KV cache, GQA: query heads share KV heads, f16 KV with an
  FP8 E4M3 option), "CUDA 그래프 리플레이" (block tables and context lengths
  are per-step metadata; sampling is outside the captured forward), the
  supported-architecture table (Llama / Qwen2 decoders) and the H100 benchmark
  section (greedy decoding).
* zingnex.cn article "rvLLM：用Rust重写vLLM…", sections 直接GPU调用 (f16 GEMM
  for projections) and 支持的参数 (temperature 0 = greedy).
* aitrends.kr article 1847, glossary (용어 해설): KV cache holds past tokens'
  keys/values; PagedAttention splits it into fixed-size pages.

Precision: every function takes ``acc`` (numpy float dtype for arithmetic,
float64 by default, float32 allowed where the target asks for fp32
accumulation).  Values that cross a library call boundary (hidden state,
q/k/v stored to the cache, attention output, logits) are rounded to IEEE
binary16 with round-to-nearest-even, which is what ``numpy.float16`` does.

Parity pins (tests/test_oracle_*.py) check every function here against
invariants, closed forms and independent library routines; the end-to-end
logits of a random-weight model have no external pin ("parity unpinned by the
pages": the pages publish no logits or tokens).
"""
from .fp8 import e4m3_decode, e4m3_encode, e4m3_quantize, e4m3_table
from .sampling import apply_penalties, candidates, draw, exp_f32, sample, sample_penalized, sample_row, weight_fixed
from .decoder import (
    ModelConfig,
    rmsnorm,
    silu,
    rope,
    rope_angles,
    paged_attention,
    paged_attention_batch,
    kv_append,
    decode_layer,
    decode_layer_xr,
    decode_step,
    embed_rows,
    greedy_argmax,
    causal_forward,
    prefill,
)

__all__ = [
    "e4m3_decode", "e4m3_encode", "e4m3_quantize", "e4m3_table", "apply_penalties", "candidates", "draw",
    "exp_f32", "sample", "sample_penalized", "sample_row", "weight_fixed", "ModelConfig", "rmsnorm", "silu", "rope",
    "rope_angles", "paged_attention", "paged_attention_batch", "kv_append",
    "decode_layer", "decode_layer_xr", "decode_step", "embed_rows", "greedy_argmax", "causal_forward", "prefill",
]
