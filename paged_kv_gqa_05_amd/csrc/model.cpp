// Model object, decode layer / decode step orchestration, greedy argmax and
// hipGraph capture / replay.
//
// Per layer (rvLLM post on discuss.pytorch.kr, section "퓨즈드 CUDA 커널" for
// the fused ops; section "PagedAttention과 FlashAttention-3" for the paged GQA
// attention):
//   1. RMSNorm(h) * w_in + QKV projection + bias, RoPE of q and k, q out and
//      the new token's k and v into the cache            (one kernel)
//   2. paged GQA attention: split + merge                (two kernels)
//   3. O projection + residual add into h                (one kernel)
//   4. RMSNorm(h) * w_post + gate/up projection + SiLU*mul (one kernel)
//   5. down projection + residual add into h             (one kernel)
// The step adds the embedding gather before the layers and RMSNorm + LM head
// after them.  Section "CUDA 그래프 리플레이": the forward is captured once in
// a graph and replayed on the caller's stream; sampling (argmax) stays outside.
#include <algorithm>
#include <cmath>
#include <new>
#include <string>
#include <vector>

#include "linear.h"
#include "ops.h"
#include "pkv_internal.h"

using namespace pkv;

struct pkv_model {
  pkv_model_desc d;
  const void* embed;
  std::vector<pkv_layer_weights> layers;
  const void* w_final;
  const void* w_lm;
  void* rope;  // device float2 [max_positions][D/2]: (cos, sin)
  void* layer_table = nullptr;  // device PersistLayer [num_layers] for the persistent batch-1 step
  int persistent = 0;           // PKV_OPT_PERSISTENT_BATCH1
};

struct pkv_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

// One captured step per batch-size bucket over the same caller buffers.
struct pkv_graph_set {
  std::vector<int> buckets;  // strictly ascending
  std::vector<pkv_graph*> graphs;
  int32_t* tokens = nullptr;
  int32_t* lens = nullptr;
};

namespace {

struct StepBuffers {
  _Float16* h;    // hidden [B][H] (when the caller gives none)
  _Float16* q;    // [B][Hq][D]
  _Float16* o;    // [B][Hq][D]
  _Float16* act;  // [B][F]
  void* attn_ws;  // attention workspace; starts with its arrival counters
  void* gemm_ws;  // split-K partial tiles of the MFMA projections
  int* counters;  // split-K arrival counters, followed directly by the
                  // attention counters: n_counters ints zeroed at the start
                  // of each call
  int n_counters;
  size_t total;
};

StepBuffers carve(const pkv_model* m, int batch, const AttnPlan& plan, void* base) {
  const pkv_model_desc& d = m->d;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  StepBuffers b{};
  b.h = reinterpret_cast<_Float16*>(take((size_t)batch * d.hidden * 2));
  b.q = reinterpret_cast<_Float16*>(take((size_t)batch * d.num_q_heads * d.head_dim * 2));
  b.o = reinterpret_cast<_Float16*>(take((size_t)batch * d.num_q_heads * d.head_dim * 2));
  b.act = reinterpret_cast<_Float16*>(take((size_t)batch * d.ffn * 2));
  const int qkv_n = (d.num_q_heads + 2 * d.num_kv_heads) * d.head_dim;
  size_t g = 0;
  g = std::max(g, linear_ws_bytes(batch, qkv_n / 2, d.hidden, EPI_ROPE));
  g = std::max(g, linear_ws_bytes(batch, d.hidden, d.num_q_heads * d.head_dim, EPI_RESID));
  g = std::max(g, linear_ws_bytes(batch, d.ffn, d.hidden, EPI_SILU));
  g = std::max(g, linear_ws_bytes(batch, d.hidden, d.ffn, EPI_RESID));
  g = std::max(g, linear_ws_bytes(batch, d.vocab, d.hidden, EPI_F16));
  b.gemm_ws = take(g);
  static_assert(kGemmMaxCounters * sizeof(int) % 256 == 0, "attention counters follow the GEMM counters");
  b.counters = reinterpret_cast<int*>(take((size_t)kGemmMaxCounters * sizeof(int)));
  b.attn_ws = take(plan.ws_bytes);
  b.n_counters = kGemmMaxCounters + (int)(plan.counter_bytes / sizeof(int));
  b.total = off;
  return b;
}

int cache_elt(const pkv_cache_desc& cd) { return cd.dtype == PKV_KV_FP8_E4M3 ? 1 : 2; }

// A prefill's attention is the causal multi-token kernel, which needs none of
// the decode attention's counters or partials: its step buffers are carved
// with an empty attention workspace.
AttnPlan prefill_attn_plan() {
  AttnPlan p{};
  p.counter_bytes = 0;
  p.ws_bytes = 0;
  return p;
}

// A prefill runs the decode layers over its n_tokens new tokens as rows of
// their own; after the step buffers for that many rows come the per-token
// rows (context length, block-table copy), the last row of every sequence,
// their hidden states and the LM head's split-K scratch for n_seqs rows.
struct PrefillBuffers {
  StepBuffers sb;
  int stride_tok;
  int32_t* lens_tok;
  int32_t* bt_tok;
  int32_t* last_idx;
  int32_t* items;    // prefill attention work list: max_items int32 pairs
  int32_t* n_items;
  int max_items;
  _Float16* h_last;
  void* lm_ws;
  size_t total;
};

PrefillBuffers carve_prefill(const pkv_model* m, int n_tokens, int n_seqs, int max_context, const AttnPlan& plan,
                             void* base) {
  PrefillBuffers pb{};
  pb.sb = carve(m, n_tokens, plan, base);
  char* p = static_cast<char*>(base);
  size_t off = pb.sb.total;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  pb.stride_tok = ceil_div(max_context, kBlock);
  pb.lens_tok = reinterpret_cast<int32_t*>(take((size_t)n_tokens * 4));
  pb.bt_tok = reinterpret_cast<int32_t*>(take((size_t)n_tokens * pb.stride_tok * 4));
  pb.last_idx = reinterpret_cast<int32_t*>(take((size_t)n_seqs * 4));
  pb.max_items = prefill_max_items(n_tokens, n_seqs, m->d.num_q_heads / m->d.num_kv_heads);
  pb.items = reinterpret_cast<int32_t*>(take((size_t)pb.max_items * 8));
  pb.n_items = reinterpret_cast<int32_t*>(take(4));
  pb.h_last = reinterpret_cast<_Float16*>(take((size_t)n_seqs * m->d.hidden * 2));
  pb.lm_ws = take(linear_ws_bytes(n_seqs, m->d.vocab, m->d.hidden, EPI_F16));
  pb.total = off;
  return pb;
}

pkv_status check_step(const pkv_model* m, const pkv_cache* cache, const int32_t* bt, int bt_stride,
                      const int32_t* lens, int batch, int max_context, void* ws, size_t ws_bytes,
                      StepBuffers* bufs, AttnPlan* plan) {
  if (!m || !cache) return fail(PKV_E_ARG, "model / cache is NULL");
  const pkv_cache_desc& cd = cache->desc;
  if (cd.num_kv_heads != m->d.num_kv_heads || cd.head_dim != m->d.head_dim)
    return fail(PKV_E_ARG, "cache heads / head_dim differ from the model's");
  if (!bt || !lens) return fail(PKV_E_ARG, "block_tables / context_lens is NULL");
  if (batch < 1) return fail(PKV_E_ARG, "batch must be >= 1");
  if (max_context < 1 || max_context > m->d.max_positions)
    return fail(PKV_E_ARG, "max_context must be in [1, max_positions]");
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (bt_stride < ceil_div(max_context, kBlock)) return fail(PKV_E_ARG, "bt_stride < ceil(max_context / 16)");
  if (!attn_grid_fits(batch, cd.num_kv_heads, max_context)) return fail(PKV_E_UNSUPPORTED, "batch x KV heads x partitions of max_context above 2^30 workgroups");
  *plan = attn_plan(batch, m->d.num_q_heads, m->d.num_kv_heads, m->d.head_dim, cache_elt(cd), max_context);
  const StepBuffers need = carve(m, batch, *plan, nullptr);
  if (!ws || ws_bytes < need.total)
    return fail(PKV_E_ARG, "workspace too small: need " + std::to_string(need.total) + " bytes");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(PKV_E_ARG, "workspace must be 256-byte aligned");
  *bufs = carve(m, batch, *plan, ws);
  return PKV_OK;
}

// Arguments of fused op `op` (PKV_OP_QKV, _O, _GATE_UP, _DOWN) of a layer.
LinArgs layer_lin_args(const pkv_model* m, const pkv_cache* cache, int layer, int op, _Float16* h,
                       const int32_t* bt, int bt_stride, const int32_t* lens, int batch, const StepBuffers& sb) {
  const pkv_model_desc& d = m->d;
  const pkv_layer_weights& w = m->layers[layer];
  const int qkv_n = (d.num_q_heads + 2 * d.num_kv_heads) * d.head_dim;
  const int qd = d.num_q_heads * d.head_dim;
  const bool fp8 = cache->desc.dtype == PKV_KV_FP8_E4M3;
  LinArgs a{};
  a.eps = d.rms_eps;
  a.M = batch;
  switch (op) {
    case PKV_OP_QKV:  // RMSNorm + QKV (+ bias) + RoPE; q out, k and v of the new token into the cache
      a.A = h; a.lda = d.hidden; a.K = d.hidden;
      a.W = static_cast<const _Float16*>(w.w_qkv);
      a.gain = static_cast<const _Float16*>(w.w_in); a.norm = 1;
      a.bias = static_cast<const _Float16*>(w.b_qkv);
      a.n_out = qkv_n / 2;  // rotation pairs (i, i + D/2) of every head
      a.rope.cos_sin = static_cast<const float2*>(m->rope);
      a.rope.lens = lens; a.rope.bt = bt; a.rope.bt_stride = bt_stride;
      a.rope.q_out = sb.q;
      a.rope.k_pool = cache->k_pool(layer); a.rope.v_pool = cache->v_pool(layer);
      a.rope.hq = d.num_q_heads; a.rope.hkv = d.num_kv_heads; a.rope.d = d.head_dim;
      a.rope.fp8 = fp8;
      a.rope.k_scale = fp8 ? cache->k_scales[layer] : 1.f;
      a.rope.v_scale = fp8 ? cache->v_scales[layer] : 1.f;
      a.rope.num_blocks = cache->desc.num_blocks;
      a.rope.max_pos = d.max_positions;
      break;
    case PKV_OP_O:  // O projection + residual add
      a.A = sb.o; a.lda = qd; a.K = qd;
      a.W = static_cast<const _Float16*>(w.w_o);
      a.out = h; a.ldo = d.hidden; a.n_out = d.hidden;
      break;
    case PKV_OP_GATE_UP:  // RMSNorm + gate/up + SiLU*mul -> act
      a.A = h; a.lda = d.hidden; a.K = d.hidden;
      a.W = static_cast<const _Float16*>(w.w_gate_up);
      a.gain = static_cast<const _Float16*>(w.w_post); a.norm = 1;
      a.out = sb.act; a.ldo = d.ffn; a.n_out = d.ffn;
      break;
    default:  // PKV_OP_DOWN: down projection + residual add
      a.A = sb.act; a.lda = d.ffn; a.K = d.ffn;
      a.W = static_cast<const _Float16*>(w.w_down);
      a.out = h; a.ldo = d.hidden; a.n_out = d.hidden;
      break;
  }
  return a;
}

AttnArgs layer_attn_args(const pkv_model* m, const pkv_cache* cache, int layer, const int32_t* bt, int bt_stride,
                         const int32_t* lens, int batch, const StepBuffers& sb) {
  const pkv_model_desc& d = m->d;
  const bool fp8 = cache->desc.dtype == PKV_KV_FP8_E4M3;
  AttnArgs at{};
  at.k_pool = cache->k_pool(layer); at.v_pool = cache->v_pool(layer); at.q = sb.q; at.out = sb.o; at.lse = nullptr;
  at.bt = bt; at.bt_stride = bt_stride; at.lens = lens; at.batch = batch;
  at.hq = d.num_q_heads; at.hkv = d.num_kv_heads; at.head_dim = d.head_dim; at.fp8 = fp8;
  at.num_blocks = cache->desc.num_blocks;
  at.scale = 1.0f / std::sqrt((float)d.head_dim);
  at.k_scale = fp8 ? cache->k_scales[layer] : 1.f;
  at.v_scale = fp8 ? cache->v_scales[layer] : 1.f;
  at.ws = sb.attn_ws;
  return at;
}

// One of the layer's five fused ops (PKV_OP_*).  pre (prefill only):
// attention runs as the causal multi-token kernel over the new tokens'
// sequences instead of one decode row per token.
hipError_t run_layer_op(const pkv_model* m, pkv_cache* cache, int layer, int op, _Float16* h, const int32_t* bt,
                        int bt_stride, const int32_t* lens, int batch, const StepBuffers& sb, const AttnPlan& plan,
                        hipStream_t s, const PrefillAttnArgs* pre = nullptr) {
  static const int kEpi[5] = {EPI_ROPE, -1, EPI_RESID, EPI_SILU, EPI_RESID};
  if (op < PKV_OP_QKV || op > PKV_OP_DOWN) return hipErrorInvalidValue;
  if (op != PKV_OP_ATTN)
    return launch_linear(layer_lin_args(m, cache, layer, op, h, bt, bt_stride, lens, batch, sb), kEpi[op],
                         sb.gemm_ws, sb.counters, s);
  const AttnArgs at = layer_attn_args(m, cache, layer, bt, bt_stride, lens, batch, sb);
  if (pre) {
    PrefillAttnArgs pa = *pre;
    pa.k_pool = at.k_pool; pa.v_pool = at.v_pool; pa.q = sb.q; pa.out = sb.o;
    pa.hq = at.hq; pa.hkv = at.hkv; pa.head_dim = at.head_dim; pa.fp8 = at.fp8;
    pa.scale = at.scale; pa.k_scale = at.k_scale; pa.v_scale = at.v_scale;
    pa.num_blocks = at.num_blocks;
    return launch_prefill_attention(pa, s);
  }
  return launch_paged_attention(at, plan, s);
}

// The batch-1 step's layers as one persistent kernel when the shapes fit its
// variants and the model allows it (false: run the per-op kernels).
bool persistent_args(const pkv_model* m, pkv_cache* cache, _Float16* h, const int32_t* bt, int bt_stride,
                     const int32_t* lens, int batch, const StepBuffers& sb, const AttnPlan& plan, PersistArgs* pa) {
  if (batch != 1 || !m->persistent || !m->layer_table) return false;
  pa->qkv = layer_lin_args(m, cache, 0, PKV_OP_QKV, h, bt, bt_stride, lens, batch, sb);
  pa->o = layer_lin_args(m, cache, 0, PKV_OP_O, h, bt, bt_stride, lens, batch, sb);
  pa->gu = layer_lin_args(m, cache, 0, PKV_OP_GATE_UP, h, bt, bt_stride, lens, batch, sb);
  pa->down = layer_lin_args(m, cache, 0, PKV_OP_DOWN, h, bt, bt_stride, lens, batch, sb);
  pa->attn = layer_attn_args(m, cache, 0, bt, bt_stride, lens, batch, sb);
  pa->plan = plan;
  pa->layers = static_cast<const PersistLayer*>(m->layer_table);
  pa->pool_stride = 2 * cache->pool_bytes;
  pa->v_off = cache->pool_bytes;
  pa->k_scales = cache->k_scales.empty() ? nullptr : cache->k_scales.data();
  pa->v_scales = cache->v_scales.empty() ? nullptr : cache->v_scales.data();
  pa->n_layers = m->d.num_layers;
  pa->barrier = reinterpret_cast<unsigned*>(sb.counters);  // split-K counters: unused by the batch-1 GEMV
  int c1 = 0, c2 = 0;
  return persistent_config(*pa, &c1, &c2);
}

hipError_t run_layer(const pkv_model* m, pkv_cache* cache, int layer, _Float16* h, const int32_t* bt,
                     int bt_stride, const int32_t* lens, int batch, const StepBuffers& sb,
                     const AttnPlan& plan, hipStream_t s, const PrefillAttnArgs* pre = nullptr) {
  for (int op = PKV_OP_QKV; op <= PKV_OP_DOWN; ++op) {
    const hipError_t e = run_layer_op(m, cache, layer, op, h, bt, bt_stride, lens, batch, sb, plan, s, pre);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t run_step(const pkv_model* m, pkv_cache* cache, const int32_t* tokens, const int32_t* bt,
                    int bt_stride, const int32_t* lens, int batch, void* logits, _Float16* h,
                    const StepBuffers& sb, const AttnPlan& plan, hipStream_t s) {
  const pkv_model_desc& d = m->d;
  hipError_t e = launch_embed(m->embed, d.vocab, tokens, h, batch, d.hidden, sb.counters, sb.n_counters, s);
  if (e != hipSuccess) return e;
  PersistArgs pa{};
  if (persistent_args(m, cache, h, bt, bt_stride, lens, batch, sb, plan, &pa)) {
    e = launch_persistent_layers(pa, s);
    if (e != hipSuccess) return e;
  } else {
    for (int l = 0; l < d.num_layers; ++l) {
      e = run_layer(m, cache, l, h, bt, bt_stride, lens, batch, sb, plan, s);
      if (e != hipSuccess) return e;
    }
  }
  LinArgs a{};
  a.eps = d.rms_eps;
  a.A = h; a.lda = d.hidden; a.K = d.hidden; a.M = batch;
  a.W = static_cast<const _Float16*>(m->w_lm);
  a.gain = static_cast<const _Float16*>(m->w_final); a.norm = 1;
  a.out = logits; a.ldo = d.vocab; a.n_out = d.vocab;
  return launch_linear(a, EPI_F16, sb.gemm_ws, sb.counters, s);
}

}  // namespace

extern "C" {

pkv_status pkv_model_create(const pkv_model_desc* desc, const void* embed, const pkv_layer_weights* layers,
                            const void* w_final_norm, const void* w_lm_head, pkv_model** out) {
  if (!out) return fail(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (!desc || !embed || !layers || !w_final_norm || !w_lm_head) return fail(PKV_E_ARG, "NULL argument");
  const pkv_model_desc& d = *desc;
  if (d.hidden < 8 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.ffn < 8 || d.vocab < 1 ||
      d.num_layers < 1 || d.max_positions < 1)
    return fail(PKV_E_ARG, "model desc: sizes must be positive");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(PKV_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d.num_q_heads % d.num_kv_heads) return fail(PKV_E_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (d.num_q_heads / d.num_kv_heads > kMaxGroup) return fail(PKV_E_UNSUPPORTED, "more than 16 query heads per KV head");
  if (d.hidden % 8 || d.ffn % 8) return fail(PKV_E_UNSUPPORTED, "hidden and ffn must be multiples of 8");
  if (d.hidden > 16384 || d.ffn > 65536) return fail(PKV_E_UNSUPPORTED, "hidden <= 16384 and ffn <= 65536 required");
  if (!(d.rms_eps > 0.f) || !(d.rope_theta > 1.f)) return fail(PKV_E_ARG, "rms_eps > 0 and rope_theta > 1 required");
  for (int l = 0; l < d.num_layers; ++l) {
    const pkv_layer_weights& w = layers[l];
    if (!w.w_in || !w.w_qkv || !w.w_o || !w.w_post || !w.w_gate_up || !w.w_down)
      return fail(PKV_E_ARG, "layer " + std::to_string(l) + ": NULL weight");
  }
  pkv_model* m = new (std::nothrow) pkv_model();
  if (!m) return fail(PKV_E_NOMEM, "host allocation failed");
  m->d = d;
  m->embed = embed;
  m->layers.assign(layers, layers + d.num_layers);
  m->w_final = w_final_norm;
  m->w_lm = w_lm_head;
  // RoPE table: angle pos * theta^(-2i/D) in double, stored as f32 (cos, sin)
  const int half = d.head_dim / 2;
  std::vector<float> tab((size_t)d.max_positions * half * 2);
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow((double)d.rope_theta, -2.0 * i / d.head_dim);
    for (int p = 0; p < d.max_positions; ++p) {
      const double ang = (double)p * inv;
      tab[((size_t)p * half + i) * 2] = (float)std::cos(ang);
      tab[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  hipError_t e = hipMalloc(&m->rope, tab.size() * sizeof(float));
  if (e != hipSuccess) {
    delete m;
    return hip_fail(e, "hipMalloc(rope table)");
  }
  e = hipMemcpy(m->rope, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(m->rope);
    delete m;
    return hip_fail(e, "hipMemcpy(rope table)");
  }
  // per-layer weight pointers for the persistent batch-1 step
  std::vector<PersistLayer> lt(d.num_layers);
  for (int l = 0; l < d.num_layers; ++l) {
    const pkv_layer_weights& w = layers[l];
    lt[l] = PersistLayer{static_cast<const _Float16*>(w.w_in), static_cast<const _Float16*>(w.w_qkv),
                         static_cast<const _Float16*>(w.b_qkv), static_cast<const _Float16*>(w.w_o),
                         static_cast<const _Float16*>(w.w_post), static_cast<const _Float16*>(w.w_gate_up),
                         static_cast<const _Float16*>(w.w_down)};
  }
  e = hipMalloc(&m->layer_table, lt.size() * sizeof(PersistLayer));
  if (e == hipSuccess) e = hipMemcpy(m->layer_table, lt.data(), lt.size() * sizeof(PersistLayer), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (m->layer_table) (void)hipFree(m->layer_table);
    (void)hipFree(m->rope);
    delete m;
    return hip_fail(e, "layer table");
  }
  *out = m;
  return PKV_OK;
}

void pkv_model_destroy(pkv_model* m) {
  if (!m) return;
  if (m->rope) (void)hipFree(m->rope);
  if (m->layer_table) (void)hipFree(m->layer_table);
  delete m;
}

pkv_status pkv_model_set_option(pkv_model* m, int option, int value) {
  if (!m) return fail(PKV_E_ARG, "model is NULL");
  if (option != PKV_OPT_PERSISTENT_BATCH1) return fail(PKV_E_ARG, "unknown option");
  if (value != 0 && value != 1) return fail(PKV_E_ARG, "value must be 0 or 1");
  m->persistent = value;
  return PKV_OK;
}

pkv_status pkv_step_workspace_bytes(const pkv_model* m, const pkv_cache* cache, int batch, int max_context,
                                    size_t* bytes) {
  if (!m || !cache || !bytes) return fail(PKV_E_ARG, "NULL argument");
  if (batch < 1 || max_context < 1) return fail(PKV_E_ARG, "batch and max_context must be >= 1");
  const pkv_cache_desc& cd = cache->desc;
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (!attn_grid_fits(batch, cd.num_kv_heads, max_context)) return fail(PKV_E_UNSUPPORTED, "batch x KV heads x partitions of max_context above 2^30 workgroups");
  const AttnPlan plan =
      attn_plan(batch, m->d.num_q_heads, m->d.num_kv_heads, m->d.head_dim, cache_elt(cd), max_context);
  *bytes = carve(m, batch, plan, nullptr).total;
  return PKV_OK;
}

pkv_status pkv_decode_layer(const pkv_model* m, pkv_cache* cache, int layer, void* hidden,
                            const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                            int max_context, void* ws, size_t ws_bytes, pkv_stream_t stream) {
  StepBuffers sb{};
  AttnPlan plan{};
  pkv_status st = check_step(m, cache, bt, bt_stride, lens, batch, max_context, ws, ws_bytes, &sb, &plan);
  if (st != PKV_OK) return st;
  if (!hidden) return fail(PKV_E_ARG, "hidden is NULL");
  if (layer < 0 || layer >= m->d.num_layers || layer >= cache->desc.num_layers)
    return fail(PKV_E_ARG, "layer out of range");
  PKV_HIP(launch_zero_i32(sb.counters, sb.n_counters, static_cast<hipStream_t>(stream)));
  PKV_HIP(run_layer(m, cache, layer, static_cast<_Float16*>(hidden), bt, bt_stride, lens, batch, sb, plan,
                    static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

pkv_status pkv_decode_layer_xr(const pkv_model* m, pkv_cache* cache, int layer, void* x, void* residual,
                               const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                               int max_context, void* ws, size_t ws_bytes, pkv_stream_t stream) {
  StepBuffers sb{};
  AttnPlan plan{};
  pkv_status st = check_step(m, cache, bt, bt_stride, lens, batch, max_context, ws, ws_bytes, &sb, &plan);
  if (st != PKV_OK) return st;
  if (!x || !residual) return fail(PKV_E_ARG, "x or residual is NULL");
  if (x == residual) return fail(PKV_E_ARG, "x and residual must be different buffers");
  if (layer < 0 || layer >= m->d.num_layers || layer >= cache->desc.num_layers)
    return fail(PKV_E_ARG, "layer out of range");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  _Float16* h = static_cast<_Float16*>(residual);
  PKV_HIP(launch_add_clear(residual, x, (size_t)batch * m->d.hidden, sb.counters, sb.n_counters, s));
  for (int op = PKV_OP_QKV; op <= PKV_OP_GATE_UP; ++op)
    PKV_HIP(run_layer_op(m, cache, layer, op, h, bt, bt_stride, lens, batch, sb, plan, s));
  LinArgs a = layer_lin_args(m, cache, layer, PKV_OP_DOWN, h, bt, bt_stride, lens, batch, sb);
  a.out = x;  // zeroed above: the residual epilogue leaves f16(W_down act) in x
  PKV_HIP(launch_linear(a, EPI_RESID, sb.gemm_ws, sb.counters, s));
  return PKV_OK;
}

pkv_status pkv_layer_op(const pkv_model* m, pkv_cache* cache, int layer, int op, void* hidden,
                        const int32_t* bt, int bt_stride, const int32_t* lens, int batch, int max_context,
                        void* ws, size_t ws_bytes, pkv_stream_t stream) {
  StepBuffers sb{};
  AttnPlan plan{};
  pkv_status st = check_step(m, cache, bt, bt_stride, lens, batch, max_context, ws, ws_bytes, &sb, &plan);
  if (st != PKV_OK) return st;
  if (!hidden) return fail(PKV_E_ARG, "hidden is NULL");
  if (layer < 0 || layer >= m->d.num_layers || layer >= cache->desc.num_layers)
    return fail(PKV_E_ARG, "layer out of range");
  if (op < PKV_OP_QKV || op > PKV_OP_DOWN) return fail(PKV_E_ARG, "op must be one of PKV_OP_*");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // no counter reset here (it would add a launch to every op): the caller's
  // workspace starts zero-filled and every kernel leaves its counters zero
  PKV_HIP(run_layer_op(m, cache, layer, op, static_cast<_Float16*>(hidden), bt, bt_stride, lens, batch, sb, plan, s));
  return PKV_OK;
}

static pkv_status enqueue_step(const pkv_model* m, pkv_cache* cache, const int32_t* tokens, const int32_t* bt,
                               int bt_stride, const int32_t* lens, int batch, int max_context, void* logits,
                               void* hidden_out, void* ws, size_t ws_bytes, hipStream_t s) {
  StepBuffers sb{};
  AttnPlan plan{};
  pkv_status st = check_step(m, cache, bt, bt_stride, lens, batch, max_context, ws, ws_bytes, &sb, &plan);
  if (st != PKV_OK) return st;
  if (!tokens || !logits) return fail(PKV_E_ARG, "token_ids / logits is NULL");
  if (cache->desc.num_layers < m->d.num_layers) return fail(PKV_E_ARG, "cache has fewer layers than the model");
  _Float16* h = hidden_out ? static_cast<_Float16*>(hidden_out) : sb.h;
  PKV_HIP(run_step(m, cache, tokens, bt, bt_stride, lens, batch, logits, h, sb, plan, s));
  return PKV_OK;
}

pkv_status pkv_decode_step(const pkv_model* m, pkv_cache* cache, const int32_t* tokens, const int32_t* bt,
                           int bt_stride, const int32_t* lens, int batch, int max_context, void* logits,
                           void* hidden_out, void* ws, size_t ws_bytes, pkv_stream_t stream) {
  return enqueue_step(m, cache, tokens, bt, bt_stride, lens, batch, max_context, logits, hidden_out, ws,
                      ws_bytes, static_cast<hipStream_t>(stream));
}

pkv_status pkv_prefill_workspace_bytes(const pkv_model* m, const pkv_cache* cache, int n_tokens, int n_seqs,
                                       int max_context, size_t* bytes) {
  if (!m || !cache || !bytes) return fail(PKV_E_ARG, "NULL argument");
  if (n_tokens < 1 || n_seqs < 1 || max_context < 1)
    return fail(PKV_E_ARG, "n_tokens, n_seqs and max_context must be >= 1");
  *bytes = carve_prefill(m, n_tokens, n_seqs, max_context, prefill_attn_plan(), nullptr).total;
  return PKV_OK;
}

pkv_status pkv_prefill(const pkv_model* m, pkv_cache* cache, const int32_t* tokens, const int32_t* seq_starts,
                       const int32_t* prior_lens, int n_seqs, int n_tokens, const int32_t* bt, int bt_stride,
                       int max_context, void* logits, void* ws, size_t ws_bytes, pkv_stream_t stream) {
  if (!m || !cache) return fail(PKV_E_ARG, "model / cache is NULL");
  const pkv_cache_desc& cd = cache->desc;
  if (cd.num_kv_heads != m->d.num_kv_heads || cd.head_dim != m->d.head_dim)
    return fail(PKV_E_ARG, "cache heads / head_dim differ from the model's");
  if (cd.num_layers < m->d.num_layers) return fail(PKV_E_ARG, "cache has fewer layers than the model");
  if (!tokens || !seq_starts || !prior_lens || !bt || !logits)
    return fail(PKV_E_ARG, "token_ids / seq_starts / prior_lens / block_tables / logits is NULL");
  if (n_tokens < 1 || n_seqs < 1) return fail(PKV_E_ARG, "n_tokens and n_seqs must be >= 1");
  if (max_context < 1 || max_context > m->d.max_positions)
    return fail(PKV_E_ARG, "max_context must be in [1, max_positions]");
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (bt_stride < ceil_div(max_context, kBlock)) return fail(PKV_E_ARG, "bt_stride < ceil(max_context / 16)");
  const AttnPlan plan = prefill_attn_plan();
  const size_t need = carve_prefill(m, n_tokens, n_seqs, max_context, plan, nullptr).total;
  if (!ws || ws_bytes < need) return fail(PKV_E_ARG, "workspace too small: need " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(PKV_E_ARG, "workspace must be 256-byte aligned");
  const PrefillBuffers pb = carve_prefill(m, n_tokens, n_seqs, max_context, plan, ws);
  const StepBuffers& sb = pb.sb;
  const pkv_model_desc& d = m->d;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  PKV_HIP(launch_prefill_rows(seq_starts, prior_lens, bt, bt_stride, n_seqs, n_tokens, pb.stride_tok, max_context,
                              pb.lens_tok, pb.bt_tok, pb.last_idx, s));
  PKV_HIP(launch_embed(m->embed, d.vocab, tokens, sb.h, n_tokens, d.hidden, sb.counters, sb.n_counters, s));
  PrefillAttnArgs pre{};
  pre.seq_starts = seq_starts; pre.prior_lens = prior_lens; pre.bt = bt; pre.bt_stride = bt_stride;
  pre.items = pb.items; pre.n_items = pb.n_items; pre.max_items = pb.max_items;
  pre.n_seqs = n_seqs; pre.n_tokens = n_tokens; pre.max_context = max_context;
  PKV_HIP(launch_prefill_items(pre, d.num_q_heads / d.num_kv_heads, s));
  for (int l = 0; l < d.num_layers; ++l)
    PKV_HIP(run_layer(m, cache, l, sb.h, pb.bt_tok, pb.stride_tok, pb.lens_tok, n_tokens, sb, plan, s, &pre));
  // the last new token of every sequence -> final RMSNorm -> LM head
  PKV_HIP(launch_embed(sb.h, n_tokens, pb.last_idx, pb.h_last, n_seqs, d.hidden, sb.counters, sb.n_counters, s));
  LinArgs a{};
  a.eps = d.rms_eps;
  a.A = pb.h_last; a.lda = d.hidden; a.K = d.hidden; a.M = n_seqs;
  a.W = static_cast<const _Float16*>(m->w_lm);
  a.gain = static_cast<const _Float16*>(m->w_final); a.norm = 1;
  a.out = logits; a.ldo = d.vocab; a.n_out = d.vocab;
  PKV_HIP(launch_linear(a, EPI_F16, pb.lm_ws, sb.counters, s));
  return PKV_OK;
}

pkv_status pkv_argmax(const void* logits, int batch, int vocab, int32_t* tokens, const int32_t* context_lens,
                      pkv_stream_t stream) {
  if (!logits || !tokens) return fail(PKV_E_ARG, "NULL argument");
  if (batch < 1 || vocab < 1) return fail(PKV_E_ARG, "batch and vocab must be >= 1");
  PKV_HIP(launch_argmax(logits, batch, vocab, tokens, context_lens, static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

pkv_status pkv_stream_read(const void* data, size_t bytes, int32_t* sink, pkv_stream_t stream) {
  if (!data || !sink) return fail(PKV_E_ARG, "NULL argument");
  if (bytes == 0 || bytes % 16 != 0) return fail(PKV_E_ARG, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(data) % 16 != 0) return fail(PKV_E_ARG, "data must be 16-byte aligned");
  PKV_HIP(launch_stream_read(data, bytes, sink, static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

pkv_status pkv_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* uniform, int32_t* tokens, const int32_t* context_lens,
                      pkv_stream_t stream) {
  if (batch < 1 || vocab < 1) return fail(PKV_E_ARG, "batch and vocab must be >= 1");
  if (vocab > (1 << 24)) return fail(PKV_E_ARG, "vocab must be <= 2^24");
  if (!logits || !temperature || !top_k || !top_p || !uniform || !tokens) return fail(PKV_E_ARG, "NULL argument");
  PKV_HIP(launch_sample(logits, batch, vocab, temperature, top_k, top_p, uniform, context_lens, tokens,
                        static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

pkv_status pkv_sample_penalized(void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                                const float* top_p, const float* repetition, const float* frequency,
                                const float* presence, const float* uniform, int32_t* counts, int32_t* tokens,
                                const int32_t* context_lens, pkv_stream_t stream) {
  if (batch < 1 || vocab < 1) return fail(PKV_E_ARG, "batch and vocab must be >= 1");
  if (vocab > (1 << 24)) return fail(PKV_E_ARG, "vocab must be <= 2^24");
  if (!logits || !temperature || !top_k || !top_p || !repetition || !frequency || !presence || !uniform ||
      !counts || !tokens)
    return fail(PKV_E_ARG, "NULL argument");
  PKV_HIP(launch_sample(logits, batch, vocab, temperature, top_k, top_p, uniform, context_lens, tokens,
                        static_cast<hipStream_t>(stream), logits, counts, repetition, frequency, presence));
  return PKV_OK;
}

pkv_status pkv_graph_capture(const pkv_model* m, pkv_cache* cache, const int32_t* tokens, const int32_t* bt,
                             int bt_stride, const int32_t* lens, int batch, int max_context, void* logits,
                             void* hidden_out, void* ws, size_t ws_bytes, pkv_stream_t capture_stream,
                             pkv_graph** out) {
  if (!out) return fail(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (!capture_stream) return fail(PKV_E_ARG, "capture_stream must not be the null stream");
  hipStream_t cs = static_cast<hipStream_t>(capture_stream);
  // validate before capturing so that a bad argument leaves no open capture
  {
    StepBuffers sb{};
    AttnPlan plan{};
    pkv_status st = check_step(m, cache, bt, bt_stride, lens, batch, max_context, ws, ws_bytes, &sb, &plan);
    if (st != PKV_OK) return st;
    if (!tokens || !logits) return fail(PKV_E_ARG, "token_ids / logits is NULL");
  }
  pkv_graph* g = new (std::nothrow) pkv_graph();
  if (!g) return fail(PKV_E_NOMEM, "host allocation failed");
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    delete g;
    return hip_fail(e, "hipStreamBeginCapture");
  }
  pkv_status st = enqueue_step(m, cache, tokens, bt, bt_stride, lens, batch, max_context, logits, hidden_out,
                               ws, ws_bytes, cs);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  if (st != PKV_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    delete g;
    return st != PKV_OK ? st : hip_fail(e, "hipStreamEndCapture");
  }
  g->graph = graph;
  e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    delete g;
    return hip_fail(e, "hipGraphInstantiate");
  }
  *out = g;
  return PKV_OK;
}

pkv_status pkv_graph_replay(pkv_graph* g, pkv_stream_t stream) {
  if (!g || !g->exec) return fail(PKV_E_STATE, "graph is not instantiated");
  PKV_HIP(hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

void pkv_graph_destroy(pkv_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

void pkv_graph_set_destroy(pkv_graph_set* set) {
  if (!set) return;
  for (pkv_graph* g : set->graphs) pkv_graph_destroy(g);
  delete set;
}

pkv_status pkv_graph_set_capture(const pkv_model* m, pkv_cache* cache, const int32_t* buckets, int n_buckets,
                                 int32_t* tokens, const int32_t* bt, int bt_stride, int32_t* lens,
                                 int max_context, void* logits, void* hidden_out, void* ws, size_t ws_bytes,
                                 pkv_stream_t capture_stream, pkv_graph_set** out) {
  if (!out) return fail(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (!buckets || n_buckets < 1 || n_buckets > 64) return fail(PKV_E_ARG, "1 to 64 buckets required");
  for (int i = 0; i < n_buckets; ++i)
    if (buckets[i] < 1 || (i > 0 && buckets[i] <= buckets[i - 1]))
      return fail(PKV_E_ARG, "buckets must be positive and strictly ascending");
  for (int i = 0; i < n_buckets; ++i) {  // the workspace must serve every bucket
    size_t need = 0;
    pkv_status st = pkv_step_workspace_bytes(m, cache, buckets[i], max_context, &need);
    if (st != PKV_OK) return st;
    if (ws_bytes < need)
      return fail(PKV_E_ARG, "workspace too small for bucket " + std::to_string(buckets[i]) + ": need " +
                                 std::to_string(need) + " bytes");
  }
  pkv_graph_set* set = new (std::nothrow) pkv_graph_set();
  if (!set) return fail(PKV_E_NOMEM, "host allocation failed");
  set->buckets.assign(buckets, buckets + n_buckets);
  set->tokens = tokens;
  set->lens = lens;
  for (int i = 0; i < n_buckets; ++i) {
    pkv_graph* g = nullptr;
    pkv_status st = pkv_graph_capture(m, cache, tokens, bt, bt_stride, lens, buckets[i], max_context, logits,
                                      hidden_out, ws, ws_bytes, capture_stream, &g);
    if (st != PKV_OK) {
      pkv_graph_set_destroy(set);
      return st;
    }
    set->graphs.push_back(g);
  }
  *out = set;
  return PKV_OK;
}

pkv_status pkv_graph_set_replay(pkv_graph_set* set, int batch, pkv_stream_t stream, int* bucket_out) {
  if (!set || set->graphs.empty()) return fail(PKV_E_STATE, "graph set is not captured");
  if (batch < 1 || batch > set->buckets.back()) return fail(PKV_E_ARG, "batch outside the captured buckets");
  size_t i = 0;
  while (set->buckets[i] < batch) ++i;
  const int bk = set->buckets[i];
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bk > batch) {  // padding rows: inactive (length 0), token 0
    PKV_HIP(launch_zero_i32(set->tokens + batch, bk - batch, s));
    PKV_HIP(launch_zero_i32(set->lens + batch, bk - batch, s));
  }
  PKV_HIP(hipGraphLaunch(set->graphs[i]->exec, s));
  if (bucket_out) *bucket_out = bk;
  return PKV_OK;
}

}  // extern "C"
