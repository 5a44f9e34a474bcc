// Host side of the C ABI: errors, paged KV cache objects, the host block
// allocator, metadata validation and the attention / append entry points.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace pkv

using namespace pkv;

struct pkv_alloc {
  std::vector<int32_t> free_list;  // stack: back() is handed out first
  std::vector<uint8_t> in_use;
};

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

// --------------------------------------------------------------------- cache

static pkv_status check_desc(const pkv_cache_desc* d) {
  if (!d) return fail(PKV_E_ARG, "cache desc is NULL");
  if (d->num_layers < 1 || d->num_blocks < 1 || d->num_kv_heads < 1)
    return fail(PKV_E_ARG, "cache desc: num_layers, num_blocks and num_kv_heads must be >= 1");
  if (d->block_size != kBlock) return fail(PKV_E_UNSUPPORTED, "cache desc: block_size must be 16");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "cache desc: head_dim must be 64 or 128");
  if (d->dtype != PKV_KV_F16 && d->dtype != PKV_KV_FP8_E4M3)
    return fail(PKV_E_UNSUPPORTED, "cache desc: unknown dtype");
  return PKV_OK;
}

static size_t pool_bytes_of(const pkv_cache_desc* d) {
  const size_t elt = d->dtype == PKV_KV_FP8_E4M3 ? 1 : 2;
  return align_up((size_t)d->num_blocks * d->num_kv_heads * kBlock * d->head_dim * elt, 256);
}

pkv_status pkv_cache_bytes(const pkv_cache_desc* desc, size_t* bytes) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (!bytes) return fail(PKV_E_ARG, "bytes is NULL");
  *bytes = pool_bytes_of(desc) * 2 * (size_t)desc->num_layers;
  return PKV_OK;
}

pkv_status pkv_kv_cache_create(const pkv_cache_desc* desc, void* dev_mem, size_t bytes,
                               const float* k_scales, const float* v_scales, pkv_cache** out) {
  pkv_status st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (!out) return fail(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (!dev_mem) return fail(PKV_E_ARG, "dev_mem is NULL");
  if (reinterpret_cast<uintptr_t>(dev_mem) % 256) return fail(PKV_E_ARG, "dev_mem must be 256-byte aligned");
  size_t need = 0;
  pkv_cache_bytes(desc, &need);
  if (bytes < need)
    return fail(PKV_E_ARG, "cache memory too small: need " + std::to_string(need) + " bytes");
  const bool fp8 = desc->dtype == PKV_KV_FP8_E4M3;
  if (fp8 && (!k_scales || !v_scales)) return fail(PKV_E_ARG, "fp8 cache needs k_scales and v_scales");
  if (!fp8 && (k_scales || v_scales)) return fail(PKV_E_ARG, "f16 cache takes no scales");
  pkv_cache* c = new (std::nothrow) pkv_cache();
  if (!c) return fail(PKV_E_NOMEM, "host allocation failed");
  c->desc = *desc;
  c->base = static_cast<char*>(dev_mem);
  c->pool_bytes = pool_bytes_of(desc);
  if (fp8) {
    c->k_scales.assign(k_scales, k_scales + desc->num_layers);
    c->v_scales.assign(v_scales, v_scales + desc->num_layers);
    for (int l = 0; l < desc->num_layers; ++l) {
      if (!(c->k_scales[l] > 0.f) || !(c->v_scales[l] > 0.f)) {
        delete c;
        return fail(PKV_E_ARG, "fp8 scales must be positive and finite");
      }
    }
  }
  *out = c;
  return PKV_OK;
}

void pkv_kv_cache_destroy(pkv_cache* cache) { delete cache; }

pkv_status pkv_kv_cache_layer(const pkv_cache* cache, int layer, void** k_pool, void** v_pool) {
  if (!cache || !k_pool || !v_pool) return fail(PKV_E_ARG, "NULL argument");
  if (layer < 0 || layer >= cache->desc.num_layers) return fail(PKV_E_ARG, "layer out of range");
  *k_pool = cache->k_pool(layer);
  *v_pool = cache->v_pool(layer);
  return PKV_OK;
}

static pkv_status check_meta_args(const pkv_cache* cache, int layer, const int32_t* bt, int bt_stride,
                                  const int32_t* lens, int batch, int max_context) {
  if (!cache) return fail(PKV_E_ARG, "cache is NULL");
  if (layer < 0 || layer >= cache->desc.num_layers) return fail(PKV_E_ARG, "layer out of range");
  if (!bt || !lens) return fail(PKV_E_ARG, "block_tables / context_lens is NULL");
  if (batch < 1) return fail(PKV_E_ARG, "batch must be >= 1");
  if (max_context < 1) return fail(PKV_E_ARG, "max_context must be >= 1");
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (bt_stride < ceil_div(max_context, kBlock))
    return fail(PKV_E_ARG, "bt_stride < ceil(max_context / 16)");
  return PKV_OK;
}

pkv_status pkv_kv_append(pkv_cache* cache, int layer, const void* k, const void* v,
                         const int32_t* block_tables, int bt_stride, const int32_t* context_lens,
                         int batch, pkv_stream_t stream) {
  pkv_status st = check_meta_args(cache, layer, block_tables, bt_stride, context_lens, batch, 1);
  if (st != PKV_OK) return st;
  if (!k || !v) return fail(PKV_E_ARG, "k / v is NULL");
  const bool fp8 = cache->desc.dtype == PKV_KV_FP8_E4M3;
  PKV_HIP(launch_kv_append(cache->k_pool(layer), cache->v_pool(layer), k, v, block_tables, bt_stride,
                           context_lens, batch, cache->desc.num_kv_heads, cache->desc.head_dim, fp8,
                           fp8 ? cache->k_scales[layer] : 1.f, fp8 ? cache->v_scales[layer] : 1.f,
                           cache->desc.num_blocks, static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

// ----------------------------------------------------------------- attention

pkv_status pkv_attn_workspace_bytes(const pkv_cache* cache, int batch, int num_q_heads,
                                    int max_context, size_t* bytes) {
  if (!cache || !bytes) return fail(PKV_E_ARG, "NULL argument");
  if (batch < 1 || max_context < 1) return fail(PKV_E_ARG, "batch and max_context must be >= 1");
  const int hkv = cache->desc.num_kv_heads;
  if (num_q_heads < hkv || num_q_heads % hkv) return fail(PKV_E_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / hkv > kMaxGroup) return fail(PKV_E_UNSUPPORTED, "more than 16 query heads per KV head");
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (!attn_grid_fits(batch, hkv, max_context)) return fail(PKV_E_UNSUPPORTED, "batch x KV heads x partitions of max_context above 2^30 workgroups");
  *bytes = attn_standalone_bytes(attn_plan(batch, num_q_heads, hkv, cache->desc.head_dim, cache->elt(), max_context));
  return PKV_OK;
}

pkv_status pkv_paged_attn_decode(const pkv_cache* cache, int layer, const void* q, void* out,
                                 float* lse, const int32_t* block_tables, int bt_stride,
                                 const int32_t* context_lens, int batch, int num_q_heads,
                                 int max_context, float scale, void* workspace,
                                 size_t workspace_bytes, pkv_stream_t stream) {
  pkv_status st = check_meta_args(cache, layer, block_tables, bt_stride, context_lens, batch, max_context);
  if (st != PKV_OK) return st;
  if (!q || !out) return fail(PKV_E_ARG, "q / out is NULL");
  size_t need = 0;
  st = pkv_attn_workspace_bytes(cache, batch, num_q_heads, max_context, &need);
  if (st != PKV_OK) return st;
  const pkv_cache_desc& d = cache->desc;
  const AttnPlan plan = attn_plan(batch, num_q_heads, d.num_kv_heads, d.head_dim, cache->elt(), max_context);
  if (!workspace || !attn_ws_fits(plan, workspace_bytes))
    return fail(PKV_E_ARG, "workspace too small: need " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(PKV_E_ARG, "workspace must be 256-byte aligned");
  if (!(scale > 0.f)) return fail(PKV_E_ARG, "scale must be positive");
  AttnArgs a{};
  a.k_pool = cache->k_pool(layer);
  a.v_pool = cache->v_pool(layer);
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.lens = context_lens;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = d.num_kv_heads;
  a.head_dim = d.head_dim;
  a.num_blocks = d.num_blocks;
  a.fp8 = d.dtype == PKV_KV_FP8_E4M3;
  a.scale = scale;
  a.k_scale = a.fp8 ? cache->k_scales[layer] : 1.f;
  a.v_scale = a.fp8 ? cache->v_scales[layer] : 1.f;
  a.ws = workspace;
  a.counter_region = attn_counter_region(workspace_bytes);
  PKV_HIP(launch_paged_attention(a, plan, static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

// ------------------------------------------------------------ block allocator

// splitmix64 (Steele, Lea, Flood 2014): a small, well-known 64-bit mixer used
// here only to shuffle the free list reproducibly.
static uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

pkv_status pkv_alloc_create(int num_blocks, uint64_t seed, pkv_alloc** out) {
  if (!out) return fail(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1) return fail(PKV_E_ARG, "num_blocks must be >= 1");
  pkv_alloc* a = new (std::nothrow) pkv_alloc();
  if (!a) return fail(PKV_E_NOMEM, "host allocation failed");
  try {
    a->free_list.resize(num_blocks);
    a->in_use.assign(num_blocks, 0);
  } catch (...) {
    delete a;
    return fail(PKV_E_NOMEM, "host allocation failed");
  }
  // back() is handed out first: store descending so seed 0 gives 0, 1, 2, ...
  for (int i = 0; i < num_blocks; ++i) a->free_list[i] = num_blocks - 1 - i;
  if (seed) {
    uint64_t s = seed;
    for (int i = num_blocks - 1; i > 0; --i) {  // Fisher-Yates
      const int j = (int)(splitmix64(s) % (uint64_t)(i + 1));
      std::swap(a->free_list[i], a->free_list[j]);
    }
  }
  *out = a;
  return PKV_OK;
}

pkv_status pkv_alloc_grow(pkv_alloc* a, int32_t* row, int bt_stride, int old_len, int new_len) {
  if (!a || !row) return fail(PKV_E_ARG, "NULL argument");
  if (old_len < 0 || new_len < old_len) return fail(PKV_E_ARG, "need 0 <= old_len <= new_len");
  const int have = ceil_div(old_len, kBlock), want = ceil_div(new_len, kBlock);
  if (want > bt_stride) return fail(PKV_E_ARG, "row too short for new_len");
  const int n = want - have;
  if (n > (int)a->free_list.size())
    return fail(PKV_E_CAPACITY, "block allocator exhausted: need " + std::to_string(n) + ", free " +
                                    std::to_string(a->free_list.size()));
  for (int i = have; i < want; ++i) {
    const int32_t id = a->free_list.back();
    a->free_list.pop_back();
    a->in_use[id] = 1;
    row[i] = id;
  }
  return PKV_OK;
}

pkv_status pkv_alloc_release(pkv_alloc* a, const int32_t* row, int len) {
  if (!a || (!row && len > 0)) return fail(PKV_E_ARG, "NULL argument");
  if (len < 0) return fail(PKV_E_ARG, "len must be >= 0");
  const int n = ceil_div(len, kBlock);
  const int nb = (int)a->in_use.size();
  for (int i = 0; i < n; ++i) {  // validate first: all or nothing
    if (row[i] < 0 || row[i] >= nb || !a->in_use[row[i]])
      return fail(PKV_E_ARG, "release of a block id that is not in use: " + std::to_string(row[i]));
    for (int j = 0; j < i; ++j)
      if (row[j] == row[i]) return fail(PKV_E_ARG, "block id repeated in row");
  }
  for (int i = n - 1; i >= 0; --i) {
    a->in_use[row[i]] = 0;
    a->free_list.push_back(row[i]);
  }
  return PKV_OK;
}

int pkv_alloc_free_blocks(const pkv_alloc* a) { return a ? (int)a->free_list.size() : -1; }

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

pkv_status pkv_validate_metadata(const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                                 int num_blocks, int max_context) {
  if (!bt || !lens) return fail(PKV_E_ARG, "NULL argument");
  if (batch < 1 || num_blocks < 1 || max_context < 1) return fail(PKV_E_ARG, "sizes must be >= 1");
  if (bt_stride < ceil_div(max_context, kBlock)) return fail(PKV_E_ARG, "bt_stride < ceil(max_context / 16)");
  std::vector<int32_t> owner(num_blocks, -1);
  for (int b = 0; b < batch; ++b) {
    if (lens[b] < 0 || lens[b] > max_context)
      return fail(PKV_E_ARG, "row " + std::to_string(b) + ": context length out of [0, max_context]");
    for (int i = 0; i < ceil_div(lens[b], kBlock); ++i) {
      const int32_t id = bt[(size_t)b * bt_stride + i];
      if (id < 0 || id >= num_blocks)
        return fail(PKV_E_ARG, "row " + std::to_string(b) + ": block id out of range");
      if (owner[id] >= 0)
        return fail(PKV_E_ARG, "block " + std::to_string(id) + " used by rows " +
                                   std::to_string(owner[id]) + " and " + std::to_string(b));
      owner[id] = b;
    }
  }
  return PKV_OK;
}

}  // extern "C"
