// Internal declarations shared by the host runtime and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pkv.h"

// A paged KV cache over caller-owned device memory: per layer the K pool
// followed by the V pool.  One (block, KV head) tile of K holds 16 tokens in
// 16-byte chunks: f16 [D/8][16][8], fp8 [D/16][16][16] (dims within a chunk
// contiguous); a V tile is dim-major [D][16].
struct pkv_cache {
  pkv_cache_desc desc;
  char* base;
  size_t pool_bytes;  // bytes of one K (or V) pool of one layer
  std::vector<float> k_scales, v_scales;
  int elt() const { return desc.dtype == PKV_KV_FP8_E4M3 ? 1 : 2; }
  void* k_pool(int l) const { return base + (size_t)l * 2 * pool_bytes; }
  void* v_pool(int l) const { return base + ((size_t)l * 2 + 1) * pool_bytes; }
};

namespace pkv {

constexpr int kBlock = 16;   // tokens per KV block
constexpr int kMaxGroup = 16;  // query heads per KV head handled by one MFMA tile
constexpr int kAttnMaxContext = 262144;  // 512 partitions of 512 tokens

// Thread-local error message + status helpers (host).
pkv_status fail(pkv_status st, const std::string& msg);
pkv_status hip_fail(hipError_t e, const char* what);
#define PKV_HIP(call)                                   \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return ::pkv::hip_fail(e_, #call); \
  } while (0)

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Calls whose attention could need more than 2^30 workgroups (batch x Hkv x
// the partitions of max_context at the smallest partition, 128 tokens) are
// refused, so that grid sizes and workgroup indices stay within int.
inline bool attn_grid_fits(int batch, int hkv, int max_context) {
  return (long long)batch * hkv * ceil_div(max_context, 128) <= (1LL << 30);
}

// ---------------------------------------------------------------- attention
struct AttnPlan {
  int waves;        // waves per workgroup (4 or 8)
  int nt;           // 16-token blocks per wave (2, 4 or 8)
  int part;         // tokens per partition (16 nt waves)
  int n_parts_max;  // partitions per (row, kv head) for max_context
  int grid;         // workgroups of the attention kernel
  int max_context;  // the call's max_context (longer context lengths are taken as it)
  int worklist;     // long rows over a grid of several rounds: the work-list form
  size_t counter_bytes;  // leading workspace bytes: [B][Hkv] int arrival counters and
                         // the work-list item and exit counts, zero before the first
                         // call, left zero by every call
  size_t ws_bytes;  // workspace bytes (counters + partials of multi-partition rows)
};
AttnPlan attn_plan(int batch, int hq, int hkv, int head_dim, int elt_bytes, int max_context);
// Wall-clock ticks the first partition of a row waits for the others before
// it publishes its partial (pkv_debug_attn_merge_wait; 0 = publish at once).
extern unsigned long long attn_merge_wait_ticks;
// Whether plans of the work-list form run it (pkv_debug_attn_worklist;
// default 1) or the direct grid of the same partitions.
extern int attn_worklist_enabled;

// A standalone attention workspace (pkv_paged_attn_decode) of W bytes keeps
// its arrival counters in a leading region whose size depends on W alone
// (1/64 of it in whole 256-byte units, at least 256 bytes); the partial
// results follow that region.  Every call that fits W therefore uses the same
// counter region, and the partials of one call never land on the counters of
// a later call of another shape.  A call fits when its counters fit the region
// and its partials fit behind it.
inline size_t attn_counter_region(size_t ws_bytes) {
  const size_t r = ws_bytes / 64 / 256 * 256;
  return r < 256 ? 256 : r;
}
inline size_t attn_partial_bytes(const AttnPlan& p) { return p.ws_bytes - p.counter_bytes; }
inline bool attn_ws_fits(const AttnPlan& p, size_t ws_bytes) {
  const size_t r = attn_counter_region(ws_bytes);
  return r >= p.counter_bytes && ws_bytes >= r + attn_partial_bytes(p);
}
// Smallest standalone workspace that fits the plan.
inline size_t attn_standalone_bytes(const AttnPlan& p) {
  size_t w = align_up(64 * p.counter_bytes, 256);
  const size_t part = attn_partial_bytes(p);
  if (part) w = std::max(w, align_up(part + part / 63 + 512, 256));
  while (!attn_ws_fits(p, w)) w += 256;
  return w;
}

struct AttnArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;      // f16 [B][Hq][D]
  void* out;          // f16 [B][Hq][D]
  float* lse;         // nullable [B][Hq]
  const int32_t* bt;
  int bt_stride;
  const int32_t* lens;
  int batch, hq, hkv, head_dim;
  int num_blocks;     // blocks in the pool (ids outside it are read as block 0)
  bool fp8;
  float scale;        // softmax scale
  float k_scale, v_scale;
  void* ws;           // counters, then the partials (layout of attn_plan)
  size_t counter_region;  // bytes before the partials: 0 = the plan's counter_bytes
};
hipError_t launch_paged_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s);

// ------------------------------------------------------------------ KV ops
hipError_t launch_kv_append(void* k_pool, void* v_pool, const void* k, const void* v,
                            const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                            int hkv, int head_dim, bool fp8, float k_scale, float v_scale, int num_blocks,
                            hipStream_t s);

}  // namespace pkv
