// Allocation-free paged attention: pkv_paged_attn_decode with its workspace
// (per-(row, KV head) arrival counters and the partial results of rows split
// over several partitions) in a static device array instead of caller memory,
// for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in, not a device address): the array's
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept per device.  The array uses the standalone
// workspace layout (counter region sized from the array's size, partials
// behind it), so every call leaves the counters zero for the next call of any
// shape that fits.
#include <mutex>

#include "linear.h"
#include "pkv_internal.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];     // device address of `scratch` on each device
bool g_zeroed[kMaxDevices];   // counter region cleared by a call that was not captured

// The current device's scratch address (looked up on first use).
pkv_status scratch_for_current_device(void** out, int* dev_out) {
  int dev = -1;
  PKV_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return pkv::fail(PKV_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    PKV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return pkv::fail(PKV_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  *dev_out = dev;
  return PKV_OK;
}

}  // namespace

using namespace pkv;

extern "C" pkv_status pkv_paged_attn_decode_noalloc(const pkv_cache* cache, int layer, const void* q, void* out,
                                                    float* lse, const int32_t* block_tables, int bt_stride,
                                                    const int32_t* context_lens, int batch, int num_q_heads,
                                                    int max_context, float scale, pkv_stream_t stream) {
  if (!cache) return fail(PKV_E_ARG, "cache is NULL");
  if (layer < 0 || layer >= cache->desc.num_layers) return fail(PKV_E_ARG, "layer out of range");
  if (!block_tables || !context_lens) return fail(PKV_E_ARG, "block_tables / context_lens is NULL");
  if (batch < 1) return fail(PKV_E_ARG, "batch must be >= 1");
  if (max_context < 1) return fail(PKV_E_ARG, "max_context must be >= 1");
  if (max_context > kAttnMaxContext) return fail(PKV_E_UNSUPPORTED, "max_context above 262144");
  if (bt_stride < ceil_div(max_context, kBlock)) return fail(PKV_E_ARG, "bt_stride < ceil(max_context / 16)");
  if (!attn_grid_fits(batch, cache->desc.num_kv_heads, max_context)) return fail(PKV_E_UNSUPPORTED, "batch x KV heads x partitions of max_context above 2^30 workgroups");
  if (!q || !out) return fail(PKV_E_ARG, "q / out is NULL");
  const pkv_cache_desc& d = cache->desc;
  if (num_q_heads < d.num_kv_heads || num_q_heads % d.num_kv_heads)
    return fail(PKV_E_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / d.num_kv_heads > kMaxGroup) return fail(PKV_E_UNSUPPORTED, "more than 16 query heads per KV head");
  if (!(scale > 0.f)) return fail(PKV_E_ARG, "scale must be positive");
  const AttnPlan plan = attn_plan(batch, num_q_heads, d.num_kv_heads, d.head_dim, cache->elt(), max_context);
  if (!attn_ws_fits(plan, kScratchBytes))
    return fail(PKV_E_ARG, "shape needs " + std::to_string(attn_standalone_bytes(plan)) +
                               " bytes of scratch; the static scratch holds " + std::to_string(kScratchBytes));
  void* ptr = nullptr;
  int dev = -1;
  pkv_status st = scratch_for_current_device(&ptr, &dev);
  if (st != PKV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t region = attn_counter_region(kScratchBytes);
  {
    // The counters must be zero before the first call; every call leaves them
    // zero.  Cleared with a kernel on the caller's stream (no memset node if
    // the stream is being captured).  A captured first call keeps the clear in
    // its graph and the next uncaptured call clears again.
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_zeroed[dev]) {
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      PKV_HIP(hipStreamIsCapturing(s, &cap));
      PKV_HIP(launch_zero_i32(static_cast<int*>(ptr), (int)(region / sizeof(int)), s));
      if (cap == hipStreamCaptureStatusNone) g_zeroed[dev] = true;
    }
  }
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
  a.ws = ptr;
  a.counter_region = region;
  PKV_HIP(launch_paged_attention(a, plan, s));
  return PKV_OK;
}
