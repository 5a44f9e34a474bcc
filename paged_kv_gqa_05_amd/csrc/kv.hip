// KV append into the block-table paged cache: each active row's new k and v
// go to the slot of position context_lens[b] - 1, as f16 or as E4M3 codes
// under the layer's scales (aitrends.kr glossary: the KV cache keeps the keys
// and values of earlier tokens; rvLLM post, section
// "PagedAttention과 FlashAttention-3": the cache is paged through block
// tables, optionally FP8 E4M3).
#include "kvstore.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ void kv_append_kernel(void* __restrict__ kpool, void* __restrict__ vpool,
                                 const _Float16* __restrict__ k, const _Float16* __restrict__ v,
                                 const int32_t* __restrict__ bt, int bt_stride,
                                 const int32_t* __restrict__ lens, int hkv, int head_dim, int fp8,
                                 float k_scale, float v_scale, int num_blocks) {
  const int b = blockIdx.x;
  const int c = lens[b];
  if (c <= 0) return;
  const int pos = c - 1;
  // a length beyond the block table or a block id outside the pool (caller
  // errors) stores nothing rather than writing outside the pool
  if (pos / kBlock >= bt_stride) return;
  const int blk = bt[(size_t)b * bt_stride + pos / kBlock];
  if ((unsigned)blk >= (unsigned)num_blocks) return;
  const int slot = pos % kBlock;
  for (int idx = threadIdx.x; idx < hkv * head_dim; idx += blockDim.x) {
    const int g = idx / head_dim, d = idx - g * head_dim;
    const size_t tile = ((size_t)blk * hkv + g) * kBlock * head_dim;
    kv_store(kpool, tile + k_tile_off(fp8, slot, d), fp8, k_scale, (float)k[(size_t)b * hkv * head_dim + idx]);
    kv_store(vpool, tile + v_tile_off(fp8, slot, d), fp8, v_scale, (float)v[(size_t)b * hkv * head_dim + idx]);
  }
}

}  // namespace

hipError_t launch_kv_append(void* k_pool, void* v_pool, const void* k, const void* v,
                            const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                            int hkv, int head_dim, bool fp8, float k_scale, float v_scale, int num_blocks,
                            hipStream_t s) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(batch), dim3(256), 0, s, k_pool, v_pool,
                     static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), bt, bt_stride, lens,
                     hkv, head_dim, fp8 ? 1 : 0, k_scale, v_scale, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
