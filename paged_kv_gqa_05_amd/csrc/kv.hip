// KV append into the block-table paged cache (a plain copy into the slot of
// position context_lens[b] - 1; aitrends.kr glossary: the KV cache keeps the
// keys and values of earlier tokens; rvLLM post, section
// "PagedAttention과 FlashAttention-3": the cache is paged through block tables).
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ void kv_append_kernel(uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
                                 const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                 const int32_t* __restrict__ bt, int bt_stride,
                                 const int32_t* __restrict__ lens, int hkv, int head_dim) {
  const int b = blockIdx.x;
  const int c = lens[b];
  if (c <= 0) return;
  const int pos = c - 1;
  const int blk = bt[(size_t)b * bt_stride + pos / kBlock];
  const int slot = pos % kBlock;
  for (int idx = threadIdx.x; idx < hkv * head_dim; idx += blockDim.x) {
    const int g = idx / head_dim, d = idx - g * head_dim;
    const size_t bg = (size_t)blk * hkv + g;
    // K tile [D/8][16][8]: 8-dim chunk, token, dim within the chunk
    kpool[bg * kBlock * head_dim + (d >> 3) * (kBlock * 8) + slot * 8 + (d & 7)] = k[(size_t)b * hkv * head_dim + idx];
    vpool[(bg * head_dim + d) * kBlock + slot] = v[(size_t)b * hkv * head_dim + idx];
  }
}

}  // namespace

hipError_t launch_kv_append(void* k_pool, void* v_pool, const void* k, const void* v,
                            const int32_t* bt, int bt_stride, const int32_t* lens, int batch,
                            int hkv, int head_dim, hipStream_t s) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(batch), dim3(256), 0, s,
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), bt,
                     bt_stride, lens, hkv, head_dim);
  return hipGetLastError();
}

}  // namespace pkv
