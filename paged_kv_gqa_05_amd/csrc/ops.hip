// Small per-step kernels: embedding gather, RoPE + KV append of the new
// token, and greedy argmax.
//
// RoPE (rotate-half form) is not named by the pages; it is the position
// encoding of the Llama/Qwen2 families the rvLLM post lists as supported.  The
// angles pos * theta^(-2i/D) come from a host-built table (double precision,
// stored as f32 cos/sin), so the device evaluates no trigonometry.
#include "ops.h"

namespace pkv {
namespace {

typedef _Float16 h16;

// Also zeroes zero_n ints at zero_p (the split-K arrival counters of the step).
__global__ void embed_kernel(const h16* __restrict__ table, const int32_t* __restrict__ tokens,
                             h16* __restrict__ h, int hidden, int* __restrict__ zero_p, int zero_n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < zero_n; i += gridDim.x * blockDim.x) zero_p[i] = 0;
  const int b = blockIdx.x;
  const h16* src = table + (size_t)tokens[b] * hidden;
  h16* dst = h + (size_t)b * hidden;
  for (int i = threadIdx.x * 8; i < hidden; i += blockDim.x * 8)
    *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
}

// qkv: f32 [B][(Hq + 2 Hkv) D] (bias and norm already applied).  Writes the
// rotated q as f16 [B][Hq][D] and stores the rotated k and the v of the new
// token into the paged cache at pos = lens[b] - 1.
__global__ void rope_append_kernel(const float* __restrict__ qkv, const float2* __restrict__ cs,
                                   h16* __restrict__ q_out, h16* __restrict__ kpool,
                                   h16* __restrict__ vpool, const int32_t* __restrict__ bt,
                                   int bt_stride, const int32_t* __restrict__ lens, int hq, int hkv,
                                   int d) {
  const int b = blockIdx.x;
  const int c = lens[b];
  const int pos = c > 0 ? c - 1 : 0;
  const int half = d / 2;
  const int nrow = (hq + 2 * hkv) * d;
  const float* row = qkv + (size_t)b * nrow;
  const float2* csp = cs + (size_t)pos * half;
  int blk = 0;
  if (c > 0) blk = bt[(size_t)b * bt_stride + pos / kBlock];
  const int slot = pos % kBlock;
  // rotated pairs of q and k heads
  for (int idx = threadIdx.x; idx < (hq + hkv) * half; idx += blockDim.x) {
    const int head = idx / half, i = idx - head * half;
    const float x1 = row[head * d + i], x2 = row[head * d + half + i];
    const float2 t = csp[i];
    const float y1 = x1 * t.x - x2 * t.y;
    const float y2 = x2 * t.x + x1 * t.y;
    if (head < hq) {
      h16* qo = q_out + ((size_t)b * hq + head) * d;
      qo[i] = (h16)y1;
      qo[half + i] = (h16)y2;
    } else if (c > 0) {
      const int g = head - hq;
      // K tile [D/8][16][8]: 8-dim chunk, token, dim within the chunk
      h16* kp = kpool + ((size_t)blk * hkv + g) * kBlock * d + slot * 8;
      kp[(i >> 3) * (kBlock * 8) + (i & 7)] = (h16)y1;
      kp[((half + i) >> 3) * (kBlock * 8) + ((half + i) & 7)] = (h16)y2;
    }
  }
  if (c > 0) {
    for (int idx = threadIdx.x; idx < hkv * d; idx += blockDim.x) {
      const int g = idx / d, i = idx - g * d;
      vpool[(((size_t)blk * hkv + g) * d + i) * kBlock + slot] = (h16)row[(hq + hkv) * d + idx];
    }
  }
}

// Lowest index of the largest value per row; NaN logits never win.
__global__ void argmax_kernel(const h16* __restrict__ logits, int vocab, int32_t* __restrict__ out) {
  const int b = blockIdx.x;
  const h16* row = logits + (size_t)b * vocab;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = threadIdx.x; i < vocab; i += blockDim.x) {
    const float v = (float)row[i];
    if (v > best) {  // strictly greater: the first (lowest) index of a tie stays
      best = v;
      idx = i;
    }
  }
  __shared__ float sv[1024 / 64];
  __shared__ int si[1024 / 64];
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > best || (ov == best && oi < idx)) {
      best = ov;
      idx = oi;
    }
  }
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = best;
    si[wave] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < nw; ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < idx)) {
        best = sv[w];
        idx = si[w];
      }
    for (int w = 0; w < nw; ++w)
      if (sv[w] == best && si[w] < idx) idx = si[w];
    out[b] = idx == 0x7fffffff ? 0 : idx;
  }
}

}  // namespace

hipError_t launch_embed(const void* table, const int32_t* tokens, void* h, int batch, int hidden,
                        int* zero_p, int zero_n, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(batch), dim3(256), 0, s, static_cast<const h16*>(table), tokens,
                     static_cast<h16*>(h), hidden, zero_p, zero_n);
  return hipGetLastError();
}

hipError_t launch_rope_append(const float* qkv, const void* cos_sin, void* q_out, void* k_pool,
                              void* v_pool, const int32_t* bt, int bt_stride, const int32_t* lens,
                              int batch, int hq, int hkv, int d, hipStream_t s) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(batch), dim3(256), 0, s, qkv,
                     static_cast<const float2*>(cos_sin), static_cast<h16*>(q_out),
                     static_cast<h16*>(k_pool), static_cast<h16*>(v_pool), bt, bt_stride, lens, hq, hkv, d);
  return hipGetLastError();
}

hipError_t launch_argmax(const void* logits, int batch, int vocab, int32_t* tokens, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(batch), dim3(1024), 0, s, static_cast<const h16*>(logits), vocab,
                     tokens);
  return hipGetLastError();
}

}  // namespace pkv
