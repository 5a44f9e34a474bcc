// Sampling of the next token after the captured forward pass: temperature,
// top-k, top-p and an inverse-CDF draw with a uniform number per row supplied
// by the caller (zingnex.cn article, section 支持的参数: temperature with 0 =
// greedy, top_p, top_k with -1 = disabled; rvLLM post, section "CUDA 그래프
// 리플레이": sampling stays outside the graph).
//
// Per row (one workgroup of 1024 threads):
//   z = logit / T; top-k keeps every token with z at or above the k-th
//   largest (ties kept); w = exp(z - max z); top-p keeps every token with w at
//   or above tau, the largest weight whose kept mass reaches top_p * sum w
//   (ties kept); the draw takes the first kept token in index order whose
//   running sum of w exceeds u * (kept mass).
// Both thresholds are found by radix descent over order-preserving 32-bit
// keys, 8 bits per pass over the row (the k-th largest by counts; tau by the
// mass carried per bin), so nothing is sorted.  Non-finite logits are never
// kept.  Sums are reduced in a fixed order (per-thread strides, then a fixed
// tree), so a row's result does not vary from run to run except through the
// top-p mass bins, which add in arrival order.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 h16;
constexpr int kST = 1024;
constexpr int kSW = kST / 64;

// Larger float -> larger key (negative floats reversed); -0 and +0 share a key.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < kSW; ++w) t += red[w];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int w = 0; w < kSW; ++w) t = fmaxf(t, red[w]);
  return t;
}

// f(i, logit) for the tokens [i0, i1) of a row.  With vec set, the row is
// 16-byte aligned and i0, i1 are multiples of 8 (or i1 = vocab, itself one),
// so eight logits come per 16-byte load.
template <class F>
__device__ __forceinline__ void for_range(const h16* row, int i0, int i1, int step, bool vec, F&& f) {
  if (vec) {
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    for (int v = (i0 >> 3); v < (i1 >> 3); v += step) {
      const uint4 q = rv[v];
      const h16* h = reinterpret_cast<const h16*>(&q);
#pragma unroll
      for (int j = 0; j < 8; ++j) f(v * 8 + j, (float)h[j]);
    }
  } else {
    for (int i = i0; i < i1; i += step) f(i, (float)row[i]);
  }
}
// The whole row, token i visited by thread (i / 8) % kST (vec) or i % kST.
template <class F>
__device__ __forceinline__ void for_row(const h16* row, int vocab, bool vec, F&& f) {
  for_range(row, vec ? threadIdx.x * 8 : threadIdx.x, vocab, kST, vec, f);
}

__global__ void __launch_bounds__(kST) sample_kernel(const h16* __restrict__ logits, int vocab, int vec,
                                                     const float* __restrict__ temperature,
                                                     const int32_t* __restrict__ top_k,
                                                     const float* __restrict__ top_p,
                                                     const float* __restrict__ uniform,
                                                     const int32_t* __restrict__ lens, int32_t* __restrict__ out) {
  __shared__ float red[kSW];
  __shared__ int hist[256];
  __shared__ float mass[256];
  __shared__ int bc_i[2];
  __shared__ float bc_f[2];
  __shared__ int s_tok;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (lens && lens[b] == 0) {  // inactive row
    if (tid == 0) out[b] = -1;
    return;
  }
  const h16* row = logits + (size_t)b * vocab;
  const float T = temperature[b];

  if (!(T > 0.f)) {  // greedy: lowest index of the largest logit
    float best = -INFINITY;
    int idx = 0x7fffffff;
    for_row(row, vocab, vec, [&](int i, float v) {
      if (v > best || (v == best && i < idx)) best = v, idx = i;
    });
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(idx, o, 64);
      if (ov > best || (ov == best && oi < idx)) best = ov, idx = oi;
    }
    if ((tid & 63) == 0) red[tid >> 6] = best, hist[tid >> 6] = idx;
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kSW; ++w)
        if (red[w] > best || (red[w] == best && hist[w] < idx)) best = red[w], idx = hist[w];
      out[b] = idx == 0x7fffffff ? 0 : idx;
    }
    return;
  }
  // z = logit / T; a non-finite z is never kept

  // ---- max z and the count of finite z
  float m = -INFINITY, cnt = 0.f;
  for_row(row, vocab, vec, [&](int, float x) {
    const float z = x / T;
    if (isfinite(z)) m = fmaxf(m, z), cnt += 1.f;
  });
  m = block_max(m, red);
  const int n_finite = (int)block_sum(cnt, red);

  // ---- top-k: key of the k-th largest finite z (radix select by counts)
  const int k = top_k[b];
  const bool use_k = k > 0 && k < n_finite;
  uint32_t kkey = 0;
  if (use_k) {
    uint32_t prefix = 0, mask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kST) hist[i] = 0;
      __syncthreads();
      for_row(row, vocab, vec, [&](int, float x) {
        const float z = x / T;
        if (!isfinite(z)) return;
        const uint32_t key = fkey(z);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      });
      __syncthreads();
      if (tid == 0) {
        int cum = 0, d = 255;
        for (; d > 0; --d) {
          if (cum + hist[d] >= need) break;
          cum += hist[d];
        }
        bc_i[0] = d;
        bc_i[1] = need - cum;
      }
      __syncthreads();
      prefix |= (uint32_t)bc_i[0] << shift;
      mask |= 255u << shift;
      need = bc_i[1];
      __syncthreads();
    }
    kkey = prefix;
  }
  auto kept_k = [&](float z) { return isfinite(z) && (!use_k || fkey(z) >= kkey); };

  // ---- total weight of the top-k set
  float zs = 0.f;
  for_row(row, vocab, vec, [&](int, float x) {
    const float z = x / T;
    if (kept_k(z)) zs += expf(z - m);
  });
  const float Z = block_sum(zs, red);

  // ---- top-p: tau, the largest weight whose kept mass reaches top_p * Z
  float p = top_p[b];
  const bool use_p = p < 1.f;  // NaN: disabled
  if (use_p && !(p > 0.f)) p = 1e-30f;  // keep only the largest weight (and its ties)
  uint32_t pkey = 0;
  if (use_p) {
    const float target = p * Z;
    uint32_t prefix = 0, mask = 0;
    float above = 0.f;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kST) mass[i] = 0.f;
      __syncthreads();
      for_row(row, vocab, vec, [&](int, float x) {
        const float z = x / T;
        if (!kept_k(z)) return;
        const float w = expf(z - m);
        const uint32_t key = fkey(w);
        if ((key & mask) == prefix) atomicAdd(&mass[(key >> shift) & 255], w);
      });
      __syncthreads();
      if (tid == 0) {
        float cum = above;
        int d = 255;
        for (; d > 0; --d) {
          if (cum + mass[d] >= target) break;
          cum += mass[d];
        }
        bc_i[0] = d;
        bc_f[0] = cum;
      }
      __syncthreads();
      prefix |= (uint32_t)bc_i[0] << shift;
      mask |= 255u << shift;
      above = bc_f[0];
      __syncthreads();
    }
    pkey = prefix;
  }
  auto weight = [&](float x) {  // w if the token is kept, else 0
    const float z = x / T;
    if (!kept_k(z)) return 0.f;
    const float w = expf(z - m);
    return (!use_p || fkey(w) >= pkey) ? w : 0.f;
  };

  // ---- the draw: contiguous chunks per thread, prefix over chunks
  const int chunk = vec ? 8 * ((vocab + 8 * kST - 1) / (8 * kST)) : (vocab + kST - 1) / kST;
  const int i0 = min(tid * chunk, vocab), i1 = min(i0 + chunk, vocab);
  float cs = 0.f;
  int last = -1;
  for_range(row, i0, i1, 1, vec, [&](int i, float x) {
    const float w = weight(x);
    if (w > 0.f) cs += w, last = i;
  });
  // inclusive scan of the chunk sums in thread order
  float incl = cs;
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o, 64);
    if ((tid & 63) >= o) incl += t;
  }
  __syncthreads();  // every read of red by the reductions above is done
  if ((tid & 63) == 63) red[tid >> 6] = incl;
  __syncthreads();
  float wave_off = 0.f;
  for (int w = 0; w < (tid >> 6); ++w) wave_off += red[w];
  float total = 0.f;
  for (int w = 0; w < kSW; ++w) total += red[w];
  const float excl = wave_off + incl - cs;
  float u = uniform[b];
  u = u < 0.f ? 0.f : (u >= 1.f ? 0.99999994f : u);
  const float target = u * total;
  // the first thread whose running total passes the target walks its chunk;
  // with no such thread (rounding), the last kept token of the row
  int first = (cs > 0.f && excl + cs > target) ? tid : kST;
  int lk = last;
  for (int o = 32; o > 0; o >>= 1) {
    first = min(first, __shfl_xor(first, o, 64));
    lk = max(lk, __shfl_xor(lk, o, 64));
  }
  if ((tid & 63) == 0) {
    hist[tid >> 6] = first;
    hist[kSW + (tid >> 6)] = lk;
  }
  __syncthreads();
  int f = kST, l = -1;
  for (int w = 0; w < kSW; ++w) f = min(f, hist[w]), l = max(l, hist[kSW + w]);
  if (tid == 0 && f == kST) s_tok = l < 0 ? 0 : l;
  if (tid == f) {
    float run = excl;
    int tok = -1;
    for_range(row, i0, i1, 1, vec, [&](int i, float x) {
      const float w = weight(x);
      if (tok < 0 && w > 0.f) {
        run += w;
        if (run > target) tok = i;
      }
    });
    s_tok = tok < 0 ? last : tok;
  }
  __syncthreads();
  if (tid == 0) out[b] = s_tok;
}

}  // namespace

hipError_t launch_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* uniform, const int32_t* lens, int32_t* tokens,
                         hipStream_t s) {
  const int vec = (vocab % 8 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0) ? 1 : 0;
  hipLaunchKernelGGL(sample_kernel, dim3(batch), dim3(kST), 0, s, static_cast<const h16*>(logits), vocab, vec,
                     temperature, top_k, top_p, uniform, lens, tokens);
  return hipGetLastError();
}

}  // namespace pkv
