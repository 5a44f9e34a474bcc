// Sampling of the next token after the captured forward pass: penalties,
// temperature, top-k, top-p and an inverse-CDF draw with a uniform number per
// row supplied by the caller (zingnex.cn article, section 支持的参数:
// temperature with 0 = greedy, top_p, top_k with -1 = disabled; section
// CPU操作优化: repetition, frequency and presence penalties, combined; rvLLM
// post, section "CUDA 그래프 리플레이": sampling stays outside the graph).
//
// Penalties (penalize_kernel, before the sampler, in place): for every token
// already sampled c > 0 times for the row, in float32 with one rounding per
// operation, x = x > 0 ? x / r : x * r, then x = (x - f c) - p, rounded to f16.
//
// Per row (one workgroup of 1024 threads), for T > 0:
//   every finite logit x weighs W(x) = floor(2^40 E((x - m) (1/T))), m the
//   largest finite logit and E a float32 exponential with one rounding per
//   operation (no fused multiply-add), so the weights, every mass and the
//   draw are exact integers that a plain reimplementation reproduces;
//   top-k keeps every token whose logit is at least the k-th largest (ties
//   kept); top-p keeps the tokens whose logit is at least the largest value t
//   for which the kept tokens at or above t carry ceil(top_p sum W) (ties
//   kept); the draw takes the first kept token in index order whose running
//   sum of W exceeds floor(u24 Z / 2^24), u24 = floor(u 2^24), Z the kept mass.
// Both thresholds are found as a logit: radix descent over the logit's
// 16-bit order-preserving key, an 11-bit digit then a 5-bit one, counting
// tokens (top-k) or summing W (top-p) per bin; sums are 64-bit integers, so
// they are exact and order-free.  Passes over the row: max and count (fused
// into the first top-k pass), two for top-k, two for top-p (the first also
// gives sum W), one to sum W per wave segment and per 64-unit step of it;
// then one wave loads the step where the draw lands.  Non-finite logits are
// never kept.  With a counts buffer the row's count of the sampled token is
// incremented at the end.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 h16;
constexpr int kST = 1024;
constexpr int kSW = kST / 64;
constexpr int kBins = 2048;
constexpr int kMaxSteps = 64;                         // step sums kept per wave segment                           // the first digit: key bits 15..5
constexpr uint32_t kKeyNegInf = 0x03ffu, kKeyPosInf = 0xfc00u;

// Larger logit -> larger key; -0 and +0 share a key; NaNs fall outside
// [key(-inf), key(+inf)].
__device__ __forceinline__ uint32_t hkey(uint32_t u) {
  if ((u & 0x7fffu) == 0) u = 0;
  return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
}
__device__ __forceinline__ bool key_finite(uint32_t k) { return k > kKeyNegInf && k < kKeyPosInf; }
__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
  return (float)__builtin_bit_cast(h16, (uint16_t)u);
}
__device__ __forceinline__ float logit_of(uint32_t u) { return (float)__builtin_bit_cast(h16, (uint16_t)u); }

// A unit is eight logits (one 16-byte load) when VEC, else one logit.
template <bool VEC>
struct Row {
  static constexpr int kElems = VEC ? 8 : 1;
  const uint16_t* p;
  int vocab;
  __device__ int units() const { return VEC ? vocab >> 3 : vocab; }
  __device__ uint4 load(int unit) const {
    if (VEC) return reinterpret_cast<const uint4*>(p)[unit];
    return make_uint4(p[unit], 0u, 0u, 0u);
  }
  __device__ static uint32_t elem(const uint4& q, int j) {
    const uint32_t w = j < 2 ? q.x : (j < 4 ? q.y : (j < 6 ? q.z : q.w));
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
  }
};

// f(index, f16 bits) for every token, token unit v by thread v % kST; four
// units in flight per thread.
template <bool VEC, class F>
__device__ __forceinline__ void for_row(const Row<VEC>& r, F&& f) {
  const int n = r.units();
  for (int v0 = threadIdx.x; v0 < n; v0 += 4 * kST) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = r.load(min(v0 + u * kST, n - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * kST;
      if (v < n) {
#pragma unroll
        for (int j = 0; j < Row<VEC>::kElems; ++j) f(v * Row<VEC>::kElems + j, Row<VEC>::elem(q[u], j));
      }
    }
  }
}

typedef unsigned long long u64;

// float32 constants of the exponential: log2(e), ln 2 split as c1 + c2 (c1
// exact in 9 bits, so n c1 is exact), Taylor coefficients 1/k!
__device__ constexpr float kL2E = (float)1.4426950408889634;
__device__ constexpr float kLn2Hi = 0.693359375f;
__device__ constexpr float kLn2Lo = (float)-2.12194440e-4;
__device__ constexpr float kC7 = (float)(1.0 / 5040.0), kC6 = (float)(1.0 / 720.0), kC5 = (float)(1.0 / 120.0),
                           kC4 = (float)(1.0 / 24.0), kC3 = (float)(1.0 / 6.0);

// W = floor(2^40 e^y) for y = (x - mx) * inv_t <= 0 (1 for x = mx, 0 for
// y < -30): n = floor(y log2 e + 1/2), r = (y - n c1) - n c2, e^r by the
// degree-7 Taylor polynomial in Horner form, scaled by 2^(n + 40).  Every
// operation is rounded on its own (no contraction into fused multiply-adds),
// so the integer is fixed by the float32 arithmetic alone.
__device__ __forceinline__ u64 wfixed(float x, float mx, float inv_t) {
#pragma clang fp contract(off)
  const float d = x - mx;
  const float y = d == 0.f ? 0.f : d * inv_t;
  if (!(y >= -30.f)) return 0ull;
  const float n = floorf(y * kL2E + 0.5f);
  const float r = (y - n * kLn2Hi) - n * kLn2Lo;
  float p = kC7;
  p = p * r + kC6;
  p = p * r + kC5;
  p = p * r + kC4;
  p = p * r + kC3;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return (u64)ldexpf(p, (int)n + 40);
}

struct Smem {
  union {
    uint32_t i[2 * kBins];
    u64 l[kBins];
  } hist;
  u64 wl[kSW];
  u64 steps[kSW * kMaxSteps];
  u64 wf[kSW];
  int wi[kSW];
  int bin;
  u64 before, total, target;
  int tok;
};

// Descending selection over the kBins bins (32-bit counts, or 64-bit masses
// when kWide): the first bin, from the top, at which above + (all higher
// bins) + (the bin itself) reaches target_abs + ceil(frac * (sum of all
// bins)); bin 0 if none does.  Leaves the bin, the amount above it (above
// included), the bins' sum and the target in sm.  Only non-empty bins are
// taken, so a target of 0 gives the highest non-empty bin.
template <bool kWide>
__device__ void select_bin(Smem& sm, u64 above, u64 target_abs, float frac) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b0 = kBins - 1 - 2 * tid;
  const u64 a = kWide ? sm.hist.l[b0] : sm.hist.i[b0];
  const u64 c = kWide ? sm.hist.l[b0 - 1] : sm.hist.i[b0 - 1];
  const u64 loc = a + c;
  u64 incl = loc;
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sm.wl[wave] = incl;
  __syncthreads();
  u64 off = above, tot = 0;
  for (int w = 0; w < kSW; ++w) {
    const u64 x = sm.wl[w];
    if (w < wave) off += x;
    tot += x;
  }
  const u64 target = target_abs + (frac > 0.f ? (u64)ceil((double)frac * (double)tot) : 0ull);
  const u64 before = off + incl - loc;
  int cand = 2 * kBins;
  // a bin is taken only if it holds something: with target 0 the first
  // non-empty bin, otherwise the crossing bin (never empty anyway)
  if (a > 0 && before + a >= target)
    cand = 2 * tid;
  else if (c > 0 && before + loc >= target)
    cand = 2 * tid + 1;
  for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, 64));
  if (lane == 0) sm.wi[wave] = cand;
  __syncthreads();
  int j = 2 * kBins;
  for (int w = 0; w < kSW; ++w) j = min(j, sm.wi[w]);
  if (j == 2 * kBins) j = kBins - 1;
  if (tid == (j >> 1)) {
    sm.bin = kBins - 1 - j;
    sm.before = (j & 1) ? before + a : before;
  }
  if (tid == 0) sm.total = tot, sm.target = target;
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(Smem& sm) {
#pragma unroll
  for (int j = 0; j < 4; ++j) sm.hist.i[threadIdx.x + j * kST] = 0;
  __syncthreads();
}

template <bool VEC>
__global__ void __launch_bounds__(kST) sample_kernel(const uint16_t* __restrict__ logits, int vocab,
                                                     const float* __restrict__ temperature,
                                                     const int32_t* __restrict__ top_k,
                                                     const float* __restrict__ top_p,
                                                     const float* __restrict__ uniform,
                                                     const int32_t* __restrict__ lens, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ counts) {
  __shared__ Smem sm;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (lens && lens[b] == 0) {  // inactive row
    if (tid == 0) out[b] = -1;
    return;
  }
  const Row<VEC> row{logits + (size_t)b * vocab, vocab};
  const float T = temperature[b];

  if (!(T > 0.f)) {  // greedy: lowest index of the largest non-NaN logit
    unsigned long long best = 0;
    for_row(row, [&](int i, uint32_t u) {
      const uint32_t k = hkey(u);
      const unsigned long long c = ((unsigned long long)k << 32) | (0xffffffffu - (uint32_t)i);
      if (k >= kKeyNegInf && k <= kKeyPosInf && c > best) best = c;
    });
    uint32_t hi = (uint32_t)(best >> 32), lo = (uint32_t)best;
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t oh = __shfl_xor(hi, o, 64), ol = __shfl_xor(lo, o, 64);
      if (oh > hi || (oh == hi && ol > lo)) hi = oh, lo = ol;
    }
    if (lane == 0) sm.hist.i[2 * wave] = hi, sm.hist.i[2 * wave + 1] = lo;
    __syncthreads();
    if (tid == 0) {
      for (int w = 0; w < kSW; ++w) {
        const uint32_t oh = (uint32_t)sm.hist.i[2 * w], ol = (uint32_t)sm.hist.i[2 * w + 1];
        if (oh > hi || (oh == hi && ol > lo)) hi = oh, lo = ol;
      }
      const int tok = hi == 0 ? 0 : (int)(0xffffffffu - lo);
      out[b] = tok;
      if (counts) counts[(size_t)b * vocab + tok] += 1;
    }
    return;
  }
  const float inv_t = 1.f / T;

  // ---- pass 1: largest finite key; with top-k also the first-digit counts
  const int k = top_k[b];
  if (k > 0) clear_hist(sm);
  uint32_t kmax = 0;
  for_row(row, [&](int, uint32_t u) {
    const uint32_t key = hkey(u);
    if (!key_finite(key)) return;
    kmax = max(kmax, key);
    if (k > 0) atomicAdd(&sm.hist.i[key >> 5], 1u);
  });
  for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  if (lane == 0) sm.wi[wave] = (int)kmax;
  __syncthreads();
  for (int w = 0; w < kSW; ++w) kmax = max(kmax, (uint32_t)sm.wi[w]);
  const float mx = key_value(kmax);  // unused when no logit is finite
  __syncthreads();

  // ---- top-k: the k-th largest key (counts, ties at it all kept)
  uint32_t thr = kKeyNegInf + 1;  // smallest finite key
  if (k > 0) {
    select_bin<false>(sm, 0, (u64)k, 0.f);
    if ((u64)k < sm.total) {  // else every finite logit is kept
      const uint32_t hb = sm.bin;
      const u64 need = (u64)k - sm.before;
      __syncthreads();
      clear_hist(sm);
      for_row(row, [&](int, uint32_t u) {
        const uint32_t key = hkey(u);
        if (key_finite(key) && (key >> 5) == hb) atomicAdd(&sm.hist.i[key & 31], 1u);
      });
      __syncthreads();
      select_bin<false>(sm, 0, need, 0.f);
      thr = (hb << 5) | sm.bin;
    }
    __syncthreads();
  }
  auto kept = [&](uint32_t key) { return key_finite(key) && key >= thr; };
  auto weight_of = [&](float x) { return wfixed(x, mx, inv_t); };
  auto weight = [&](uint32_t u) { return weight_of(logit_of(u)); };

  // ---- top-p: the key of tau (mass per bin; the first pass also gives sum w)
  const float p = top_p[b];
  if (p < 1.f) {  // NaN: off
    const float frac = p > 0.f ? p : 0.f;  // 0 keeps the largest weight and its ties
    clear_hist(sm);
    for_row(row, [&](int, uint32_t u) {
      const uint32_t key = hkey(u);
      if (kept(key)) atomicAdd(&sm.hist.l[key >> 5], weight(u));
    });
    __syncthreads();
    select_bin<true>(sm, 0, 0, frac);
    const uint32_t hb = sm.bin;
    const u64 above = sm.before, target = sm.target;
    __syncthreads();
    clear_hist(sm);
    // the second digit completes the key, so a bin's mass is its count times
    // the weight of that one logit value: the same integers as summing per token
    for_row(row, [&](int, uint32_t u) {
      const uint32_t key = hkey(u);
      if (kept(key) && (key >> 5) == hb) atomicAdd(&sm.hist.i[key & 31], 1u);
    });
    __syncthreads();
    const uint32_t cnt = tid < 32 ? sm.hist.i[tid] : 0u;
    __syncthreads();
    if (tid < 32) sm.hist.l[tid] = cnt ? (u64)cnt * weight_of(key_value((hb << 5) | tid)) : 0ull;
    __syncthreads();
    select_bin<true>(sm, above, target, 0.f);
    thr = max(thr, (hb << 5) | sm.bin);
    __syncthreads();
  }

  // ---- the draw: each wave sums W over its contiguous segment of units, 64
  // units per step, keeping the step sums (up to kMaxSteps) for the walk
  const int n = row.units();
  const int seg = (n + kSW - 1) / kSW;
  const int s0 = min(wave * seg, n), s1 = min(s0 + seg, n);
  const int nsteps = (s1 - s0 + 63) >> 6;
  u64 ws = 0;
  int lastk = -1;
  for (int st0 = 0; st0 < nsteps; st0 += 4) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = row.load(min(s0 + (st0 + u) * 64 + lane, s1 - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = st0 + u, v = s0 + st * 64 + lane;
      if (st >= nsteps) break;
      u64 uw = 0;
      if (v < s1) {
#pragma unroll
        for (int j = 0; j < Row<VEC>::kElems; ++j) {
          const uint32_t e = Row<VEC>::elem(q[u], j);
          if (kept(hkey(e))) uw += weight(e), lastk = v * Row<VEC>::kElems + j;
        }
      }
      for (int o = 32; o > 0; o >>= 1) uw += __shfl_xor(uw, o, 64);
      if (lane == 0 && st < kMaxSteps) sm.steps[wave * kMaxSteps + st] = uw;
      ws += uw;
    }
  }
  for (int o = 32; o > 0; o >>= 1) lastk = max(lastk, __shfl_xor(lastk, o, 64));
  if (lane == 0) sm.wf[wave] = ws, sm.wi[wave] = lastk;
  __syncthreads();
  u64 total = 0;
  for (int w = 0; w < kSW; ++w) total += sm.wf[w];
  float uu = uniform[b];
  uu = uu > 0.f ? fminf(uu, 0.99999994f) : 0.f;  // [0, 1 - 2^-24]; NaN -> 0
  const u64 u24 = (u64)(uu * 16777216.f);         // exact scaling, then truncation
  // floor(u24 * total / 2^24) without overflow (total < 2^58)
  const u64 target = ((u24 * (total >> 32)) << 8) + ((u24 * (total & 0xffffffffull)) >> 24);
  // the first segment whose running total passes the target (none only when
  // nothing is kept: then token 0)
  int hit = -1;
  u64 run = 0;
  int last_all = -1;
  for (int w = 0; w < kSW; ++w) {
    last_all = max(last_all, sm.wi[w]);
    if (hit < 0 && sm.wf[w] > 0 && run + sm.wf[w] > target) hit = w;
    if (hit < 0) run += sm.wf[w];
  }
  if (tid == 0) sm.tok = last_all < 0 ? 0 : last_all;
  __syncthreads();
  if (wave == hit) {
    // the step where the draw lands (from the kept step sums), else every step
    int stb = 0, ste = nsteps;
    if (nsteps <= kMaxSteps) {
      int st = 0;
      for (; st < nsteps; ++st) {
        const u64 t = sm.steps[wave * kMaxSteps + st];
        if (t > 0 && run + t > target) break;
        run += t;
      }
      stb = st;
      ste = st < nsteps ? st + 1 : st;
    }
    int tok = -1;
    for (int st = stb; st < ste && tok < 0; ++st) {
      const int v = s0 + st * 64 + lane;
      const uint4 q = row.load(min(v, s1 - 1));
      u64 uw = 0;
      if (v < s1) {
#pragma unroll
        for (int j = 0; j < Row<VEC>::kElems; ++j) {
          const uint32_t e = Row<VEC>::elem(q, j);
          if (kept(hkey(e))) uw += weight(e);
        }
      }
      u64 incl = uw;
      for (int o = 1; o < 64; o <<= 1) {
        const u64 t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const unsigned long long m = __ballot(uw > 0 && run + incl > target);
      if (m) {
        const int f = __ffsll((long long)m) - 1;
        if (lane == f) {
          u64 r = run + incl - uw;
#pragma unroll
          for (int j = 0; j < Row<VEC>::kElems; ++j) {
            const uint32_t e = Row<VEC>::elem(q, j);
            if (kept(hkey(e))) {
              r += weight(e);
              if (r > target) {
                tok = v * Row<VEC>::kElems + j;
                break;
              }
            }
          }
          sm.tok = tok;
        }
        tok = __shfl(tok, f, 64);
      } else {
        run += __shfl(incl, 63, 64);
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    out[b] = sm.tok;
    if (counts) counts[(size_t)b * vocab + sm.tok] += 1;
  }
}

// Penalties in place, before the sampler: tokens already sampled for the row
// (counts > 0) get x / r (x > 0) or x * r, then - f c - p, in float32 with
// one rounding per operation, stored back as f16.  Rows that are inactive or
// whose three parameters are neutral are left untouched.
__global__ void __launch_bounds__(256) penalize_kernel(uint16_t* __restrict__ logits, int vocab,
                                                       const int32_t* __restrict__ counts,
                                                       const float* __restrict__ repetition,
                                                       const float* __restrict__ frequency,
                                                       const float* __restrict__ presence,
                                                       const int32_t* __restrict__ lens) {
#pragma clang fp contract(off)
  const int b = blockIdx.y;
  if (lens && lens[b] == 0) return;
  const float r = repetition[b], f = frequency[b], p = presence[b];
  if (r == 1.f && f == 0.f && p == 0.f) return;
  const int32_t* crow = counts + (size_t)b * vocab;
  uint16_t* lrow = logits + (size_t)b * vocab;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < vocab; i += gridDim.x * blockDim.x) {
    const int c = crow[i];
    if (c > 0) {
      float x = logit_of(lrow[i]);
      x = x > 0.f ? x / r : x * r;
      x = (x - f * (float)c) - p;
      lrow[i] = __builtin_bit_cast(uint16_t, (h16)x);
    }
  }
}

}  // namespace

hipError_t launch_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* uniform, const int32_t* lens, int32_t* tokens,
                         hipStream_t s, void* penalized_logits, int32_t* counts, const float* repetition,
                         const float* frequency, const float* presence) {
  if (counts && penalized_logits) {
    const int per_row = std::min(64, (vocab + 1023) / 1024);
    hipLaunchKernelGGL(penalize_kernel, dim3(per_row, batch), dim3(256), 0, s,
                       static_cast<uint16_t*>(penalized_logits), vocab, counts, repetition, frequency, presence, lens);
  }
  const auto* l = static_cast<const uint16_t*>(logits);
  if (vocab % 8 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0)
    hipLaunchKernelGGL(sample_kernel<true>, dim3(batch), dim3(kST), 0, s, l, vocab, temperature, top_k, top_p,
                       uniform, lens, tokens, counts);
  else
    hipLaunchKernelGGL(sample_kernel<false>, dim3(batch), dim3(kST), 0, s, l, vocab, temperature, top_k, top_p,
                       uniform, lens, tokens, counts);
  return hipGetLastError();
}

}  // namespace pkv
