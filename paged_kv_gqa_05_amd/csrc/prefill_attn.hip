// Causal multi-token attention of a prefill over the paged KV cache (rvLLM
// post on discuss.pytorch.kr, section "PagedAttention과 FlashAttention-3":
// causal attention of many query tokens over the block-table cache, GQA).
//
// New token j of sequence s (position prior_s + j) and query head h of KV
// group g attend over key positions 0 .. prior_s + j of the sequence:
//   out[t][h] = sum_k softmax_k(scale * <q[t][h], K_k>) V_k.
// The k and v of every new token are already in the cache (the QKV
// projection's epilogue appends them before this kernel runs).
//
// Design (MI355X):
//  * The query rows of one (sequence, KV head) are numbered token-major,
//    r = j * G + (h - g G), and cut into 16-row chunks; one wave takes one
//    chunk: its 16 rows are the 16 columns of the MFMA tiles, so every
//    16-token K/V page it loads serves 16 query rows (a decode-style row per
//    token would use 1 to 16 of them and re-read the prefix per token).
//  * Pages stream in groups of four, K and V of the group in flight at once,
//    straight into MFMA operand registers in the layouts of the decode kernel:
//    S^T[key][row] from v_mfma_f32_16x16x32_f16 (K page as A, the rows' q as
//    B), then O^T[dim][row] += V^T P^T with v_mfma_f32_16x16x16f16, whose B
//    operand is the score accumulator layout itself.  Online softmax per
//    column: running max and sum, the 32 output accumulators rescaled once
//    per group of pages.
//  * Causal mask per column (key position <= the row's position); value slots
//    at or past the sequence's cached length (prior + new tokens) are zeroed
//    before the PV product, since unwritten slots may hold anything.
//  * The (sequence, chunk) work list is built on the device by a one-workgroup
//    kernel from the sequence offsets (once per prefill call, shared by all
//    layers), so the host needs no copy of them.
#include "ops.h"

namespace pkv {
namespace {

typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896341f;
constexpr int kPagesPerGroup = 4;

struct Params {
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  const h16* q;
  h16* out;
  const int32_t* seq_starts;
  const int32_t* prior_lens;
  const int32_t* bt;
  int bt_stride;
  const int2* items;
  const int32_t* n_items;
  int n_tokens, hq, hkv, group, max_context;
  int num_blocks;    // blocks in the pool: a block id outside [0, num_blocks) is read as block 0
  float scale_log2;  // softmax scale * log2(e) * K dequant scale
  float v_scale;     // V dequant scale (1 for f16)
};

template <bool HI>
__device__ __forceinline__ h16x2 fp8x2_to_h16x2(int w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
__device__ __forceinline__ h16x4 fp8x4_to_h16x4(int w) {
  const h16x2 a = fp8x2_to_h16x2<false>(w), b = fp8x2_to_h16x2<true>(w);
  return h16x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ h16x8 fp8x8_to_h16x8(int lo, int hi) {
  const h16x4 a = fp8x4_to_h16x4(lo), b = fp8x4_to_h16x4(hi);
  return h16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The 8-dim chunk that lane group q4 feeds at QK step s: f16 K pages are
// [D/8][16 keys][8 dims] (step s reads chunks 4s .. 4s+3), fp8 K pages
// [D/16][16 keys][16 dims] (one 16-byte load covers steps 2u and 2u+1).
template <bool FP8>
__device__ __forceinline__ int q_chunk(int s, int q4) {
  return FP8 ? 8 * (s >> 1) + 2 * q4 + (s & 1) : 4 * s + q4;
}

// One page's K and V registers for one lane (n = key of the K rows and
// dim-in-group of the V rows, q4 = lane group).
template <int D, bool FP8>
struct Page;

template <int D>
struct Page<D, false> {
  h16x8 k[D / 32];  // step s: key n, dims of chunk 4s + q4
  h16x4 v[D / 16];  // V^T[dim 16j + n][keys 4 q4 .. +4]
  __device__ __forceinline__ void load(const Params& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const h16* kp = reinterpret_cast<const h16*>(p.k_pool) + tile * kBlock * D + lane * 8;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) k[s] = *reinterpret_cast<const h16x8*>(kp + s * 512);
    const h16* vp = reinterpret_cast<const h16*>(p.v_pool) + tile * D * kBlock + (lane & 15) * kBlock +
                    (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) v[j] = *reinterpret_cast<const h16x4*>(vp + j * 16 * kBlock);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const { return k[s]; }
  __device__ __forceinline__ h16x4 vfrag(int j) const { return v[j]; }
};

template <int D>
struct Page<D, true> {
  int4 k[D / 64];  // 16 codes: key n, dims 16 (4u + q4) .. +16 (steps 2u, 2u + 1)
  int4 v[D / 64];  // 4 x 4 codes: V^T[dim 16j + n][keys 4 q4 .. +4] for j = 4u .. 4u + 3
  __device__ __forceinline__ void load(const Params& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const unsigned char* kp = p.k_pool + tile * kBlock * D + lane * 16;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) k[u] = *reinterpret_cast<const int4*>(kp + u * 1024);
    const unsigned char* vp = p.v_pool + tile * D * kBlock + lane * 16;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) v[u] = *reinterpret_cast<const int4*>(vp + u * 1024);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const {
    const int4 w = k[s >> 1];
    return (s & 1) ? fp8x8_to_h16x8(w.z, w.w) : fp8x8_to_h16x8(w.x, w.y);
  }
  __device__ __forceinline__ h16x4 vfrag(int j) const {
    const int4 w = v[j >> 2];
    const int r = j & 3;
    return fp8x4_to_h16x4(r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w);
  }
};

// Sequence s's new tokens [t0, t1), clamped as the per-token rows are.
__device__ __forceinline__ void seq_range(const int32_t* seq_starts, int s, int n_tokens, int& t0, int& t1) {
  t0 = min(max(seq_starts[s], 0), n_tokens);
  t1 = min(max(seq_starts[s + 1], t0), n_tokens);
}

// Work list: for every sequence s, its ceil(n_s G / 16) chunks (s, c), in
// sequence order; *n_items gets the count (capped at max_items, which the
// host sizes as ceil(T G / 16) + S).
__global__ void __launch_bounds__(1024) items_kernel(const int32_t* __restrict__ seq_starts, int n_seqs,
                                                     int n_tokens, int group, int2* __restrict__ items,
                                                     int32_t* __restrict__ n_items, int max_items) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n_seqs; base += 1024) {
    const int s = base + tid;
    int cnt = 0;
    if (s < n_seqs) {
      int t0, t1;
      seq_range(seq_starts, s, n_tokens, t0, t1);
      cnt = (int)(((long long)(t1 - t0) * group + 15) / 16);
    }
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int off = carry, tot = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) off += wsum[w];
      tot += wsum[w];
    }
    off += incl - cnt;
    for (int c = 0; c < cnt && off + c < max_items; ++c) items[off + c] = make_int2(s, c);
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) *n_items = min(carry, max_items);
}

template <int D, bool FP8>
__global__ void __launch_bounds__(256) prefill_attn_kernel(Params p) {
  constexpr int NP = kPagesPerGroup;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int item = blockIdx.x * 4 + wave;
  const int g = blockIdx.y;
  if (item >= *p.n_items) return;  // wave-uniform; the kernel has no workgroup barrier
  const int2 it = p.items[item];
  const int s = it.x, c = it.y;
  int t0, t1;
  seq_range(p.seq_starts, s, p.n_tokens, t0, t1);
  const int n_s = t1 - t0, prior = p.prior_lens[s], G = p.group;

  // this lane's column: query row r = token j, head hh of the group
  const int r = 16 * c + n;
  const int j = r / G, hh = r - j * G;
  const int pcol = prior + j;  // keys 0 .. pcol
  const bool col_ok = j < n_s && pcol >= 0 && pcol < p.max_context;
  // the wave's last query position, and the sequence's cached length
  const int plast = min(prior + min(n_s - 1, (16 * c + 15) / G), p.max_context - 1);
  if (plast < 0) return;
  const int total = min(prior + n_s, p.max_context);
  const int n_pages = plast / kBlock + 1;

  h16x8 qf[D / 32];
  {
    const h16* qrow = p.q + ((size_t)(t0 + min(j, max(n_s - 1, 0))) * p.hq + g * G + hh) * D;
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
      qf[st] = col_ok ? *reinterpret_cast<const h16x8*>(qrow + 8 * q_chunk<FP8>(st, q4))
                      : h16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const int32_t* btrow = p.bt + (size_t)s * p.bt_stride;

  float m = -INFINITY, l = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int jj = 0; jj < D / 16; ++jj) o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int pg0 = 0; pg0 < n_pages; pg0 += NP) {
    Page<D, FP8> pg[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const int blk = btrow[min(pg0 + t, n_pages - 1)];
      pg[t].load(p, (unsigned)blk < (unsigned)p.num_blocks ? blk : 0, g, lane);
    }
    // scores of the group's pages, log2 domain, causal mask per column
    float x[NP][4];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < D / 32; ++st)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pg[t].kfrag(st), qf[st], sacc, 0, 0, 0);
      const int key0 = (pg0 + t) * kBlock + 4 * q4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        x[t][rr] = (col_ok && pg0 + t < n_pages && key0 + rr <= pcol) ? sacc[rr] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[t][rr]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // every lane runs every product (MFMA reads the whole wave's operands): a
    // column with nothing visible yet keeps m = -inf and gets zero weights
    const float m_new = fmaxf(m, mt);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);  // 0 while m is still -inf
    l *= alpha;
#pragma unroll
    for (int jj = 0; jj < D / 16; ++jj) o[jj] *= alpha;
    m = m_new;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      if (pg0 + t < n_pages) {
        float pr[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pr[rr] = __builtin_amdgcn_exp2f(x[t][rr] - m_ref);
        l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        const h16x4 pf = h16x4{(h16)pr[0], (h16)pr[1], (h16)pr[2], (h16)pr[3]};
        const int key0 = (pg0 + t) * kBlock + 4 * q4;
        if ((pg0 + t + 1) * kBlock > total) {
          // the sequence's last, partial page: slots past its cached length
          // may hold anything (NaN included)
#pragma unroll
          for (int jj = 0; jj < D / 16; ++jj) {
            h16x4 vf = pg[t].vfrag(jj);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              if (key0 + rr >= total) vf[rr] = (h16)0.f;
            o[jj] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf, o[jj], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < D / 16; ++jj)
            o[jj] = __builtin_amdgcn_mfma_f32_16x16x16f16(pg[t].vfrag(jj), pf, o[jj], 0, 0, 0);
        }
      }
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (j < n_s) {
    // lane holds O^T[dims 16 jj + 4 q4 .. +4][column n]; a token past
    // max_context attends to nothing and gets 0
    const float inv = (col_ok && l > 0.f) ? p.v_scale / l : 0.f;
    h16* orow = p.out + ((size_t)(t0 + j) * p.hq + g * G + hh) * D + 4 * q4;
#pragma unroll
    for (int jj = 0; jj < D / 16; ++jj)
      *reinterpret_cast<h16x4*>(orow + 16 * jj) =
          h16x4{(h16)(o[jj][0] * inv), (h16)(o[jj][1] * inv), (h16)(o[jj][2] * inv), (h16)(o[jj][3] * inv)};
  }
}

template <int D, bool FP8>
hipError_t launch_d(const Params& p, int max_items, hipStream_t s) {
  hipLaunchKernelGGL((prefill_attn_kernel<D, FP8>), dim3((max_items + 3) / 4, p.hkv), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int prefill_max_items(int n_tokens, int n_seqs, int group) {
  return (int)(((long long)n_tokens * group + 15) / 16) + n_seqs;
}

hipError_t launch_prefill_items(const PrefillAttnArgs& a, int group, hipStream_t s) {
  hipLaunchKernelGGL(items_kernel, dim3(1), dim3(1024), 0, s, a.seq_starts, a.n_seqs, a.n_tokens, group,
                     reinterpret_cast<int2*>(a.items), a.n_items, a.max_items);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillAttnArgs& a, hipStream_t s) {
  if (a.head_dim != 64 && a.head_dim != 128) return hipErrorInvalidValue;
  const int group = a.hq / a.hkv;
  Params p{};
  p.k_pool = static_cast<const unsigned char*>(a.k_pool);
  p.v_pool = static_cast<const unsigned char*>(a.v_pool);
  p.q = static_cast<const h16*>(a.q);
  p.out = static_cast<h16*>(a.out);
  p.seq_starts = a.seq_starts;
  p.prior_lens = a.prior_lens;
  p.bt = a.bt;
  p.bt_stride = a.bt_stride;
  p.items = reinterpret_cast<const int2*>(a.items);
  p.n_items = a.n_items;
  p.n_tokens = a.n_tokens;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = group;
  p.max_context = a.max_context;
  p.num_blocks = a.num_blocks;
  p.scale_log2 = a.scale * kLog2e * (a.fp8 ? a.k_scale : 1.0f);
  p.v_scale = a.fp8 ? a.v_scale : 1.0f;
  if (a.head_dim == 64) return a.fp8 ? launch_d<64, true>(p, a.max_items, s) : launch_d<64, false>(p, a.max_items, s);
  return a.fp8 ? launch_d<128, true>(p, a.max_items, s) : launch_d<128, false>(p, a.max_items, s);
}

}  // namespace pkv
