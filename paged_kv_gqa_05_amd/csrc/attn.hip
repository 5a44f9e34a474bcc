// Paged GQA decode attention for gfx950: split over the context + merge pass.
//
// What it computes (rvLLM post on discuss.pytorch.kr, section
// "PagedAttention과 FlashAttention-3": block-table KV cache, GQA reads each KV
// head once for its whole group of query heads, f16 KV or FP8 E4M3 KV):
//   out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) V_t,  t < context_lens[b]
// with K_t, V_t gathered through the row's block table.
//
// Design (MI355X, not the pages' FlashAttention-3 kernels):
//  * One workgroup (4 waves) per (row b, KV head g, partition of `part`
//    tokens).  Workgroup ids are mapped onto the list of non-empty partitions
//    (a prefix sum over the rows' partition counts), so active work is packed
//    at the front of the grid whatever the context-length mix.
//  * Each wave takes every 4th 16-token block of the partition.  The block's
//    K tile [16][D] feeds v_mfma_f32_16x16x32_f16 directly from registers as
//    the A operand (token = MFMA row, 8 contiguous dims per lane), the group's
//    query rows (G <= 16, zero padded) are the B operand, giving S^T
//    [token][head].  That C layout is exactly the B operand of
//    v_mfma_f32_16x16x16f16 for O^T += V^T P^T, whose A operand is read from
//    the dim-major V block [D][16] with one 8-byte load per 16 dims.  No LDS
//    staging and no shuffles between the two products.
//  * Online softmax in the log2 domain per head column; the running max lives
//    in the four lanes of a column, the running sum per lane.  The four waves'
//    (max, sum, O) are combined through LDS at the end.
//  * A row with a single partition writes its normalised f16 output directly;
//    otherwise the partition writes (max, sum, unnormalised O) in fp32 and the
//    merge kernel combines them.  Nothing is zero-filled.
//  * FP8 E4M3 codes are converted to f16 in registers with the gfx950
//    conversion instruction (exact: every E4M3 value is an f16 value); the
//    per-tensor K scale is folded into the score scale and the V scale into
//    the output.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;

struct SplitParams {
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  const h16* q;
  h16* out;
  float* lse;
  const int* bt;
  const int* lens;
  float2* ws_ml;
  float* ws_o;
  int bt_stride;
  int batch, hq, hkv, group, part, n_parts_max;
  float scale_log2;  // softmax scale * log2(e) * K dequant scale
  float v_scale;     // V dequant scale (1 for f16)
};

// Two E4M3 codes (low or high 16 bits of w) -> two f16, exactly.
template <bool HI>
__device__ __forceinline__ h16x2 e4m3x2_to_h16x2(int w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

__device__ __forceinline__ h16x4 e4m3x4_to_h16x4(int w) {
  const h16x2 a = e4m3x2_to_h16x2<false>(w), b = e4m3x2_to_h16x2<true>(w);
  return h16x4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ h16x8 e4m3x8_to_h16x8(int lo, int hi) {
  const h16x4 a = e4m3x4_to_h16x4(lo), b = e4m3x4_to_h16x4(hi);
  return h16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Registers of one 16-token tile for one lane.
template <int D, bool FP8>
struct Tile;

template <int D>
struct Tile<D, false> {
  h16x8 k[D / 32];  // K[token n][dims q4*D/4 + 8s .. +8]
  h16x4 v[D / 16];  // V^T[dim 16j + n][tokens 4*q4 .. +4]
  __device__ __forceinline__ void load(const SplitParams& p, int blk, int g, int n, int q4) {
    const h16* kp = reinterpret_cast<const h16*>(p.k_pool) +
                    ((size_t)(blk * p.hkv + g) * kBlock + n) * D + q4 * (D / 4);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) k[s] = *reinterpret_cast<const h16x8*>(kp + 8 * s);
    const h16* vp = reinterpret_cast<const h16*>(p.v_pool) +
                    (size_t)(blk * p.hkv + g) * D * kBlock + n * kBlock + q4 * 4;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) v[j] = *reinterpret_cast<const h16x4*>(vp + j * 16 * kBlock);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const { return k[s]; }
  __device__ __forceinline__ h16x4 vfrag(int j) const { return v[j]; }
};

template <int D>
struct Tile<D, true> {
  int4 k[D / 64];  // 16 codes per int4: dims q4*D/4 + 16i .. +16
  int v[D / 16];   // 4 codes: V^T[dim 16j + n][tokens 4*q4 .. +4]
  __device__ __forceinline__ void load(const SplitParams& p, int blk, int g, int n, int q4) {
    const unsigned char* kp =
        p.k_pool + ((size_t)(blk * p.hkv + g) * kBlock + n) * D + q4 * (D / 4);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) k[i] = *reinterpret_cast<const int4*>(kp + 16 * i);
    const unsigned char* vp = p.v_pool + (size_t)(blk * p.hkv + g) * D * kBlock + n * kBlock + q4 * 4;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) v[j] = *reinterpret_cast<const int*>(vp + j * 16 * kBlock);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const {
    const int4 w = k[s >> 1];
    return (s & 1) ? e4m3x8_to_h16x8(w.z, w.w) : e4m3x8_to_h16x8(w.x, w.y);
  }
  __device__ __forceinline__ h16x4 vfrag(int j) const { return e4m3x4_to_h16x4(v[j]); }
};

// Inclusive block-wide prefix sum of one int per thread (256 threads).
__device__ __forceinline__ int block_incl_scan(int x, int* s_wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wsum[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    int v = s_wsum[w];
    pre += (w < wave) ? v : 0;
    tot += v;
  }
  *total = tot;
  __syncthreads();
  return x + pre;
}

template <int D, bool FP8>
__global__ void __launch_bounds__(kThreads) attn_split_kernel(SplitParams p) {
  constexpr int OSTR = D + 4;  // padded LDS row (floats)
  __shared__ float s_o[kWaves][kMaxGroup][OSTR];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_item[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;

  // ---- map this workgroup onto the packed list of (row, kv head, partition)
  const int wg = blockIdx.x;
  if (tid == 0) s_item[0] = -1;
  int carry = 0;
  for (int base = 0; base < p.batch; base += kThreads) {
    const int b = base + tid;
    const int cnt = (b < p.batch) ? (p.lens[b] + p.part - 1) / p.part * p.hkv : 0;
    int total;
    const int incl = block_incl_scan(cnt, s_wsum, &total) + carry;
    if (cnt > 0 && wg >= incl - cnt && wg < incl) {
      s_item[0] = b;
      s_item[1] = incl - cnt;
    }
    carry += total;
    __syncthreads();
    if (s_item[0] >= 0) break;  // uniform: read after the barrier
  }
  const int b = s_item[0];
  if (b < 0) return;
  const int c = p.lens[b];
  const int np = (c + p.part - 1) / p.part;
  const int r = wg - s_item[1];
  const int g = r / np, part_idx = r - g * np;

  const int tok0 = part_idx * p.part;
  const int tok_end = min(c, tok0 + p.part);
  const int n_tiles = (tok_end - tok0 + kBlock - 1) / kBlock;
  const int hbase = g * p.group;

  // ---- query rows of this group as the B operand of the QK^T product
  h16x8 qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    if (n < p.group) {
      qf[s] = *reinterpret_cast<const h16x8*>(p.q + ((size_t)b * p.hq + hbase + n) * D +
                                              q4 * (D / 4) + 8 * s);
    } else {
      qf[s] = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int my_tiles = wave < n_tiles ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
  const int* btrow = p.bt + (size_t)b * p.bt_stride + tok0 / kBlock;
  const int blk_l = lane < my_tiles ? btrow[wave + kWaves * lane] : 0;

  Tile<D, FP8> cur, nxt;
  if (my_tiles > 0) cur.load(p, __shfl(blk_l, 0, 64), g, n, q4);
  for (int t = 0; t < my_tiles; ++t) {
    if (t + 1 < my_tiles) nxt.load(p, __shfl(blk_l, t + 1, 64), g, n, q4);
    const int i = wave + kWaves * t;

    // S^T[token][head] over the head dim
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.kfrag(s), qf[s], sacc, 0, 0, 0);

    const int tb = tok0 + i * kBlock + 4 * q4;  // this lane's first token
    float x[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) x[rr] = (tb + rr < tok_end) ? sacc[rr] * p.scale_log2 : -INFINITY;
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pr[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) pr[rr] = __builtin_amdgcn_exp2f(x[rr] - m_new);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j) o[j] *= alpha;
    }
    m_run = m_new;
    const h16x4 pf = h16x4{(h16)pr[0], (h16)pr[1], (h16)pr[2], (h16)pr[3]};

    const bool partial = (tok0 + (i + 1) * kBlock > tok_end);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      h16x4 vf = cur.vfrag(j);
      if (partial) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (tb + rr >= tok_end) vf[rr] = (h16)0.f;
      }
      o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf, o[j], 0, 0, 0);
    }
    if (t + 1 < my_tiles) cur = nxt;
  }

  // ---- combine the four lane groups' sums, then the four waves
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    *reinterpret_cast<f32x4*>(&s_o[wave][n][16 * j + 4 * q4]) = o[j];
  if (q4 == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_run;
  }
  __syncthreads();

  const bool single = (np == 1);
  for (int idx = tid; idx < p.group * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    float mw[kWaves];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = s_m[w][h];
      mx = fmaxf(mx, mw[w]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = __builtin_amdgcn_exp2f(mw[w] - mx);
      L += s_l[w][h] * e;
      O += s_o[w][h][d] * e;
    }
    const size_t bh = (size_t)b * p.hq + hbase + h;
    if (single) {
      p.out[bh * D + d] = (h16)(O * p.v_scale / L);
      if (d == 0 && p.lse) p.lse[bh] = (mx + __log2f(L)) * kLn2;
    } else {
      const size_t slot = bh * p.n_parts_max + part_idx;
      p.ws_o[slot * D + d] = O * p.v_scale;
      if (d == 0) p.ws_ml[slot] = make_float2(mx, L);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(D) attn_merge_kernel(SplitParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.hq;
  const int d = threadIdx.x;
  const int c = p.lens[b];
  if (c == 0) {  // inactive row
    p.out[(size_t)bh * D + d] = (h16)0.f;
    if (d == 0 && p.lse) p.lse[bh] = -INFINITY;
    return;
  }
  const int np = (c + p.part - 1) / p.part;
  if (np == 1) return;  // written by the split kernel
  const float2* ml = p.ws_ml + (size_t)bh * p.n_parts_max;
  const float* po = p.ws_o + (size_t)bh * p.n_parts_max * D + d;
  float mx = -INFINITY;
  for (int i = 0; i < np; ++i) mx = fmaxf(mx, ml[i].x);
  float L = 0.f, O = 0.f;
  for (int i = 0; i < np; ++i) {
    const float2 v = ml[i];
    const float e = __builtin_amdgcn_exp2f(v.x - mx);
    L += v.y * e;
    O += po[(size_t)i * D] * e;
  }
  p.out[(size_t)bh * D + d] = (h16)(O / L);
  if (d == 0 && p.lse) p.lse[bh] = (mx + __log2f(L)) * kLn2;
}

template <int D, bool FP8>
hipError_t launch_impl(const SplitParams& sp, const AttnPlan& plan, hipStream_t s) {
  if (plan.grid > 0) {
    hipLaunchKernelGGL((attn_split_kernel<D, FP8>), dim3(plan.grid), dim3(kThreads), 0, s, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(sp.batch * sp.hq), dim3(D), 0, s, sp);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int batch, int hq, int hkv, int head_dim, int elt_bytes, int max_context) {
  (void)hq;
  AttnPlan p{};
  // About 128 KB of K+V per workgroup, but shrink partitions (down to 64
  // tokens) while the whole grid would hold fewer than 1024 workgroups.
  const int bytes_per_token = 2 * head_dim * elt_bytes;
  int part = 64;
  while (part * 2 * bytes_per_token <= 128 * 1024 && part * 2 <= 4096) part *= 2;
  const int mc = max_context > 0 ? max_context : 1;
  while (part > 64 && (long)batch * hkv * ceil_div(mc, part) < 1024) part /= 2;
  p.part = part;
  p.n_parts_max = ceil_div(mc, part);
  p.grid = batch * hkv * p.n_parts_max;
  const size_t ml = align_up((size_t)batch * hq * p.n_parts_max * sizeof(float2), 256);
  const size_t o = align_up((size_t)batch * hq * p.n_parts_max * head_dim * sizeof(float), 256);
  p.ws_bytes = ml + o;
  return p;
}

hipError_t launch_paged_attention(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  SplitParams sp{};
  sp.k_pool = static_cast<const unsigned char*>(a.k_pool);
  sp.v_pool = static_cast<const unsigned char*>(a.v_pool);
  sp.q = static_cast<const h16*>(a.q);
  sp.out = static_cast<h16*>(a.out);
  sp.lse = a.lse;
  sp.bt = a.bt;
  sp.lens = a.lens;
  sp.bt_stride = a.bt_stride;
  sp.batch = a.batch;
  sp.hq = a.hq;
  sp.hkv = a.hkv;
  sp.group = a.hq / a.hkv;
  sp.part = plan.part;
  sp.n_parts_max = plan.n_parts_max;
  sp.scale_log2 = a.scale * kLog2e * (a.fp8 ? a.k_scale : 1.0f);
  sp.v_scale = a.fp8 ? a.v_scale : 1.0f;
  const size_t ml = align_up((size_t)a.batch * a.hq * plan.n_parts_max * sizeof(float2), 256);
  sp.ws_ml = static_cast<float2*>(a.ws);
  sp.ws_o = reinterpret_cast<float*>(static_cast<char*>(a.ws) + ml);
  if (a.head_dim == 128) {
    return a.fp8 ? launch_impl<128, true>(sp, plan, s) : launch_impl<128, false>(sp, plan, s);
  }
  return a.fp8 ? launch_impl<64, true>(sp, plan, s) : launch_impl<64, false>(sp, plan, s);
}

}  // namespace pkv
