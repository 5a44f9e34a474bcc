#pragma once
// Device side of the paged GQA decode attention (the kernel body and its
// helpers), shared by the attention kernel (attn.hip) and the persistent
// small-batch layer kernel (persist.hip).  See attn.hip for the design.
#include "coherent.h"
#include "pkv_internal.h"

namespace pkv {
namespace {


typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x4 __attribute__((ext_vector_type(4)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;
// Partitions the merge reads per round trip.
constexpr int kMergeBatch = 8;

#ifdef PKV_ATTN_STAMPS
// measurement variant: wall-clock stamps per workgroup (start, context known,
// partition computed, end) and what it did
constexpr int kStampWgs = 16384;
static __device__ unsigned long long g_attn_stamps[kStampWgs * 6];
#define ATTN_STAMP(k) \
  do { if (threadIdx.x == 0 && wg < kStampWgs) { if ((k) == 1) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); \
       g_attn_stamps[wg * 6 + (k)] = wall_clock64(); } } while (0)
#define ATTN_STAMP_INFO(v) \
  do { if (threadIdx.x == 0 && wg < kStampWgs) { g_attn_stamps[wg * 6 + 4] = (v); g_attn_stamps[wg * 6 + 5] = __smid(); } } while (0)
#else
#define ATTN_STAMP(k) do {} while (0)
#define ATTN_STAMP_INFO(v) do {} while (0)
#endif

struct SplitParams {
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  const h16* q;
  h16* out;
  float* lse;
  const int* bt;
  const int* lens;
  int* counters;   // [B][Hkv] partitions arrived (zero between calls)
  float2* ws_ml;   // [B][Hq][P] (max, sum) per partition
  float* ws_o;     // [B][Hq][P][D] unnormalised O per partition
  int bt_stride;
  int batch, hq, hkv, group, part, n_parts_max;
  int num_blocks;    // blocks in the pool: a block id outside [0, num_blocks) is read as block 0
  int max_context;   // a longer context length is taken as max_context
  int worklist;      // work-list mode (attn_worklist): the grid takes the call's
                     // (row, KV head, partition) items longest rows first
  int merge_poll;    // every workgroup of the call is resident at once: the first
                     // partition of a row waits for the others and merges
  unsigned long long poll_ticks;  // its wait limit (wall-clock ticks; 0: publish at once)
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

// The 8-dim chunk that lane group q4 feeds at QK step s (D/32 steps).  f16 K
// is stored as [D/8][16 tokens][8 dims]: step s reads chunks 4s..4s+3.  fp8 K
// is stored as [D/16][16 tokens][16 dims]: one 16-byte load covers steps 2u and
// 2u+1, i.e. chunks 8u + 2 q4 and 8u + 2 q4 + 1.
template <bool FP8>
__device__ __forceinline__ int q_chunk(int s, int q4) {
  return FP8 ? 8 * (s >> 1) + 2 * q4 + (s & 1) : 4 * s + q4;
}

// Registers of one 16-token block for one lane (n = token of the K rows and
// dim-in-group of the V rows, q4 = lane group).
template <int D, bool FP8>
struct Tile;

template <int D>
struct Tile<D, false> {
  h16x8 k[D / 32];  // step s: token n, dims of chunk 4s + q4
  h16x4 v[D / 16];  // V^T[dim 16j + n][tokens 4*q4 .. +4]
  __device__ __forceinline__ void load_k(const SplitParams& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const h16* kp = reinterpret_cast<const h16*>(p.k_pool) + tile * kBlock * D + lane * 8;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) k[s] = *reinterpret_cast<const h16x8*>(kp + s * 512);
  }
  __device__ __forceinline__ void load_v(const SplitParams& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const h16* vp = reinterpret_cast<const h16*>(p.v_pool) + tile * D * kBlock + (lane & 15) * kBlock +
                    (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) v[j] = *reinterpret_cast<const h16x4*>(vp + j * 16 * kBlock);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const { return k[s]; }
  __device__ __forceinline__ h16x4 vfrag(int j) const { return v[j]; }
};

template <int D>
struct Tile<D, true> {
  int4 k[D / 64];  // 16 codes: token n, dims 16 (4u + q4) .. +16 (steps 2u, 2u + 1)
  int4 v[D / 64];  // 4 x 4 codes: V^T[dim 16j + n][tokens 4*q4 .. +4] for j = 4u .. 4u + 3
  __device__ __forceinline__ void load_k(const SplitParams& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const unsigned char* kp = p.k_pool + tile * kBlock * D + lane * 16;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) k[u] = *reinterpret_cast<const int4*>(kp + u * 1024);
  }
  __device__ __forceinline__ void load_v(const SplitParams& p, int blk, int g, int lane) {
    const size_t tile = (size_t)blk * p.hkv + g;
    const unsigned char* vp = p.v_pool + tile * D * kBlock + lane * 16;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) v[u] = *reinterpret_cast<const int4*>(vp + u * 1024);
  }
  __device__ __forceinline__ h16x8 kfrag(int s) const {
    const int4 w = k[s >> 1];
    return (s & 1) ? e4m3x8_to_h16x8(w.z, w.w) : e4m3x8_to_h16x8(w.x, w.y);
  }
  __device__ __forceinline__ h16x4 vfrag(int j) const {
    const int4 w = v[j >> 2];
    const int r = j & 3;
    return e4m3x4_to_h16x4(r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w);
  }
};

// Waves per SIMD each configuration is compiled for (register budget
// 512 / n): 4 waves x NT <= 4 keeps three workgroups per CU resident, which
// the plan's residency estimate relies on; the others hold one.
template <int NT, int W>
constexpr int attn_min_waves() {
  return (W == 4 && NT <= 4) ? 3 : 1;
}

// The work of one (row b, KV head g, partition part_idx) item, as a device
// function, so that the kernel, its work-list mode and a persistent kernel can
// run it (COH: q read and the output written with agent-scope accesses; every
// exit is uniform over the workgroup, and the caller separates two items with
// a workgroup barrier).  wg names the item in measurement builds only.
template <int D, bool FP8, int NT, int kWaves, bool COH>
__device__ __forceinline__ void attn_item(const SplitParams& p, const int wg, const int b, const int g,
                                          const int part_idx) {
  constexpr int kThreads = 64 * kWaves;
  ATTN_STAMP(0);
  // padded LDS row (floats) for the combine of the four waves
  constexpr int OSTR = D + 4;
  __shared__ float s_o[kWaves][kMaxGroup][OSTR];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;

  const int bg = b * p.hkv + g;
  const int tok0 = part_idx * p.part;
  const int hbase = g * p.group;
  // issued together, before the context length is known: the block-table
  // entries of this wave's blocks (clamped inside the row) and the query rows
  const int* btrow = p.bt + (size_t)b * p.bt_stride;
  // (a block id outside the pool, a caller error, reads block 0 instead)
  const int blk_raw = btrow[min(tok0 / kBlock + wave + kWaves * min(lane, NT - 1), p.bt_stride - 1)];
  const int blk_l = (unsigned)blk_raw < (unsigned)p.num_blocks ? blk_raw : 0;
  h16x8 qf[D / 32];
  {
    const h16* qrow = p.q + ((size_t)b * p.hq + hbase + min(n, p.group - 1)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = COH ? ld_agent_h8(qrow + 8 * q_chunk<FP8>(s, q4))
                  : *reinterpret_cast<const h16x8*>(qrow + 8 * q_chunk<FP8>(s, q4));
  }
  const int c = min(max(p.lens[b], 0), p.max_context);  // (out-of-range lengths clamped)
  ATTN_STAMP(1);
  if (tok0 >= c) {  // beyond the row's context (or an inactive row)
    ATTN_STAMP(3);
    ATTN_STAMP_INFO(0);
    if (c == 0 && g == 0 && part_idx == 0) {
      for (int idx = tid; idx < p.hq * D; idx += kThreads) {
        if constexpr (COH) st_agent_h(p.out + (size_t)b * p.hq * D + idx, (h16)0.f);
        else p.out[(size_t)b * p.hq * D + idx] = (h16)0.f;
      }
      if (p.lse)
        for (int h = tid; h < p.hq; h += kThreads) p.lse[(size_t)b * p.hq + h] = -INFINITY;
    }
    return;
  }
  if (n >= p.group) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const int np = (c + p.part - 1) / p.part;
  const int tok_end = min(c, tok0 + p.part);
  const int n_tiles = (tok_end - tok0 + kBlock - 1) / kBlock;
  const int my_tiles = wave < n_tiles ? (n_tiles - wave + kWaves - 1) / kWaves : 0;  // <= NT

#ifdef PKV_ATTN_QK_VALU
  // measurement variant (build.py --variant attn_qk_valu): the f16 scores on
  // the VALU, from the group's query rows in LDS
  __shared__ h16 s_qv[16][D + 8];
  __shared__ float s_sv[kWaves][2][16][17];
  if (!FP8 && wave == 0) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) *reinterpret_cast<h16x8*>(&s_qv[n][8 * (4 * s + q4)]) = qf[s];
  }
  __syncthreads();
#endif
  float m_w = -INFINITY, l_w = 0.f;  // this lane's head column (n), over the wave's tiles
  f32x4 o[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (my_tiles > 0) {  // wave-uniform
    if constexpr (FP8) {
      // (1) every K and then every V block of this wave in flight at once (a
      //     missing block re-reads the wave's last one, so the loads in flight
      //     never depend on data and the compiler waits for exactly the ones it
      //     uses); the scores start as soon as the K blocks land
      Tile<D, FP8> tl[NT];
      int blk[NT];
  #pragma unroll
      for (int t = 0; t < NT; ++t) blk[t] = __shfl(blk_l, min(t, my_tiles - 1), 64);
  #pragma unroll
      for (int t = 0; t < NT; ++t) tl[t].load_k(p, blk[t], g, lane);
  #pragma unroll
      for (int t = 0; t < NT; ++t) tl[t].load_v(p, blk[t], g, lane);

      // (2) scores S^T[token][head] of every block, in the log2 domain
      float x[NT][4];
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int s = 0; s < D / 32; ++s)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(tl[t].kfrag(s), qf[s], sacc, 0, 0, 0);
        const int tb = tok0 + (wave + kWaves * t) * kBlock + 4 * q4;  // this lane's first token
  #pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          x[t][rr] = (t < my_tiles && tb + rr < tok_end) ? sacc[rr] * p.scale_log2 : -INFINITY;
      }
      // (3) one max per head over the wave's tokens (in-lane, then the 4 lane groups)
      float mt = -INFINITY;
  #pragma unroll
      for (int t = 0; t < NT; ++t) mt = fmaxf(mt, fmaxf(fmaxf(x[t][0], x[t][1]), fmaxf(x[t][2], x[t][3])));
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      m_w = mt;
      // (4) P = exp2(S - m) and O^T += V^T P^T, no rescaling
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < my_tiles) {
          float pr[4];
  #pragma unroll
          for (int rr = 0; rr < 4; ++rr) pr[rr] = __builtin_amdgcn_exp2f(x[t][rr] - mt);
          l_w += (pr[0] + pr[1]) + (pr[2] + pr[3]);
          const h16x4 pf = h16x4{(h16)pr[0], (h16)pr[1], (h16)pr[2], (h16)pr[3]};
          const int tb = tok0 + (wave + kWaves * t) * kBlock + 4 * q4;
          if (tok0 + (wave + kWaves * t + 1) * kBlock > tok_end) {
            // the row's last, partial block: slots past the context may hold
            // anything (NaN included), so zero them before the product
  #pragma unroll
            for (int j = 0; j < D / 16; ++j) {
              h16x4 vf = tl[t].vfrag(j);
  #pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                if (tb + rr >= tok_end) vf[rr] = (h16)0.f;
              o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf, o[j], 0, 0, 0);
            }
          } else {
  #pragma unroll
            for (int j = 0; j < D / 16; ++j)
              o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(tl[t].vfrag(j), pf, o[j], 0, 0, 0);
          }
        }
      }
    } else {
      // f16: the wave's blocks in pairs (X, Y) = (t, t + 1).  The two score
      //     products of a pair take their 16 K rows in a permuted token order:
      //     row 4G + i of product A is token 8G + i of the pair (tokens 0-15
      //     of X, then 16-31 of Y) and row 4G + i of product B is token
      //     8G + 4 + i.  Lane group G then holds the scores of 8 consecutive
      //     tokens of one block, which is the k range it feeds as the B
      //     operand of v_mfma_f32_16x16x32_f16 for O^T += V^T P^T; the A
      //     operand is one 16-byte load of the dim-major V block per lane and
      //     16 dims.  No shuffles, and half the V load instructions of the
      //     16x16x16 product: a wave of 8 blocks issues 64 tile loads.
      constexpr int NP = NT / 2;
      int blk[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) blk[t] = __shfl(blk_l, min(t, my_tiles - 1), 64);
      const int rsel = n >> 3;                          // K row n: from Y (1) or X (0)
      const int rslot = 8 * ((n >> 2) & 1) + (n & 3);  // its slot in product A (B: + 4)
      const int vsel = q4 >> 1;                         // this lane's 8 tokens: Y (1) or X (0)
      const int vslot = 8 * (q4 & 1);                   // their first slot
      const h16* kpool = reinterpret_cast<const h16*>(p.k_pool);
      const h16* vpool = reinterpret_cast<const h16*>(p.v_pool);
      h16x8 ka[NP][D / 32], kb[NP][D / 32], vv[NP][D / 16];
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        const h16* kt = kpool + ((size_t)blk[2 * pr + rsel] * p.hkv + g) * kBlock * D + rslot * 8;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          ka[pr][s] = *reinterpret_cast<const h16x8*>(kt + (4 * s + q4) * kBlock * 8);
          kb[pr][s] = *reinterpret_cast<const h16x8*>(kt + (4 * s + q4) * kBlock * 8 + 32);
        }
      }
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        const h16* vt = vpool + ((size_t)blk[2 * pr + vsel] * p.hkv + g) * D * kBlock + n * kBlock + vslot;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) vv[pr][j] = *reinterpret_cast<const h16x8*>(vt + j * 16 * kBlock);
      }
      // scores of the lane's 8 tokens per pair (slots vslot .. vslot + 7 of
      // block 2 pr + vsel), log2 domain
      float xa[NP][4], xb[NP][4];
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
#ifdef PKV_ATTN_QK_VALU
        // each lane: v_dot2 over its 32 dims of K rows n (products A and B)
        // for every head, summed over the 4 lane groups, then moved through
        // LDS into the accumulator layout of the MFMA form
        f32x4 sa, sb;
        for (int h = 0; h < p.group; ++h) {
          float da = 0.f, db = 0.f;
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            const h16x8 qh = *reinterpret_cast<const h16x8*>(&s_qv[h][8 * (4 * s + q4)]);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              da = __builtin_amdgcn_fdot2(h16x2{ka[pr][s][e], ka[pr][s][e + 1]}, h16x2{qh[e], qh[e + 1]}, da, false);
              db = __builtin_amdgcn_fdot2(h16x2{kb[pr][s][e], kb[pr][s][e + 1]}, h16x2{qh[e], qh[e + 1]}, db, false);
            }
          }
          da += __shfl_xor(da, 16, 64);
          da += __shfl_xor(da, 32, 64);
          db += __shfl_xor(db, 16, 64);
          db += __shfl_xor(db, 32, 64);
          if (q4 == 0) {
            s_sv[wave][0][n][h] = da;
            s_sv[wave][1][n][h] = db;
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sa[i] = n < p.group ? s_sv[wave][0][4 * q4 + i][n] : 0.f;
          sb[i] = n < p.group ? s_sv[wave][1][4 * q4 + i][n] : 0.f;
        }
        __builtin_amdgcn_wave_barrier();
#else
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[pr][s], qf[s], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[pr][s], qf[s], sb, 0, 0, 0);
        }
#endif
        const int t = 2 * pr + vsel;
        const int tb = tok0 + (wave + kWaves * t) * kBlock + vslot;
        const bool tv = t < my_tiles;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xa[pr][i] = (tv && tb + i < tok_end) ? sa[i] * p.scale_log2 : -INFINITY;
          xb[pr][i] = (tv && tb + 4 + i < tok_end) ? sb[i] * p.scale_log2 : -INFINITY;
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int pr = 0; pr < NP; ++pr)
        mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(xa[pr][0], xa[pr][1]), fmaxf(xa[pr][2], xa[pr][3])),
                             fmaxf(fmaxf(xb[pr][0], xb[pr][1]), fmaxf(xb[pr][2], xb[pr][3]))));
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      m_w = mt;
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        if (2 * pr < my_tiles) {
          float pa[4], pb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pa[i] = __builtin_amdgcn_exp2f(xa[pr][i] - mt);
            pb[i] = __builtin_amdgcn_exp2f(xb[pr][i] - mt);
          }
          l_w += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
          const h16x8 pf = h16x8{(h16)pa[0], (h16)pa[1], (h16)pa[2], (h16)pa[3],
                                 (h16)pb[0], (h16)pb[1], (h16)pb[2], (h16)pb[3]};
          if (2 * pr + 1 < my_tiles && tok0 + (wave + kWaves * (2 * pr + 1) + 1) * kBlock <= tok_end) {
#pragma unroll
            for (int j = 0; j < D / 16; ++j)
              o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv[pr][j], pf, o[j], 0, 0, 0);
          } else {
            // the wave's last pair: a block past the wave's tiles (a re-read)
            // or slots past the context may hold anything (NaN included), so
            // zero them before the product
            const int t = 2 * pr + vsel;
            const int tb = tok0 + (wave + kWaves * t) * kBlock + vslot;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) {
              h16x8 vf = vv[pr][j];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (!(t < my_tiles && tb + e < tok_end)) vf[e] = (h16)0.f;
              o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, o[j], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // ---- combine the four lane groups' sums, then the four waves
  l_w += __shfl_xor(l_w, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    *reinterpret_cast<f32x4*>(&s_o[wave][n][16 * j + 4 * q4]) = o[j];
  if (q4 == 0) {
    s_m[wave][n] = m_w;
    s_l[wave][n] = l_w;
  }
  __syncthreads();
  ATTN_STAMP(2);

  const size_t bh0 = (size_t)b * p.hq + hbase;
  if (np == 1) {
    for (int idx = tid; idx < p.group * D; idx += kThreads) {
      const int h = idx / D, d = idx - h * D;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float e = __builtin_amdgcn_exp2f(s_m[w][h] - mx);  // 0 for a wave without tokens
        L += s_l[w][h] * e;
        O += s_o[w][h][d] * e;
      }
      if constexpr (COH) st_agent_h(p.out + (bh0 + h) * D + d, (h16)(O * p.v_scale / L));
      else p.out[(bh0 + h) * D + d] = (h16)(O * p.v_scale / L);
      if (d == 0 && p.lse) p.lse[bh0 + h] = (mx + __log2f(L)) * kLn2;
    }
    ATTN_STAMP(3);
    ATTN_STAMP_INFO(1);
    return;
  }

  // ---- this partition's (max, sum, O) per head, four dims per thread.
  // When every workgroup of the call is resident at once (and a thread holds
  // one (head, 4 dims) item), the row's first partition, a full one and so
  // the last to finish as a rule, keeps its own partial on chip, waits for
  // the others to arrive and merges: two memory round trips (publishing its
  // partial, counting its arrival) leave the critical path.  Otherwise, or
  // if that wait runs past its limit, every partition publishes and the last
  // to arrive merges.  Both merge the same values in partition order.
  const bool poll = p.merge_poll && part_idx == 0 && p.group * (D / 4) <= kThreads;  // uniform
  float2 own_ml = make_float2(-INFINITY, 0.f);
  f32x4 own_o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int idx = tid; idx < p.group * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float L = 0.f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = __builtin_amdgcn_exp2f(s_m[w][h] - mx);
      L += s_l[w][h] * e;
      O += *reinterpret_cast<const f32x4*>(&s_o[w][h][d]) * e;
    }
    own_ml = make_float2(mx, L);
    own_o = O * p.v_scale;
    if (!poll) {
      const size_t slot = (bh0 + h) * p.n_parts_max + part_idx;
      st_agent(p.ws_o + slot * D + d, own_o);
      if (d == 0) st_agent2(p.ws_ml + slot, own_ml);
    }
  }
  __shared__ int s_last;
  bool polled = false;
  if (poll) {
    if (tid == 0) {
      const unsigned long long t0 = wall_clock64();
      int ok = 0;
      while (p.poll_ticks > 0) {
        if (__hip_atomic_load(p.counters + bg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= np - 1) {
          ok = 1;
          break;
        }
        if (wall_clock64() - t0 > p.poll_ticks) break;
        __builtin_amdgcn_s_sleep(1);
      }
      s_last = ok;
    }
    __syncthreads();
    polled = s_last;
    if (!polled && tid < p.group * (D / 4)) {  // past the limit: publish like the others
      const int h = tid / (D / 4), d = 4 * (tid - h * (D / 4));
      const size_t slot = (bh0 + h) * p.n_parts_max + part_idx;
      st_agent(p.ws_o + slot * D + d, own_o);
      if (d == 0) st_agent2(p.ws_ml + slot, own_ml);
    }
  }
  if (!polled) {
    wait_vmcnt<0>();  // this thread's partial has reached the coherent level
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(p.counters + bg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    __syncthreads();
    if (!s_last) {
      ATTN_STAMP(3);
      ATTN_STAMP_INFO(2 + 16 * np);
      return;
    }
  }

  // ---- last partition of the row to finish: merge all np in partition order
  if (tid == 0) __hip_atomic_store(p.counters + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int idx = tid; idx < p.group * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    const size_t base = (bh0 + h) * p.n_parts_max;
    float M = -INFINITY, L = 0.f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < np; i0 += kMergeBatch) {
      // the (max, sum) and O of kMergeBatch partitions in flight together
      float2 ml[kMergeBatch];
      f32x4 po[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const size_t slot = base + min(i0 + u, np - 1);
        ml[u] = ld_agent2(p.ws_ml + slot);
        po[u] = ld_agent(p.ws_o + slot * D + d);
      }
      if (polled && i0 == 0) {  // partition 0 is this workgroup's own, never published
        ml[0] = own_ml;
        po[0] = own_o;
      }
      float mn = M;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u)
        if (i0 + u < np) mn = fmaxf(mn, ml[u].x);
      const float r = __builtin_amdgcn_exp2f(M - mn);  // 0 on the first batch (M = -inf)
      L *= r;
      O *= r;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (i0 + u < np) {
          const float e = __builtin_amdgcn_exp2f(ml[u].x - mn);
          L += ml[u].y * e;
          O += po[u] * e;
        }
      }
      M = mn;
    }
    const float inv = 1.0f / L;
    h16* o = p.out + (bh0 + h) * D + d;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (COH) st_agent_h(o + v, (h16)(O[v] * inv));
      else o[v] = (h16)(O[v] * inv);
    }
    if (d == 0 && p.lse) p.lse[bh0 + h] = (M + __log2f(L)) * kLn2;
  }
  ATTN_STAMP(3);
  ATTN_STAMP_INFO((polled ? 4 : 3) + 16 * np);
}

// The item of workgroup wg in the direct mapping, partition-major:
// wg = part * (B * Hkv) + b * Hkv + g.  The hardware dispatches workgroups in
// index order over a few microseconds, so every row's first (full) partition
// starts before any row's later, shorter one: attn15 19.0-19.6 -> 18.3-19.0
// us, 7B heads at batch 128 with 512-540-token contexts (second partitions of
// 15-28 tokens) 47.8 -> 40.7-41.4 us.  Results do not depend on the order.
template <int D, bool FP8, int NT, int kWaves, bool COH>
__device__ __forceinline__ void attn_body(const SplitParams& p, const int wg) {
  const int rows = p.batch * p.hkv;
  const int part_idx = wg / rows;
  const int bg = wg - part_idx * rows;
  const int b = bg / p.hkv;
  attn_item<D, FP8, NT, kWaves, COH>(p, wg, b, bg - b * p.hkv, part_idx);
}

// Work-list mode, for calls whose direct grid (every row's partitions counted
// at max_context) spans several rounds of resident workgroups.  The direct
// grid then spends a slot and a memory round trip on every partition past a
// shorter row's context, and the rows dispatched last finish with their
// merges at the very end.  Here a grid of resident workgroups reads the
// context lengths once, orders the rows by their partition count (longest
// first, ties by row), numbers the real items in that order (a row's items
// KV head by KV head, partitions in order within a head), and takes items
// from a shared counter: the long rows, whose merges read the most partials,
// run and merge first, short rows fill the end, and a workgroup that merges
// simply takes fewer items.  Every item is computed exactly as in the direct
// mapping.  An inactive row (length 0) is one item per KV head, which writes
// its zero output.  The counter and an exit count follow the arrival
// counters; the last workgroup to leave sets both back to zero.
constexpr int kWorklistMaxRows = 256;

template <int D, bool FP8, int NT, int kWaves>
__device__ __forceinline__ void attn_worklist(const SplitParams& p) {
  constexpr int kThreads = 64 * kWaves;
  __shared__ int s_np[kWorklistMaxRows];     // items of row r per KV head
  __shared__ int s_first[kWorklistMaxRows];  // first item of the row of rank k
  __shared__ int s_row[kWorklistMaxRows];    // the row of rank k
  __shared__ int s_total, s_item;
  const int tid = threadIdx.x;
  const int B = p.batch;
  int* work = p.counters + B * p.hkv;  // next item; then the exit count
  int next = 0;
  if (tid == 0) next = __hip_atomic_fetch_add(work, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int r = tid; r < B; r += kThreads) {
    const int c = min(max(p.lens[r], 0), p.max_context);
    s_np[r] = c > 0 ? (c + p.part - 1) / p.part : 1;
  }
  __syncthreads();
  for (int r = tid; r < B; r += kThreads) {
    const int nr = s_np[r];
    int rank = 0, before = 0;
    for (int j = 0; j < B; ++j) {
      const int nj = s_np[j];
      const bool ahead = nj > nr || (nj == nr && j < r);
      rank += ahead ? 1 : 0;
      before += ahead ? nj : 0;
    }
    s_row[rank] = r;
    s_first[rank] = before * p.hkv;
    if (rank == B - 1) s_total = (before + nr) * p.hkv;
  }
  if (tid == 0) s_item = next;
  __syncthreads();
  const int total = s_total;
  int item = s_item;
  while (item < total) {
    if (tid == 0) next = __hip_atomic_fetch_add(work, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int lo = 0, hi = B - 1;  // the last rank whose first item is <= item
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int r = s_row[lo], nr = s_np[r], j = item - s_first[lo];
    const int g = j / nr;
    attn_item<D, FP8, NT, kWaves, false>(p, item, r, g, j - g * nr);
    __syncthreads();  // the item's LDS is free again
    if (tid == 0) s_item = next;
    __syncthreads();
    item = s_item;
  }
  if (tid == 0 &&
      __hip_atomic_fetch_add(work + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
    // every workgroup has taken its last item: reset for the next call
    __hip_atomic_store(work, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(work + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Kernel arguments from the call's arguments and plan (workspace: counters,
// then the (max, sum) and O partials).
inline SplitParams make_split_params(const AttnArgs& a, const AttnPlan& plan) {
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
  sp.num_blocks = a.num_blocks;
  sp.max_context = plan.max_context;
  // the 8-wave plans keep the whole grid within one workgroup per CU
  sp.merge_poll = plan.waves == 8 && !plan.worklist ? 1 : 0;
  sp.worklist = 0;  // set by the work-list launch
  sp.poll_ticks = attn_merge_wait_ticks;
  sp.scale_log2 = a.scale * kLog2e * (a.fp8 ? a.k_scale : 1.0f);
  sp.v_scale = a.fp8 ? a.v_scale : 1.0f;
  const size_t ml = align_up((size_t)a.batch * a.hq * plan.n_parts_max * sizeof(float2), 256);
  char* ws = static_cast<char*>(a.ws);
  const size_t cr = a.counter_region ? a.counter_region : plan.counter_bytes;
  sp.counters = reinterpret_cast<int*>(ws);
  sp.ws_ml = reinterpret_cast<float2*>(ws + cr);
  sp.ws_o = reinterpret_cast<float*>(ws + cr + ml);
  return sp;
}

}  // namespace
}  // namespace pkv
