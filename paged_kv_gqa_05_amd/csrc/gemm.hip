// Batched projections (batch >= 32) on MFMA: y = W a with W [rows][K] f16
// row-major, fp32 accumulation, the RMSNorm fused in front and the consumer op
// fused behind (rvLLM post on discuss.pytorch.kr, section "퓨즈드 CUDA 커널":
// Add+RMSNorm+QKV, Add+RMSNorm+GateUp and SiLU*Mul+Down are single kernels;
// zingnex.cn article, section 直接GPU调用: batched projections are f16 GEMMs).
//
// Structure (one workgroup of 4 waves per MT x NT output tile and K range):
//  * Stages of 64 K elements.  A stage holds MT activation rows and NT weight
//    rows of 128 bytes each, copied from global memory straight into LDS with
//    the gfx950 direct-to-LDS load (global_load_lds_dwordx4): no VGPRs are
//    spent on staging, so NS stages are kept in flight.  Each load writes 1 KB
//    = 8 rows; lane i fetches the 16-byte chunk (i%8) ^ (i/8) of row i/8, so the
//    chunk c of row r lands in slot c ^ (r%8) (XOR swizzle: the fragment reads
//    below are free of bank conflicts) and every load covers 8 whole 128-byte
//    lines of global memory.
//  * 2 x 2 waves, each (MT/2) x (NT/2) of the tile with
//    v_mfma_f32_16x16x32_f16; both operands are read from LDS with one
//    ds_read_b128 per lane and fragment.
//  * RMSNorm by linearity: W (g . h * r) = r * (W (g . h)).  The gain g is
//    staged with the stage (one 128-byte row per wave) and multiplied into the
//    activation fragments; sum(h^2) accumulates from the same fragments and the
//    row scale r = 1/sqrt(mean(h^2) + eps) is applied in the epilogue.
//  * Split-K: when the weight matrix alone cannot fill the chip, the K range is
//    cut into S parts.  Each part writes its fp32 tile (and partial sum(h^2))
//    to the workspace; the last part to finish a tile (per-tile arrival
//    counter, reset by that same workgroup) adds the S parts in a fixed order
//    and runs the epilogue, so results do not depend on arrival order.
//  * Balance (tiles of up to 64 rows): when the tiles are more than the CUs
//    but not a whole number of rounds, the whole rounds run as they are and
//    the remaining tiles are split over K (the last round is a fraction of a
//    tile, not a tile).
//  * Tile order is XCD-aware: the hardware deals workgroups round-robin over
//    the 8 XCDs; each XCD takes a contiguous range of whole tiles, then a
//    contiguous range of split parts, M tiles fastest, so the M tiles that
//    share a weight tile share one L2.
#include <algorithm>

#include "coherent.h"
#include "linear.h"

namespace pkv {
namespace {

typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BK = 64;     // K elements per stage (one 128-byte chunk of a row)
constexpr int kCUs = 256;  // compute units of an MI355X (8 XCDs x 32)

__device__ __forceinline__ float dot8(h16x8 a, h16x8 b, float c) {
  c = __builtin_amdgcn_fdot2(h16x2{a[0], a[1]}, h16x2{b[0], b[1]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[2], a[3]}, h16x2{b[2], b[3]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[4], a[5]}, h16x2{b[4], b[5]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[6], a[7]}, h16x2{b[6], b[7]}, c, false);
  return c;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// One direct-to-LDS load: every lane copies the 16 bytes at g to LDS address
// m0 + 16 * lane, where m0 = lds (wave-uniform).  Written as inline asm so that
// the compiler does not treat later LDS reads as possibly aliasing an
// in-flight copy (it would drain every copy before each read, which removes
// the pipelining); completion is tracked explicitly with wait_vmcnt.
__device__ __forceinline__ void load_to_lds(const void* g, const _Float16* lds) {
  const unsigned off = (unsigned)(size_t)(lds_char*)(lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(off) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global load).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Wait for this wave's LDS reads (lgkmcnt 0), leaving vector-memory loads in flight.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

template <int MT, int NT, int NS, int EPI, bool NORM, int WM, int WN>
struct Cfg {
  static constexpr bool PAIR = epi_pair(EPI);
  static constexpr int WV = WM * WN;                  // waves per workgroup
  static constexpr int WTM = MT / WM, WTN = NT / WN;  // wave tile
  static constexpr int FM = WTM / 16, FN = WTN / 16;  // 16 x 16 fragments per wave
  static constexpr int ROWS = MT + NT;
  static constexpr int LPS = ROWS / (8 * WV);         // 8-row loads per wave per stage
  static constexpr int LPW = LPS + (NORM ? 1 : 0);    // + the gain row
  static constexpr int GAIN_OFF = ROWS * BK;          // f16 offset of the per-wave gain rows
  static constexpr int STAGE = ROWS * BK + (NORM ? WV * BK : 0);  // f16 per stage
  static_assert(ROWS % (8 * WV) == 0 && FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "tile shape");
  static_assert(!PAIR || (FN % 2 == 0), "paired tiles need an even fragment count");
  static_assert(NS >= 2 && (NS - 2) * LPW < 64, "stages");
  // Registers of one stage's fragments and of the accumulators (per lane).
  // Two fragment sets are kept (PIPE, see the main loop) when they fit, with
  // 64 registers for the rest, in a wave's share of its SIMD's 512 at the
  // number of workgroups per CU that the LDS allows: more registers then cost
  // no resident workgroup.
  static constexpr int FRAG_REGS = (2 * FM + 2 * FN + (NORM ? 2 : 0)) * 4;
  static constexpr int ACC_REGS = FM * FN * 4;
  static constexpr int LDS_BYTES = NS * STAGE * 2 + MT * 4 + 64;
  static constexpr int WG_LDS = (160 * 1024) / LDS_BYTES;
  static constexpr int WG_PER_CU = WG_LDS < 1 ? 1 : (WG_LDS > 32 / WV ? 32 / WV : WG_LDS);
  static constexpr int REG_BUDGET = 512 / ((WG_PER_CU * WV + 3) / 4);  // per wave, waves per SIMD rounded up
  static constexpr bool PIPE = 2 * FRAG_REGS + ACC_REGS + 64 <= REG_BUDGET;
};

// Wait until at most `pending` stages (of LPW loads each) are still in flight;
// pending in [0, NPEND] (s_waitcnt takes an immediate).
template <int NPEND, int LPW>
__device__ __forceinline__ void wait_stage(int pending) {
  if constexpr (NPEND > 0) {
    if (pending >= NPEND) {
      wait_vmcnt<NPEND * LPW>();
      return;
    }
    wait_stage<NPEND - 1, LPW>(pending);
  } else {
    wait_vmcnt<0>();
  }
}

template <int MT, int NT, int NS, int EPI, bool NORM, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) gemm_kernel(GemmParams p) {
  using C = Cfg<MT, NT, NS, EPI, NORM, WM, WN>;
  constexpr int WV = C::WV;
  constexpr bool PAIR = C::PAIR;
  constexpr int FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(1024))) h16 smem[NS * C::STAGE];
  __shared__ float s_ss[MT];
  __shared__ int s_last;

  // ---- tile of this workgroup (XCD-aware order, M tiles fastest)
  const int L = blockIdx.x, xcd = L & 7, li = L >> 3;
  const int n_kc = (p.K + BK - 1) / BK;
  int mt, nt, sp = 0, splits = 1, kc_per = n_kc;
  if (li < p.full_per_xcd) {  // a whole tile
    if (p.blk_m > 0) {
      // blocks of 32 tiles (blk_m along M), dealt round-robin to the XCDs:
      // the 32 workgroups an XCD runs at once share their activation and
      // weight rows through its L2
      const int k = 8 * (li >> 5) + xcd, w = li & 31;
      mt = (k % p.nbm) * p.blk_m + w % p.blk_m;
      nt = (k / p.nbm) * (32 / p.blk_m) + w / p.blk_m;
      if (mt >= p.n_mt || nt >= p.nt_full) return;
    } else {
      const int t = xcd * p.full_per_xcd + li;
      if (t >= p.nt_full * p.n_mt) return;
      mt = t % p.n_mt;
      nt = t / p.n_mt;
    }
  } else {  // a K range of a split tile
    const int u = xcd * p.per_xcd + (li - p.full_per_xcd);
    if (u >= p.split_items) return;
    splits = p.splits;
    kc_per = p.kc_per_split;
    mt = u % p.n_mt;
    const int rest = u / p.n_mt;
    sp = rest % splits;
    nt = p.nt_full + rest / splits;
  }
  const int m0 = mt * MT;
  const int kc0 = sp * kc_per;
  const int n_iter = min(n_kc, kc0 + kc_per) - kc0;  // >= 1 by construction

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- per-lane sources of this wave's direct-to-LDS row loads
  // load j of wave w covers stage rows 8 * (WV j + w) .. + 8
  const int lrow = lane >> 3;                  // row within the 8-row group
  const int lchunk = (lane & 7) ^ lrow;        // 16-byte chunk this lane fetches
  const h16* src[C::LPS];
#pragma unroll
  for (int j = 0; j < C::LPS; ++j) {
    const int r = 8 * (WV * j + wave) + lrow;  // stage row
    if (r < MT) {
      src[j] = p.A + (size_t)min(m0 + r, p.M - 1) * p.lda;
    } else {
      const int t = r - MT;
      int wr;
      if (PAIR) {
        const int jj = min(nt * (NT / 2) + (t % (NT / 2)), p.n_out - 1);
        wr = pair_row(EPI == EPI_ROPE, p.n_out, p.rope.d, jj, t >= NT / 2);
      } else {
        wr = min(nt * NT + t, p.n_out - 1);
      }
      src[j] = p.W + (size_t)wr * p.K;
    }
  }
  const int kmax = p.K - 8;  // last valid 8-element chunk start

  auto issue = [&](int it) {
    const int buf = it % NS;
    const int kbase = (kc0 + it) * BK;
    const int k = min(kbase + 8 * lchunk, kmax);
    h16* sb = smem + buf * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::LPS; ++j) load_to_lds(src[j] + k, sb + (WV * j + wave) * 8 * BK);
    if constexpr (NORM) {
      if (lane < 8) {  // this wave's copy of the 64 gain values of the stage
        const int kg = min(kbase + 8 * lane, kmax);
        load_to_lds(p.gain + kg, sb + C::GAIN_OFF + wave * BK);
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) ss[i] = 0.f;

  // fragment rows (stage row index) of this lane
  const int fr = lane & 15, fg = lane >> 4;
  int arow[FM], wrow_t[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * C::WTM + i * 16 + fr;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int t;
    if (PAIR) {
      t = (j < FN / 2) ? wn * (NT / (2 * WN)) + j * 16 : NT / 2 + wn * (NT / (2 * WN)) + (j - FN / 2) * 16;
    } else {
      t = wn * C::WTN + j * 16;
    }
    wrow_t[j] = MT + t + fr;
  }

  // The fragments of one stage for this lane (both 32-wide k steps, and with
  // the norm the gain chunks), read from LDS ...
  struct Frag {
    h16x8 af[2][FM], wf[2][FN], g[2];
  };
  auto read_frags = [&](int it, Frag& f) {
    const h16* sb = smem + (it % NS) * C::STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + fg;  // logical 16-byte chunk of this lane
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = arow[i];
        f.af[s][i] = *reinterpret_cast<const h16x8*>(sb + r * BK + ((c ^ (r & 7)) * 8));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wrow_t[j];
        f.wf[s][j] = *reinterpret_cast<const h16x8*>(sb + r * BK + ((c ^ (r & 7)) * 8));
      }
      if constexpr (NORM) f.g[s] = *reinterpret_cast<const h16x8*>(sb + C::GAIN_OFF + wave * BK + 8 * c);
    }
  };
  // ... and their products (chunks past K are zero; with the norm, sum(h^2)
  // of the raw activations, then the gain applied)
  auto mma = [&](int it, Frag& f) {
    const int kbase = (kc0 + it) * BK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * s + fg;
      if (kbase + 8 * c >= p.K) {
#pragma unroll
        for (int i = 0; i < FM; ++i) f.af[s][i] = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
      if constexpr (NORM) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          ss[i] = dot8(f.af[s][i], f.af[s][i], ss[i]);
          f.af[s][i] = f.af[s][i] * f.g[s];
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.af[s][i], f.wf[s][j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- main loop: NS - 1 stages in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n_iter) issue(s);
  if constexpr (C::PIPE) {
    // With one or two waves per SIMD nothing hides a wave's LDS read latency,
    // so the fragments of stage it are read while the products of stage
    // it - 1 run (two fragment sets in registers).  Before the barrier that
    // lets a stage's slot be refilled, each wave waits for its own reads of
    // that slot.  Same products in the same order as reading and multiplying
    // one stage at a time.
    Frag fa, fb;
    auto step = [&](int it, Frag& cur, Frag& prev) {
      const int pending = min(n_iter - 1, it + NS - 2) - it;
      wait_stage<NS - 2, C::LPW>(pending);
      wait_lds();
      barrier_only();
      if (it + NS - 1 < n_iter) issue(it + NS - 1);
      read_frags(it, cur);
      if (it > 0) mma(it - 1, prev);
    };
    int it = 0;
    for (; it + 1 < n_iter; it += 2) {
      step(it, fa, fb);
      step(it + 1, fb, fa);
    }
    if (it < n_iter) {
      step(it, fa, fb);
      mma(it, fa);
    } else {
      mma(it - 1, fb);
    }
  } else {
    // one 32-wide k step at a time: half the fragment registers
    auto compute = [&](int it) {
      const h16* sb = smem + (it % NS) * C::STAGE;
      const int kbase = (kc0 + it) * BK;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 4 * s + fg;
        const bool kin = kbase + 8 * c < p.K;
        h16x8 af[FM], wf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = arow[i];
          af[i] = *reinterpret_cast<const h16x8*>(sb + r * BK + ((c ^ (r & 7)) * 8));
          if (!kin) af[i] = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wrow_t[j];
          wf[j] = *reinterpret_cast<const h16x8*>(sb + r * BK + ((c ^ (r & 7)) * 8));
        }
        if constexpr (NORM) {
          const h16x8 g = *reinterpret_cast<const h16x8*>(sb + C::GAIN_OFF + wave * BK + 8 * c);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            ss[i] = dot8(af[i], af[i], ss[i]);
            af[i] = af[i] * g;
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
      }
    };
    for (int it = 0; it < n_iter; ++it) {
      const int pending = min(n_iter - 1, it + NS - 2) - it;
      wait_stage<NS - 2, C::LPW>(pending);
      barrier_only();
      if (it + NS - 1 < n_iter) issue(it + NS - 1);
      compute(it);
    }
  }

  // ---- sum(h^2) per activation row: reduce the four k-groups of a row
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      ss[i] += __shfl_xor(ss[i], 16, 64);
      ss[i] += __shfl_xor(ss[i], 32, 64);
    }
  }

  const int tile = mt + p.n_mt * (nt - p.nt_full);  // index among the split tiles
  if (splits > 1) {
    // partial tile in the accumulator layout: lane-contiguous float4s
    constexpr int TILE_F = MT * NT;
    float* part = p.part + ((size_t)tile * splits + sp) * TILE_F + wave * (FM * FN * 256);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) st_agent(part + ((i * FN + j) * 64 + lane) * 4, acc[i][j]);
    if constexpr (NORM) {
      if (wn == 0 && fg == 0) {
        float* ssp = p.part_ss + ((size_t)tile * splits + sp) * MT;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          __hip_atomic_store(ssp + arow[i], ss[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    wait_vmcnt<0>();  // this thread's partials have reached the coherent level
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(p.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               splits - 1;
    __syncthreads();
    if (!s_last) return;
    // the last part: add all parts in split order
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // G parts in flight at a time, added in split order
    constexpr int G = (FM * FN >= 8) ? 1 : (FM * FN >= 4 ? 2 : 4);
    for (int q0 = 0; q0 < splits; q0 += G) {
      f32x4 t[G][FM][FN];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int q = min(q0 + u, splits - 1);
        const float* pq = p.part + ((size_t)tile * splits + q) * TILE_F + wave * (FM * FN * 256);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) t[u][i][j] = ld_agent(pq + ((i * FN + j) * 64 + lane) * 4);
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (q0 + u < splits) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] += t[u][i][j];
        }
      }
    }
    if constexpr (NORM) {
      if (wn == 0 && fg == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float t = 0.f;
          for (int q = 0; q < splits; ++q)
            t += __hip_atomic_load(p.part_ss + ((size_t)tile * splits + q) * MT + arow[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          ss[i] = t;
        }
      }
    }
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (NORM) {
    if (wn == 0 && fg == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i) s_ss[arow[i]] = rsqrtf(ss[i] / (float)p.K + p.eps);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds column fr of each fragment, rows 4 fg + v.
  // Every load the epilogue needs is issued before its first store: a load
  // cannot be moved above a store to a possibly aliasing pointer, so an
  // interleaved load-modify-store costs one memory round trip per element.
  int mrow[FM][4];
  bool mok[FM][4];
  float rs[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ml = wm * C::WTM + i * 16 + 4 * fg + v;
      mok[i][v] = m0 + ml < p.M;
      mrow[i][v] = min(m0 + ml, p.M - 1);
      rs[i][v] = NORM ? s_ss[ml] : 1.0f;
    }
  if constexpr (EPI == EPI_ROPE) {
    constexpr int FP = FN / 2;  // pair fragments
    int pc[FP];
    bool pok[FP];
#pragma unroll
    for (int j = 0; j < FP; ++j) {
      const int col = nt * (NT / 2) + wn * (NT / (2 * WN)) + j * 16 + fr;
      pok[j] = col < p.n_out;
      pc[j] = min(col, p.n_out - 1);
    }
    float2 bias[FP];
#pragma unroll
    for (int j = 0; j < FP; ++j) bias[j] = rope_bias(p.rope, p.bias, pc[j]);
    // metadata in groups of RG fragment rows (all of them up to 4 row x pair
    // fragments a lane; one at a time above, where a whole tile's worth
    // would not fit in registers)
    constexpr int RG = FM * FP <= 4 ? FM : 1;
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += RG) {
      RopeRow rr[RG][4];
#pragma unroll
      for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v) rr[ii][v] = rope_row_len(p.rope, mrow[i0 + ii][v]);
#pragma unroll
      for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v) rope_row_blk(p.rope, mrow[i0 + ii][v], rr[ii][v]);
      float2 cs[RG][4][FP];
#pragma unroll
      for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < FP; ++j) cs[ii][v][j] = rope_cs(p.rope, rr[ii][v], pc[j]);
#pragma unroll
      for (int ii = 0; ii < RG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < FP; ++j)
            if (mok[i0 + ii][v] && pok[j])
              rope_put(p.rope, rr[ii][v], mrow[i0 + ii][v], pc[j], acc[i0 + ii][j][v] * rs[i0 + ii][v] + bias[j].x,
                       acc[i0 + ii][j + FP][v] * rs[i0 + ii][v] + bias[j].y, cs[ii][v][j]);
    }
  } else if constexpr (EPI == EPI_SILU) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int col = nt * (NT / 2) + wn * (NT / (2 * WN)) + j * 16 + fr;
          if (mok[i][v] && col < p.n_out) {
            const float g = acc[i][j][v] * rs[i][v], u = acc[i][j + FN / 2][v] * rs[i][v];
            static_cast<h16*>(p.out)[(size_t)mrow[i][v] * p.ldo + col] = (h16)(silu(g) * u);
          }
        }
  } else {
    int cc[FN];
    bool cok[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = nt * NT + wn * C::WTN + j * 16 + fr;
      cok[j] = col < p.n_out;
      cc[j] = min(col, p.n_out - 1);
    }
    // EPI_F16: the bias of each column; EPI_RESID: the residual h itself.
    // Loaded in groups of FG fragment rows (all of them up to 8 fragments a
    // lane; one at a time above, where a whole tile's worth would spill).
    constexpr int FG = FM * FN <= 8 ? FM : 1;
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += FG) {
      float add[FG][4][FN];
#pragma unroll
      for (int ii = 0; ii < FG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (EPI == EPI_F16)
              add[ii][v][j] = p.bias ? (float)p.bias[cc[j]] : 0.f;
            else
              add[ii][v][j] = (float)static_cast<const h16*>(p.out)[(size_t)mrow[i0 + ii][v] * p.ldo + cc[j]];
          }
#pragma unroll
      for (int ii = 0; ii < FG; ++ii)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (mok[i0 + ii][v] && cok[j])
              static_cast<h16*>(p.out)[(size_t)mrow[i0 + ii][v] * p.ldo + cc[j]] =
                  (h16)(acc[i0 + ii][j][v] * rs[i0 + ii][v] + add[ii][v][j]);
    }
  }
}

template <int MT, int NT, int NS, int EPI, int WM = 2, int WN = 2>
hipError_t launch_cfg(const GemmParams& gp, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<MT, NT, NS, EPI, epi_norm(EPI), WM, WN>), dim3((gp.full_per_xcd + gp.per_xcd) * 8),
                     dim3(64 * WM * WN), 0, s, gp);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmPlan& pl, const GemmParams& gp, hipStream_t s) {
  switch (pl.cfg) {
    case GEMM_32x64: return launch_cfg<32, 64, 4, EPI>(gp, s);
    case GEMM_64x128: return launch_cfg<64, 128, 3, EPI>(gp, s);
    case GEMM_128x128: return launch_cfg<128, 128, 2, EPI, 4, 2>(gp, s);
    case GEMM_128x256: return launch_cfg<128, 256, 3, EPI, 2, 4>(gp, s);
    // plans the planner picks for gate/up (EPI_SILU) or O/down (EPI_RESID) only
    case GEMM_128x128_S3:
      if constexpr (EPI == EPI_SILU || EPI == EPI_RESID) return launch_cfg<128, 128, 3, EPI, 4, 2>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_128x160:
      if constexpr (EPI == EPI_SILU) return launch_cfg<128, 160, 3, EPI, 4, 1>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_64x64:
      if constexpr (EPI == EPI_RESID) return launch_cfg<64, 64, 4, EPI, 2, 2>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_32x96:
      if constexpr (EPI == EPI_SILU) return launch_cfg<32, 96, 4, EPI, 2, 1>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_32x160:
      if constexpr (EPI == EPI_SILU) return launch_cfg<32, 160, 4, EPI, 2, 1>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_64x96:
      if constexpr (EPI == EPI_SILU) return launch_cfg<64, 96, 4, EPI, 4, 1>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_64x160:
      if constexpr (EPI == EPI_SILU) return launch_cfg<64, 160, 3, EPI, 4, 1>(gp, s);
      return hipErrorInvalidValue;
    case GEMM_256x256:  // not for the QKV epilogue (its per-row RoPE state would need scratch)
      if constexpr (EPI != EPI_ROPE) return launch_cfg<256, 256, 2, EPI, 4, 2>(gp, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tile shape and K split for an M x rows x K projection (host only).
// Tile table, measured at the 1.5B decode shapes (batch 64, 128, 256, weights
// rotated so the Infinity Cache cannot hold them): 32 x 64 tiles with 4 stages
// (2 x 2 waves), 64 x 128 with 3 stages (2 x 2), 128 x 128 with 2 stages (4 x 2
// waves: two workgroups per CU).  Small tiles win until they exceed ~1024
// tiles (the grid then re-reads the activations from L2 too often).  Long
// reductions (K >= 4096, split over K) start at 64 x 128 from batch 128 up:
// fewer partial tiles to merge (down projection, batch 256: 23 us vs 32 us).
// When 64 x 128 would already need 512 tiles or more, 128 x 128 (gate/up at
// batch 256: 37 us vs 41 us; LM head).  No tile is taller than the batch
// rounded up to 32.  Prefill-sized long reductions (K >= 4096 with at least
// 256 tiles of 128 x 256) take 128 x 256 tiles with 3 stages on 2 x 4 waves:
// the deeper pipeline pays over the long K (down projection, 32768 rows:
// 934 us vs 1645 us with 128 x 128 and 2 stages).  So do all projections of
// more than 1024 rows (32768 rows at the 1.5B shape: QKV 390 -> 328 us, O 252
// -> 239 us, gate/up 2918 -> 2734 us: half the stage bytes per flop).
GemmPlan gemm_plan(int M, int n_out, int K, int epi) {
  const bool pair = epi_pair(epi);
  static const int kCfg[3][3] = {{GEMM_32x64, 32, 64}, {GEMM_64x128, 64, 128}, {GEMM_128x128, 128, 128}};
  auto tiles_of = [&](int c) { return ceil_div(M, kCfg[c][1]) * ceil_div(n_out, pair ? kCfg[c][2] / 2 : kCfg[c][2]); };
  const int m_cap = ceil_div(M, 32) * 32;
  int c = 0;
  if (K >= 4096 && M >= 128) c = 1;
  while (c < 2 && kCfg[c + 1][1] <= m_cap && tiles_of(c) >= (c == 1 ? 512 : 1024)) ++c;
  GemmPlan pl{};
  pl.cfg = kCfg[c][0];
  pl.mt = kCfg[c][1];
  pl.nt = kCfg[c][2];
  if ((K >= 4096 || M > 1024) && ceil_div(M, 128) * ceil_div(n_out, pair ? 128 : 256) >= 256) {
    pl.cfg = GEMM_128x256;
    pl.mt = 128;
    pl.nt = 256;
    // prefill-sized projections other than QKV: 256 x 256 tiles on 4 x 2
    // waves, a third fewer stage bytes per flop again (32768 rows at the 1.5B
    // shape: gate/up 2631 -> 2074 us, down 1107 -> 907 us, O 216 -> 174 us;
    // QKV with RoPE was slower, 450 -> 571 us)
    if (epi != EPI_ROPE && M > 1024 && ceil_div(M, 256) * ceil_div(n_out, pair ? 128 : 256) >= 256) {
      pl.cfg = GEMM_256x256;
      pl.mt = 256;
    }
  }
  // gate/up (paired rows) at batch 97..1024: 128-row tiles 128 or 160 weight
  // rows wide, whichever loads fewer stage bytes on the busiest CU (rounds of
  // the 256 CUs x rows per stage).  Bound by each CU's stage loads, the
  // per-CU bytes set the time: 280 tiles of 128 x 128 leave 24 CUs with two
  // tiles, 224 tiles of 128 x 160 fit one round (gate/up at batch 256: 38.2
  // -> 30.6 us; 7B gate/up at batch 128: 85.7 -> 64.2 us).  A single round
  // holds one workgroup per CU, which affords a third stage (gate/up at batch
  // 128: 27.8 -> 25.1 us with 128 x 128).  These plans are never split.
  bool whole = false;
  // gate/up at batch <= 64: tiles as tall as the batch (32 or 64 rows) and 96
  // or 160 weight rows wide, by the same busiest-CU stage-byte count, when
  // that fills at least half the CUs (1.5B at batch 64: 64 x 96, 187 tiles,
  // 20.2 -> 16.5 us; 7B at batch 64: 64 x 160, 237 tiles, 62.5 -> 51.0 us;
  // 7B at batch 32: 32 x 160, 51.3 -> 49.9 us)
  if (epi == EPI_SILU && m_cap <= 64) {
    const int mt = m_cap, nm = ceil_div(M, mt);
    const int t96 = nm * ceil_div(n_out, 48), t160 = nm * ceil_div(n_out, 80);
    const long c96 = (long)ceil_div(t96, kCUs) * (mt + 96), c160 = (long)ceil_div(t160, kCUs) * (mt + 160);
    const bool wide = c160 < c96;
    if ((wide ? t160 : t96) >= kCUs / 2) {
      pl.cfg = mt == 32 ? (wide ? GEMM_32x160 : GEMM_32x96) : (wide ? GEMM_64x160 : GEMM_64x96);
      pl.mt = mt;
      pl.nt = wide ? 160 : 96;
      whole = true;
    }
  }
  if (epi == EPI_SILU && pl.cfg != GEMM_128x256 && m_cap >= 128 && M <= 1024) {
    const int t128 = ceil_div(M, 128) * ceil_div(n_out, 64), t160 = ceil_div(M, 128) * ceil_div(n_out, 80);
    const long c128 = (long)ceil_div(t128, kCUs) * 256, c160 = (long)ceil_div(t160, kCUs) * 288;
    if (c160 < c128) {
      pl.cfg = GEMM_128x160;
      pl.mt = 128;
      pl.nt = 160;
      whole = true;
    } else if (t128 <= kCUs) {
      pl.cfg = GEMM_128x128_S3;
      pl.mt = 128;
      pl.nt = 128;
      whole = true;
    }
  }
  // O and down projections over long reductions (K >= 3072) at decode batches:
  // of four tile shapes, each with its split count by the rules below, the
  // one with the fewest stage bytes on the busiest CU (rounds of the CUs x
  // stages per part x bytes per stage) plus twice the fp32 partial bytes the
  // last part of a tile reads back.  Measured over the O and down shapes of
  // the 1.5B and 7B models at batch 32-256 it keeps or beats every earlier
  // plan (7B down at batch 64: 64 x 64 tiles, 42.7 -> 35.0 us; at batch 256:
  // 3-stage 128 x 128 tiles, 80.1 -> 64.7 us; 1.5B down at batch 128: 64 x
  // 64 tiles, 21.9 -> 18.8 us).
  int planned_splits = 0;
  if (epi == EPI_RESID && K >= 3072 && M <= 1024) {
    static const int kRes[4][3] = {
        {GEMM_32x64, 32, 64}, {GEMM_64x64, 64, 64}, {GEMM_64x128, 64, 128}, {GEMM_128x128_S3, 128, 128}};
    const int kc = ceil_div(K, 64);
    long best = -1;
    for (const auto& r : kRes) {
      const int mt = r[1], nt = r[2], nm = ceil_div(M, mt), t = nm * ceil_div(n_out, nt);
      if (mt > m_cap || t > kGemmMaxCounters) continue;
      const int cap = (mt <= 32 && t >= 96 && nm > 1) ? 2 * kCUs : kCUs;
      int sp = 1;
      while (t * (sp + 1) <= cap && kc / (sp + 1) >= 4 && sp < 16) ++sp;
      const int per = ceil_div(kc, sp);
      sp = ceil_div(kc, per);
      const long cost = (long)ceil_div(t * sp, kCUs) * per * (mt + nt) * 128 + (sp > 1 ? 2L * sp * mt * nt * 4 : 0);
      if (best < 0 || cost < best) {
        best = cost;
        pl.cfg = r[0];
        pl.mt = mt;
        pl.nt = nt;
        planned_splits = sp;
      }
    }
  }
  pl.n_mt = ceil_div(M, pl.mt);
  pl.n_nt = ceil_div(n_out, pair ? pl.nt / 2 : pl.nt);
  const int n_kc = ceil_div(K, 64);
  const int tiles = pl.n_mt * pl.n_nt;
  // split K while the grid holds fewer than ~one workgroup per CU and every
  // part keeps at least 4 stages; a split tile needs an arrival counter
  int splits = 1;
  if (planned_splits > 0) {
    splits = planned_splits;
  } else if (K < 3072) {
    // short reductions: as many parts as keep the grid within one workgroup
    // per CU and every part at least 6 stages (1.5B O projection at batch
    // 256: 1 part, 11.0 -> 10.0 us; at batch 32: 4 parts, 7.5 -> 7.1 us)
    while (!whole && tiles * (splits + 1) <= kCUs && n_kc >= 6 * (splits + 1) && splits < 16 &&
           tiles <= kGemmMaxCounters)
      ++splits;
  } else if (pl.n_mt == 1) {
    // one row of tiles: a grid a little over one workgroup per CU leaves the
    // CUs that get two with twice the stages (7B at batch 32: QKV 3 parts 12.3
    // us vs 4 parts 15.3 us; O 4 vs 5 parts 10.5 vs 13.7 us; down 4 vs 8 parts
    // 29.6 vs 31.6 us), so the grid stays within one workgroup per CU
    while (!whole && tiles * (splits + 1) <= kCUs && n_kc / (splits + 1) >= 4 && splits < 16 &&
           tiles <= kGemmMaxCounters)
      ++splits;
  } else {
    // several rows of tiles: within one workgroup per CU, or two for 32-row
    // tiles when there are at least 96 of them (they sit two to a CU: 7B at
    // batch 64, QKV 3 parts (432 workgroups) 16.7 us vs 2 parts (288) 20.4 us;
    // O 4 parts 13.7 vs 3 parts 15.1 us).  Grids a little over a multiple of
    // 256 leave some CUs with twice the stages (7B down projection at batch
    // 128 with 64 x 128 tiles: 4 parts 48.3 us, 5 parts 71 us, 8 parts 58 us).
    const int cap = (pl.mt <= 32 && tiles >= 96) ? 2 * kCUs : kCUs;
    while (!whole && tiles * (splits + 1) <= cap && n_kc / (splits + 1) >= 4 && splits < 16 &&
           tiles <= kGemmMaxCounters)
      ++splits;
  }
  pl.nt_full = splits > 1 ? 0 : pl.n_nt;
  // more tiles than CUs but not whole rounds: the whole rounds stay as they
  // are and the last, partial round is split over K.  Only for tiles of up to
  // 64 rows, which sit two or three to a CU: decode step at batch 64 1.95 ->
  // 1.89 ms.  With 128 x 128 tiles the split parts share CUs with the whole
  // tiles and slowed gate/up at batch 256 (38.9 -> 42.1 us).
  int split_tiles = splits > 1 ? tiles : 0;
  if (splits == 1 && !whole && planned_splits == 0 && pl.mt <= 64 && tiles > kCUs && tiles % kCUs != 0 &&
      (tiles / kCUs * kCUs) % pl.n_mt == 0) {
    const int rem = tiles % kCUs;
    const int s = std::min(kCUs / rem, n_kc / 2);
    if (s >= 2 && rem <= kGemmMaxCounters) {
      pl.nt_full = tiles / kCUs * kCUs / pl.n_mt;
      splits = s;
      split_tiles = rem;
    }
  }
  pl.kc_per_split = ceil_div(n_kc, splits);
  pl.splits = ceil_div(n_kc, pl.kc_per_split);  // every part non-empty
  pl.part_bytes = pl.splits > 1
                      ? align_up((size_t)split_tiles * pl.splits * pl.mt * pl.nt * 4, 256) +
                            align_up((size_t)split_tiles * pl.splits * pl.mt * 4, 256)
                      : 0;
  return pl;
}

hipError_t launch_gemm(const LinArgs& a, int epi, const GemmPlan& pl, void* part_ws, int* counters,
                       hipStream_t s) {
  GemmParams gp{};
  gp.A = a.A; gp.W = a.W; gp.gain = a.gain; gp.bias = a.bias; gp.out = a.out;
  gp.M = a.M; gp.K = a.K; gp.lda = a.lda; gp.ldo = a.ldo; gp.n_out = a.n_out;
  gp.eps = a.eps;
  gp.rope = a.rope;
  gp.n_mt = pl.n_mt; gp.n_nt = pl.n_nt; gp.nt_full = pl.nt_full;
  gp.splits = pl.splits; gp.kc_per_split = pl.kc_per_split;
  gp.full_per_xcd = ceil_div(pl.nt_full * pl.n_mt, 8);
  // grids of many rounds of whole tiles (prefill): blocks of 32 tiles, 4 x 8
  // (8 x 4 for tiles wider than tall), so that an XCD's concurrent
  // workgroups share both operands through its L2
  if (pl.splits == 1 && pl.nt_full * pl.n_mt >= 4 * kCUs) {
    gp.blk_m = pl.mt < pl.nt ? 8 : 4;
    if (pl.n_mt >= gp.blk_m && pl.nt_full >= 32 / gp.blk_m) {
      gp.nbm = ceil_div(pl.n_mt, gp.blk_m);
      const int blocks = gp.nbm * ceil_div(pl.nt_full, 32 / gp.blk_m);
      gp.full_per_xcd = ceil_div(blocks, 8) * 32;
    } else {
      gp.blk_m = 0;
    }
  }
  gp.split_items = pl.splits > 1 ? (pl.n_nt - pl.nt_full) * pl.n_mt * pl.splits : 0;
  gp.per_xcd = ceil_div(gp.split_items, 8);
  gp.counters = counters;
  if (pl.splits > 1) {
    const size_t split_tiles = (size_t)(pl.n_nt - pl.nt_full) * pl.n_mt;
    gp.part = static_cast<float*>(part_ws);
    gp.part_ss = reinterpret_cast<float*>(static_cast<char*>(part_ws) +
                                          align_up(split_tiles * pl.splits * pl.mt * pl.nt * 4, 256));
  }
  switch (epi) {
    case EPI_F16: return launch_epi<EPI_F16>(pl, gp, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(pl, gp, s);
    case EPI_SILU: return launch_epi<EPI_SILU>(pl, gp, s);
    case EPI_ROPE: return launch_epi<EPI_ROPE>(pl, gp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
