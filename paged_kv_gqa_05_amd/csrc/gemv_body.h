#pragma once
// Device side of the small-batch projections (the GEMV body, its epilogues
// and helpers), shared by the GEMV kernel (linear.hip) and the persistent
// small-batch layer kernel (persist.hip).  See linear.hip for the design.
#include "linear.h"

namespace pkv {
namespace {


typedef _Float16 h16;
typedef h16 h16x8 __attribute__((ext_vector_type(8)));
typedef h16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot8(h16x8 a, h16x8 b, float c) {
  c = __builtin_amdgcn_fdot2(h16x2{a[0], a[1]}, h16x2{b[0], b[1]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[2], a[3]}, h16x2{b[2], b[3]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[4], a[5]}, h16x2{b[4], b[5]}, c, false);
  c = __builtin_amdgcn_fdot2(h16x2{a[6], a[7]}, h16x2{b[6], b[7]}, c, false);
  return c;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Writes one output element (row m, logical column col) given the
// accumulators.  COH: outputs (and the residual read) go through agent-scope
// accesses, for a persistent kernel whose next phase reads them on other XCDs.
template <int EPI, bool COH>
__device__ __forceinline__ void epilogue(const LinArgs& a, int m, int col, float y0, float y1) {
  h16* o = static_cast<h16*>(a.out) + (size_t)m * a.ldo + col;
  if constexpr (EPI == EPI_F16) {
    if (a.bias) y0 += (float)a.bias[col];
    if constexpr (COH) st_agent_h(o, (h16)y0); else *o = (h16)y0;
  } else if constexpr (EPI == EPI_RESID) {
    if constexpr (COH) st_agent_h(o, (h16)((float)ld_agent_h(o) + y0)); else *o = (h16)((float)*o + y0);
  } else if constexpr (EPI == EPI_SILU) {
    if constexpr (COH) st_agent_h(o, (h16)(silu(y0) * y1)); else *o = (h16)(silu(y0) * y1);
  } else {  // EPI_ROPE
    RopeRow r = rope_row_len(a.rope, m);
    rope_row_blk(a.rope, m, r);
    const float2 cs = rope_cs(a.rope, r, col);
    const float2 b = rope_bias(a.rope, a.bias, col);
    rope_put<COH>(a.rope, r, m, col, y0 + b.x, y1 + b.y, cs);
  }
}

// ------------------------------------------------------------------ GEMV

// LPR lanes per output row (pair), 16 to 256: a row spans a quarter wave up
// to the whole 4-wave workgroup.  Lane l of the row reads the chunks
// k = 8 l + j * 8 LPR, so every step of the row covers 16 LPR contiguous
// bytes.  LPR is sized so that a lane's whole share of the row (at most U
// chunks) is loaded in one go: HBM latency is hidden by the bytes each lane
// keeps in flight, not by other waves (at batch 1 a GEMV has few waves per
// SIMD).  The gain, activation and weight loads of an iteration are issued
// before any is used and are unconditional (past the row end they are
// clamped to its last chunk and masked to zero afterwards; batch rows past M
// read row M - 1 and are never stored), because a load under a branch makes
// the compiler drain every load in flight before it.
//
// The body is a device function of the workgroup's block index so that a
// persistent kernel can run it for several blocks (COH: activations read and
// outputs written with agent-scope accesses; the caller separates two calls
// with a workgroup barrier, since waves of a row leave early).
template <int LPR, int MT, int U, int EPI, bool NORM, bool COH>
__device__ __forceinline__ void gemv_body(const LinArgs& a, const int block) {
  constexpr bool PAIR = epi_pair(EPI);
  constexpr int STEP = LPR * 8;
  constexpr int NV = PAIR ? 2 * MT : MT;  // values reduced per row
  const int tid = threadIdx.x;
  const int lig = tid % LPR;
  const int col_raw = block * (256 / LPR) + tid / LPR;
  const int col = min(col_raw, a.n_out - 1);  // rows past the end compute row n_out - 1, never stored
  const h16* w0 = a.W + (size_t)(PAIR ? pair_row(EPI == EPI_ROPE, a.n_out, a.rope.d, col, 0) : col) * a.K;
  const h16* w1 = PAIR ? a.W + (size_t)pair_row(EPI == EPI_ROPE, a.n_out, a.rope.d, col, 1) * a.K : w0;
  const h16* xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xrow[m] = a.A + (size_t)min(m, a.M - 1) * a.lda;
  // At batch <= 4 the epilogue's inputs are fetched ahead of the weights: the
  // QKV rows' context lengths and bias (the block id and the (cos, sin) that
  // depend on the length follow once the weights are consumed, while the
  // lanes reduce), and the residual of the O and down projections.  Fetched in
  // the epilogue they were a chain of memory round trips after the reduction.
  constexpr bool EARLY = MT <= 4 && (EPI == EPI_ROPE || EPI == EPI_RESID);
  [[maybe_unused]] RopeRow rr[EARLY && EPI == EPI_ROPE ? MT : 1];
  [[maybe_unused]] float2 rcs[EARLY && EPI == EPI_ROPE ? MT : 1], rbias;
  [[maybe_unused]] float res[EARLY && EPI == EPI_RESID ? MT : 1];
  if constexpr (EARLY && EPI == EPI_ROPE) {
#pragma unroll
    for (int m = 0; m < MT; ++m) rr[m] = rope_row_len(a.rope, min(m, a.M - 1));
    rbias = rope_bias(a.rope, a.bias, col);
  }
  if constexpr (EARLY && EPI == EPI_RESID) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const h16* rp = static_cast<const h16*>(a.out) + (size_t)min(m, a.M - 1) * a.ldo + col;
      res[m] = COH ? (float)ld_agent_h(rp) : (float)*rp;
    }
  }
  float acc0[MT], acc1[MT], ss[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc0[m] = acc1[m] = ss[m] = 0.f;
  const h16x8 zero = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const int n_iter = (a.K + U * STEP - 1) / (U * STEP);
  for (int it = 0; it < n_iter; ++it) {
    const int kb = lig * 8 + it * U * STEP;
    int kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kk[u] = min(kb + u * STEP, a.K - 8);
    h16x8 gv[U], xv[U][MT], wv0[U], wv1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NORM) gv[u] = *reinterpret_cast<const h16x8*>(a.gain + kk[u]);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xv[u][m] = COH ? ld_agent_h8(xrow[m] + kk[u]) : *reinterpret_cast<const h16x8*>(xrow[m] + kk[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wv0[u] = __builtin_nontemporal_load(reinterpret_cast<const h16x8*>(w0 + kk[u]));
      if constexpr (PAIR) wv1[u] = __builtin_nontemporal_load(reinterpret_cast<const h16x8*>(w1 + kk[u]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = kb + u * STEP < a.K;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const h16x8 x = valid ? xv[u][m] : zero;
        if constexpr (NORM) ss[m] = dot8(x, x, ss[m]);
        const h16x8 xg = NORM ? x * gv[u] : x;
        acc0[m] = dot8(valid ? wv0[u] : zero, xg, acc0[m]);
        if constexpr (PAIR) acc1[m] = dot8(valid ? wv1[u] : zero, xg, acc1[m]);
      }
    }
  }
  if constexpr (EARLY && EPI == EPI_ROPE) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      rope_row_blk(a.rope, min(m, a.M - 1), rr[m]);
      rcs[m] = rope_cs(a.rope, rr[m], col);
    }
  }
  // reduce over the row's lanes: within the wave, then across waves in LDS
  constexpr int LW = LPR < 64 ? LPR : 64;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int o = LW / 2; o > 0; o >>= 1) {
      acc0[m] += __shfl_xor(acc0[m], o, 64);
      if (PAIR) acc1[m] += __shfl_xor(acc1[m], o, 64);
      if (NORM) ss[m] += __shfl_xor(ss[m], o, 64);
    }
  }
  if constexpr (LPR > 64) {
    constexpr int WPR = LPR / 64;  // waves per row
    __shared__ float red[4][NV + MT];
    const int wave = tid >> 6, lane = tid & 63;
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        red[wave][m] = acc0[m];
        if (PAIR) red[wave][MT + m] = acc1[m];
        if (NORM) red[wave][NV + m] = ss[m];
      }
    }
    __syncthreads();
    if (wave % WPR) return;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc0[m] = acc1[m] = ss[m] = 0.f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) {
        acc0[m] += red[wave + w][m];
        if (PAIR) acc1[m] += red[wave + w][MT + m];
        if (NORM) ss[m] += red[wave + w][NV + m];
      }
    }
  }
  if (col_raw >= a.n_out) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < a.M && (m % LW) == lig) {
      const float r = NORM ? rsqrtf(ss[m] / (float)a.K + a.eps) : 1.0f;
      if constexpr (EARLY && EPI == EPI_ROPE) {
        rope_put<COH>(a.rope, rr[m], m, col, acc0[m] * r + rbias.x, acc1[m] * r + rbias.y, rcs[m]);
      } else if constexpr (EARLY && EPI == EPI_RESID) {
        h16* o = static_cast<h16*>(a.out) + (size_t)m * a.ldo + col;
        if constexpr (COH) st_agent_h(o, (h16)(res[m] + acc0[m] * r)); else *o = (h16)(res[m] + acc0[m] * r);
      } else {
        epilogue<EPI, COH>(a, m, col, acc0[m] * r, acc1[m] * r);
      }
    }
  }
}

}  // namespace
}  // namespace pkv
