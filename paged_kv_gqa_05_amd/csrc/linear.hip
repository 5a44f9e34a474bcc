// Projections of the decode step: y = W a with W [out][in] f16 row-major and
// fp32 accumulation, with the RMSNorm fused in front and the op that consumes
// y fused behind (rvLLM post on discuss.pytorch.kr, section "퓨즈드 CUDA 커널":
// Add+RMSNorm+QKV, Add+RMSNorm+GateUp and SiLU*Mul+Down are single kernels;
// zingnex.cn article, section 直接GPU调用: batched projections are f16 GEMMs).
//
// Norm fusion.  RMSNorm(h) * w scales each row by one number, so
//   W (w . h * r) = r * (W (w . h)),   r = 1 / sqrt(mean(h^2) + eps).
// The kernel multiplies each activation chunk by the gain as it streams
// through, accumulates sum(h^2) of the same chunk with v_dot2 (every workgroup
// sees whole rows of the activations), and scales the accumulator by r in the
// epilogue.  No separate norm pass and no normalised-activation buffer.
//
// Epilogues: ROPE (QKV rows in rotation pairs (i, i + D/2): + bias, RoPE of
// q and k at the row's position, q out, the new token's k and v into the
// paged cache), RESID (h = f16(h + y) in place: the residual add of the next
// norm), SILU (rows [gate | up]: act = f16(silu(g) * u)), F16 (logits).
//
// This file holds the GEMV for batch < 32: a group of 16 to 256 lanes
// streams one output row of W (one row pair for SILU / ROPE) with 16-byte
// loads and v_dot2 against every batch row, then reduces across its lanes.
// Batches of 32 and more go to the MFMA GEMM in gemm.hip.
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

// Writes one output element (row m, logical column col) given the accumulators.
template <int EPI>
__device__ __forceinline__ void epilogue(const LinArgs& a, int m, int col, float y0, float y1) {
  if constexpr (EPI == EPI_F16) {
    if (a.bias) y0 += (float)a.bias[col];
    static_cast<h16*>(a.out)[(size_t)m * a.ldo + col] = (h16)y0;
  } else if constexpr (EPI == EPI_RESID) {
    h16* p = static_cast<h16*>(a.out) + (size_t)m * a.ldo + col;
    *p = (h16)((float)*p + y0);
  } else if constexpr (EPI == EPI_SILU) {
    static_cast<h16*>(a.out)[(size_t)m * a.ldo + col] = (h16)(silu(y0) * y1);
  } else {  // EPI_ROPE
    rope_store(a.rope, a.bias, m, col, y0, y1);
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
template <int LPR, int MT, int U, int EPI, bool NORM>
__global__ void __launch_bounds__(256) gemv_kernel(LinArgs a) {
  constexpr bool PAIR = epi_pair(EPI);
  constexpr int STEP = LPR * 8;
  constexpr int NV = PAIR ? 2 * MT : MT;  // values reduced per row
  const int tid = threadIdx.x;
  const int lig = tid % LPR;
  const int col_raw = blockIdx.x * (256 / LPR) + tid / LPR;
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
    for (int m = 0; m < MT; ++m) res[m] = (float)static_cast<const h16*>(a.out)[(size_t)min(m, a.M - 1) * a.ldo + col];
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
      for (int m = 0; m < MT; ++m) xv[u][m] = *reinterpret_cast<const h16x8*>(xrow[m] + kk[u]);
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
      if constexpr (EARLY && EPI == EPI_ROPE)
        rope_put(a.rope, rr[m], m, col, acc0[m] * r + rbias.x, acc1[m] * r + rbias.y, rcs[m]);
      else if constexpr (EARLY && EPI == EPI_RESID)
        static_cast<h16*>(a.out)[(size_t)m * a.ldo + col] = (h16)(res[m] + acc0[m] * r);
      else
        epilogue<EPI>(a, m, col, acc0[m] * r, acc1[m] * r);
    }
  }
}

// Batch buckets: MT rows, U steps per iteration with MT * U <= 32 activation
// chunks held in registers (U_MAX at MT = 1).
template <int LPR, int EPI, bool NORM, int U_MAX>
hipError_t gemv_dispatch_mt(const LinArgs& a, hipStream_t s) {
  const int grid = (a.n_out + 256 / LPR - 1) / (256 / LPR);
#define PKV_GEMV(MT_, U_) \
  hipLaunchKernelGGL((gemv_kernel<LPR, MT_, U_, EPI, NORM>), dim3(grid), dim3(256), 0, s, a)
  if (a.M <= 1) PKV_GEMV(1, U_MAX);
  else if (a.M <= 2) PKV_GEMV(2, U_MAX);
  else if (a.M <= 4) PKV_GEMV(4, U_MAX);
  else if (a.M <= 8) PKV_GEMV(8, (U_MAX < 4 ? U_MAX : 4));
  else if (a.M <= 16) PKV_GEMV(16, (U_MAX < 2 ? U_MAX : 2));
  else PKV_GEMV(32, 1);
#undef PKV_GEMV
  return hipGetLastError();
}

template <int LPR, int EPI>
hipError_t gemv_dispatch_lpr(const LinArgs& a, hipStream_t s) {
  constexpr bool NORM = epi_norm(EPI);
  // steps a lane of this row width needs, rounded up to 2, 4 or 8
  const int steps = (a.K / 8 + LPR - 1) / LPR;
  if (steps <= 2) return gemv_dispatch_mt<LPR, EPI, NORM, 2>(a, s);
  if (steps <= 4) return gemv_dispatch_mt<LPR, EPI, NORM, 4>(a, s);
  return gemv_dispatch_mt<LPR, EPI, NORM, 8>(a, s);
}

// Lanes per row: enough that a lane's share of the row is at most 8 chunks,
// then more while the grid is under 1024 workgroups (7B shape at batch 1: the
// QKV and O projections at 128 lanes per row instead of 64, step 2.95 ->
// 2.88 ms; 512 and 2048 workgroups were slower).
int gemv_lanes_per_row(int n_out, int K) {
  const int chunks = K / 8;
  int lpr = 16;
  while (lpr < 256 && chunks > 8 * lpr) lpr *= 2;
  while (lpr < 256 && (long)n_out * lpr / 256 < 1024 && chunks >= 2 * lpr) lpr *= 2;
  return lpr;
}

template <int EPI>
hipError_t gemv_dispatch(const LinArgs& a, hipStream_t s) {
  switch (gemv_lanes_per_row(a.n_out, a.K)) {
    case 16: return gemv_dispatch_lpr<16, EPI>(a, s);
    case 32: return gemv_dispatch_lpr<32, EPI>(a, s);
    case 64: return gemv_dispatch_lpr<64, EPI>(a, s);
    case 128: return gemv_dispatch_lpr<128, EPI>(a, s);
    default: return gemv_dispatch_lpr<256, EPI>(a, s);
  }
}

}  // namespace

__global__ void zero_i32_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

size_t linear_ws_bytes(int M, int n_out, int K, int epi) {
  if (M < kMfmaMinBatch) return 0;
  return gemm_plan(M, n_out, K, epi).part_bytes;
}

hipError_t launch_linear(const LinArgs& a, int epi, void* part_ws, int* counters, hipStream_t s) {
  if (epi < EPI_F16 || epi > EPI_ROPE || (a.norm != 0) != epi_norm(epi) || (a.norm && !a.gain))
    return hipErrorInvalidValue;
  if (a.M >= kMfmaMinBatch) return launch_gemm(a, epi, gemm_plan(a.M, a.n_out, a.K, epi), part_ws, counters, s);
  switch (epi) {
    case EPI_F16: return gemv_dispatch<EPI_F16>(a, s);
    case EPI_RESID: return gemv_dispatch<EPI_RESID>(a, s);
    case EPI_SILU: return gemv_dispatch<EPI_SILU>(a, s);
    case EPI_ROPE: return gemv_dispatch<EPI_ROPE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero_i32(int* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(std::min(64, (n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace pkv
