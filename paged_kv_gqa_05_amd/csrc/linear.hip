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
// Epilogues: F32 (QKV: + bias, fp32 out for the RoPE/append kernel), RESID
// (h = f16(h + y) in place: the residual add of the next norm), SILU (rows
// [gate | up]: act = f16(silu(g) * u)), F16 (logits).
//
// Two kernels:
//  * batch < 32: GEMV.  A group of LPC lanes (16, 32 or 64) streams one
//    output row of W (one gate/up pair for SILU) with 16-byte loads and v_dot2
//    against every batch row, then reduces across its lanes.
//  * batch >= 32: MFMA GEMM.  64 x 64 tiles (W rows), K step 64 staged through
//    LDS (double buffered), 4 waves each 32 x 32 with v_mfma_f32_16x16x32_f16.
//    Workgroup ids are remapped so that the M tiles sharing one W tile run on
//    the same XCD (the hardware deals workgroups round-robin over the 8 XCDs),
//    so each W tile is fetched from HBM into one L2 only.
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
  if constexpr (EPI == EPI_F32) {
    if (a.bias) y0 += (float)a.bias[col];
    static_cast<float*>(a.out)[(size_t)m * a.ldo + col] = y0;
  } else if constexpr (EPI == EPI_F16) {
    if (a.bias) y0 += (float)a.bias[col];
    static_cast<h16*>(a.out)[(size_t)m * a.ldo + col] = (h16)y0;
  } else if constexpr (EPI == EPI_RESID) {
    h16* p = static_cast<h16*>(a.out) + (size_t)m * a.ldo + col;
    *p = (h16)((float)*p + y0);
  } else {  // EPI_SILU
    static_cast<h16*>(a.out)[(size_t)m * a.ldo + col] = (h16)(silu(y0) * y1);
  }
}

// ------------------------------------------------------------------ GEMV

template <int LPC, int MT, int EPI>
__global__ void __launch_bounds__(256) gemv_kernel(LinArgs a) {
  constexpr bool PAIR = (EPI == EPI_SILU);
  const int tid = threadIdx.x;
  const int lig = tid % LPC;
  const int col = blockIdx.x * (256 / LPC) + tid / LPC;
  if (col >= a.n_out) return;  // whole lane group leaves; no block-wide barrier below
  const h16* w0 = a.W + (size_t)col * a.K;
  const h16* w1 = PAIR ? a.W + (size_t)(col + a.n_out) * a.K : w0;
  float acc0[MT], acc1[MT], ss[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc0[m] = acc1[m] = ss[m] = 0.f;
  const h16x8 one = h16x8{1, 1, 1, 1, 1, 1, 1, 1};
  for (int k = lig * 8; k < a.K; k += LPC * 8) {
    const h16x8 wv0 = *reinterpret_cast<const h16x8*>(w0 + k);
    h16x8 wv1;
    if (PAIR) wv1 = *reinterpret_cast<const h16x8*>(w1 + k);
    const h16x8 g = a.gain ? *reinterpret_cast<const h16x8*>(a.gain + k) : one;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < a.M) {
        const h16x8 x = *reinterpret_cast<const h16x8*>(a.A + (size_t)m * a.lda + k);
        if (a.norm) ss[m] = dot8(x, x, ss[m]);
        const h16x8 xg = a.gain ? x * g : x;
        acc0[m] = dot8(wv0, xg, acc0[m]);
        if (PAIR) acc1[m] = dot8(wv1, xg, acc1[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int o = LPC / 2; o > 0; o >>= 1) {
      acc0[m] += __shfl_xor(acc0[m], o, 64);
      if (PAIR) acc1[m] += __shfl_xor(acc1[m], o, 64);
      if (a.norm) ss[m] += __shfl_xor(ss[m], o, 64);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < a.M && (m % LPC) == lig) {
      const float r = a.norm ? rsqrtf(ss[m] / (float)a.K + a.eps) : 1.0f;
      epilogue<EPI>(a, m, col, acc0[m] * r, acc1[m] * r);
    }
  }
}

template <int LPC, int EPI>
hipError_t gemv_dispatch_mt(const LinArgs& a, hipStream_t s) {
  const int grid = (a.n_out + 256 / LPC - 1) / (256 / LPC);
#define PKV_GEMV(MT_) \
  hipLaunchKernelGGL((gemv_kernel<LPC, MT_, EPI>), dim3(grid), dim3(256), 0, s, a)
  if (a.M <= 1) PKV_GEMV(1);
  else if (a.M <= 2) PKV_GEMV(2);
  else if (a.M <= 4) PKV_GEMV(4);
  else if (a.M <= 8) PKV_GEMV(8);
  else if (a.M <= 16) PKV_GEMV(16);
  else PKV_GEMV(32);
#undef PKV_GEMV
  return hipGetLastError();
}

template <int EPI>
hipError_t gemv_dispatch(const LinArgs& a, hipStream_t s) {
  // fewest lanes per row that still gives >= 512 workgroups
  if ((long)a.n_out * 16 / 256 >= 512) return gemv_dispatch_mt<16, EPI>(a, s);
  if ((long)a.n_out * 32 / 256 >= 512) return gemv_dispatch_mt<32, EPI>(a, s);
  return gemv_dispatch_mt<64, EPI>(a, s);
}

// ------------------------------------------------------------------ GEMM

constexpr int BM = 64, BNW = 64, BK = 64, LDSK = BK + 8;

template <int EPI>
__global__ void __launch_bounds__(256) gemm_kernel(LinArgs a, int n_mt, int n_nt, int per_xcd) {
  constexpr bool PAIR = (EPI == EPI_SILU);
  __shared__ h16 sA[2][BM][LDSK];
  __shared__ h16 sW[2][BNW][LDSK];
  __shared__ float s_r[BM];

  // XCD-aware tile order: the 8 XCDs each take a contiguous range of tiles,
  // M tiles fastest, so the M tiles of one W tile share an L2.
  const int L = blockIdx.x;
  const int T = (L & 7) * per_xcd + (L >> 3);
  if (T >= n_mt * n_nt) return;
  const int mt = T % n_mt, nt = T / n_mt;
  const int m0 = mt * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // W row (global) held in tile row rr; -1 past the end
  auto wrow = [&](int rr) -> int {
    if (PAIR) {
      const int j = nt * (BNW / 2) + (rr & 31);
      return j < a.n_out ? j + (rr >= 32 ? a.n_out : 0) : -1;
    }
    const int n = nt * BNW + rr;
    return n < a.n_out ? n : -1;
  };

  // each thread stages rows lr and lr + 32 (A and W) at k-chunk lc
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const int ar0 = m0 + lr, ar1 = m0 + lr + 32;
  const int wr0 = wrow(lr), wr1 = wrow(lr + 32);
  const h16x8 zero = h16x8{0, 0, 0, 0, 0, 0, 0, 0};
  const h16x8 one = h16x8{1, 1, 1, 1, 1, 1, 1, 1};
  float ss0 = 0.f, ss1 = 0.f;

  h16x8 ra0, ra1, rw0, rw1;
  auto gload = [&](int k0) {
    const int k = k0 + lc;
    const bool kin = k < a.K;
    ra0 = (kin && ar0 < a.M) ? *reinterpret_cast<const h16x8*>(a.A + (size_t)ar0 * a.lda + k) : zero;
    ra1 = (kin && ar1 < a.M) ? *reinterpret_cast<const h16x8*>(a.A + (size_t)ar1 * a.lda + k) : zero;
    rw0 = (kin && wr0 >= 0) ? *reinterpret_cast<const h16x8*>(a.W + (size_t)wr0 * a.K + k) : zero;
    rw1 = (kin && wr1 >= 0) ? *reinterpret_cast<const h16x8*>(a.W + (size_t)wr1 * a.K + k) : zero;
    if (a.norm) {
      ss0 = dot8(ra0, ra0, ss0);
      ss1 = dot8(ra1, ra1, ss1);
    }
    if (a.gain) {
      const h16x8 g = kin ? *reinterpret_cast<const h16x8*>(a.gain + k) : one;
      ra0 = ra0 * g;
      ra1 = ra1 * g;
    }
  };
  auto lstore = [&](int buf) {
    *reinterpret_cast<h16x8*>(&sA[buf][lr][lc]) = ra0;
    *reinterpret_cast<h16x8*>(&sA[buf][lr + 32][lc]) = ra1;
    *reinterpret_cast<h16x8*>(&sW[buf][lr][lc]) = rw0;
    *reinterpret_cast<h16x8*>(&sW[buf][lr + 32][lc]) = rw1;
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile-row base of N fragment fn for this wave: pairs keep gate and up of
  // the same logical column in the same lane
  const int wb0 = PAIR ? wn * 16 : wn * 32;
  const int wb1 = PAIR ? 32 + wn * 16 : wn * 32 + 16;
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  const int nk = (a.K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      h16x8 af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const h16x8*>(&sA[buf][wm * 32 + i * 16 + fr][kk + fk]);
      wf[0] = *reinterpret_cast<const h16x8*>(&sW[buf][wb0 + fr][kk + fk]);
      wf[1] = *reinterpret_cast<const h16x8*>(&sW[buf][wb1 + fr][kk + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // per-row 1/rms: 8 consecutive threads share a row
  if (a.norm) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      ss0 += __shfl_xor(ss0, o, 64);
      ss1 += __shfl_xor(ss1, o, 64);
    }
    if ((tid & 7) == 0) {
      s_r[lr] = rsqrtf(ss0 / (float)a.K + a.eps);
      s_r[lr + 32] = rsqrtf(ss1 / (float)a.K + a.eps);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int ml = wm * 32 + i * 16 + (lane >> 4) * 4 + rr;
      const int m = m0 + ml;
      if (m >= a.M) continue;
      const float r = a.norm ? s_r[ml] : 1.0f;
      if (PAIR) {
        const int col = nt * (BNW / 2) + wn * 16 + fr;
        if (col < a.n_out) epilogue<EPI>(a, m, col, acc[i][0][rr] * r, acc[i][1][rr] * r);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * BNW + (j ? wb1 : wb0) + fr;
          if (col < a.n_out) epilogue<EPI>(a, m, col, acc[i][j][rr] * r, 0.f);
        }
      }
    }
  }
}

template <int EPI>
hipError_t gemm_dispatch(const LinArgs& a, hipStream_t s) {
  const int n_mt = (a.M + BM - 1) / BM;
  const int cols_per_tile = (EPI == EPI_SILU) ? BNW / 2 : BNW;
  const int n_nt = (a.n_out + cols_per_tile - 1) / cols_per_tile;
  const int tiles = n_mt * n_nt;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm_kernel<EPI>), dim3(per_xcd * 8), dim3(256), 0, s, a, n_mt, n_nt, per_xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinArgs& a, int epi, hipStream_t s) {
  const bool mfma = a.M >= kMfmaMinBatch;
  switch (epi) {
    case EPI_F32: return mfma ? gemm_dispatch<EPI_F32>(a, s) : gemv_dispatch<EPI_F32>(a, s);
    case EPI_F16: return mfma ? gemm_dispatch<EPI_F16>(a, s) : gemv_dispatch<EPI_F16>(a, s);
    case EPI_RESID: return mfma ? gemm_dispatch<EPI_RESID>(a, s) : gemv_dispatch<EPI_RESID>(a, s);
    case EPI_SILU: return mfma ? gemm_dispatch<EPI_SILU>(a, s) : gemv_dispatch<EPI_SILU>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
