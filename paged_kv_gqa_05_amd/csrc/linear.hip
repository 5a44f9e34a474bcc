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
// This file holds the GEMV for batch < 32: a group of LPC lanes (16, 32 or
// 64) streams one output row of W (one row pair for SILU / ROPE) with 16-byte
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

template <int LPC, int MT, int EPI>
__global__ void __launch_bounds__(256) gemv_kernel(LinArgs a) {
  constexpr bool PAIR = epi_pair(EPI);
  const int tid = threadIdx.x;
  const int lig = tid % LPC;
  const int col = blockIdx.x * (256 / LPC) + tid / LPC;
  if (col >= a.n_out) return;  // whole lane group leaves; no block-wide barrier below
  const h16* w0 = a.W + (size_t)(PAIR ? pair_row(EPI == EPI_ROPE, a.n_out, a.rope.d, col, 0) : col) * a.K;
  const h16* w1 = PAIR ? a.W + (size_t)pair_row(EPI == EPI_ROPE, a.n_out, a.rope.d, col, 1) * a.K : w0;
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

}  // namespace

__global__ void zero_i32_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

size_t linear_ws_bytes(int M, int n_out, int K, int epi) {
  if (M < kMfmaMinBatch) return 0;
  return gemm_plan(M, n_out, K, epi).part_bytes;
}

hipError_t launch_linear(const LinArgs& a, int epi, void* part_ws, int* counters, hipStream_t s) {
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
