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
#include "gemv_body.h"

namespace pkv {
namespace {

template <int LPR, int MT, int U, int EPI, bool NORM>
__global__ void __launch_bounds__(256) gemv_kernel(LinArgs a) {
  gemv_body<LPR, MT, U, EPI, NORM, false>(a, blockIdx.x);
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
  if constexpr (LPR == 256 && EPI == EPI_RESID) {
    // rows a little over 8 steps of 256 lanes (the 7B down projection: 9.25)
    // take one round of 10 steps at batch <= 2 rather than a round of 8 and
    // a nearly empty second one (each lane's chunks and their order are the
    // same, so are the bits)
    if (steps > 8 && steps <= 10 && a.M <= 2) {
      const int grid = a.n_out;
      if (a.M <= 1)
        hipLaunchKernelGGL((gemv_kernel<256, 1, 10, EPI, NORM>), dim3(grid), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((gemv_kernel<256, 2, 10, EPI, NORM>), dim3(grid), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  return gemv_dispatch_mt<LPR, EPI, NORM, 8>(a, s);
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

void gemv_config(int n_out, int K, int* lanes_per_row, int* steps_per_iter) {
  const int lpr = gemv_lanes_per_row(n_out, K);
  const int steps = (K / 8 + lpr - 1) / lpr;
  *lanes_per_row = lpr;
  *steps_per_iter = steps <= 2 ? 2 : (steps <= 4 ? 4 : 8);
}

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
