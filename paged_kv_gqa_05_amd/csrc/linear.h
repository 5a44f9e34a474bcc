// Fused projection launchers shared by the decode layer and the LM head.
#pragma once

#include "pkv_internal.h"

namespace pkv {

enum { EPI_F32 = 0, EPI_F16 = 1, EPI_RESID = 2, EPI_SILU = 3 };

// Batches at or above this size use the MFMA GEMM; smaller ones the GEMV.
constexpr int kMfmaMinBatch = 32;
// Arrival counters available to one split-K GEMM (one per output tile).
constexpr int kGemmMaxCounters = 4096;

struct LinArgs {
  const _Float16* A;     // activations [M][lda] f16
  const _Float16* W;     // weights [rows][K] f16 (rows = n_out, or 2 n_out for EPI_SILU)
  const _Float16* gain;  // RMSNorm gain [K] applied to A (with norm), or null
  const _Float16* bias;  // [n_out] or null (EPI_F32 / EPI_F16)
  void* out;             // [M][ldo]: f32 (EPI_F32) or f16
  int M, K, lda, ldo;
  int n_out;             // logical output columns
  int norm;              // scale row m by 1/sqrt(mean_k A[m][k]^2 + eps); needs gain
  float eps;
};

enum { GEMM_32x64 = 0, GEMM_64x128 = 1, GEMM_128x128 = 2 };

struct GemmPlan {
  int cfg, mt, nt;
  int n_mt, n_nt, splits, kc_per_split;
  size_t part_bytes;  // split-K workspace (0 without a split)
};

struct GemmParams {
  const _Float16* A;
  const _Float16* W;
  const _Float16* gain;
  const _Float16* bias;
  void* out;
  float* part;     // split-K partial tiles
  float* part_ss;  // split-K partial sums of squares
  int* counters;   // split-K arrival counters (zero between launches)
  int M, K, lda, ldo, n_out;
  float eps;
  int n_mt, n_nt, splits, kc_per_split, per_xcd;
};

GemmPlan gemm_plan(int M, int n_out, int K, int epi);
hipError_t launch_gemm(const LinArgs& a, int epi, const GemmPlan& pl, void* part_ws, int* counters,
                       hipStream_t s);

// Scratch one projection needs (0 for the GEMV path).
size_t linear_ws_bytes(int M, int n_out, int K, int epi);

// GEMV below kMfmaMinBatch rows, MFMA GEMM above.  part_ws / counters:
// scratch of linear_ws_bytes and kGemmMaxCounters zeroed ints.
hipError_t launch_linear(const LinArgs& a, int epi, void* part_ws, int* counters, hipStream_t s);

// Zero n ints on the stream with a kernel (graph-capturable, no memset node).
hipError_t launch_zero_i32(int* p, int n, hipStream_t s);

}  // namespace pkv
