// Fused projection launcher shared by the decode layer and the LM head.
#pragma once

#include "pkv_internal.h"

namespace pkv {

enum { EPI_F32 = 0, EPI_F16 = 1, EPI_RESID = 2, EPI_SILU = 3 };

// Batches at or above this size use the MFMA GEMM; smaller ones the GEMV.
constexpr int kMfmaMinBatch = 32;

struct LinArgs {
  const _Float16* A;     // activations [M][lda] f16
  const _Float16* W;     // weights [rows][K] f16 (rows = n_out, or 2 n_out for EPI_SILU)
  const _Float16* gain;  // RMSNorm gain [K] applied to A, or null
  const _Float16* bias;  // [n_out] or null (EPI_F32 / EPI_F16)
  void* out;             // [M][ldo]: f32 (EPI_F32) or f16
  int M, K, lda, ldo;
  int n_out;             // logical output columns
  int norm;              // scale row m by 1/sqrt(mean_k A[m][k]^2 + eps)
  float eps;
};

hipError_t launch_linear(const LinArgs& a, int epi, hipStream_t s);

}  // namespace pkv
