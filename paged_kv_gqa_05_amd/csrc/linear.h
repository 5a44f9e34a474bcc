// Fused projection launchers shared by the decode layer and the LM head.
#pragma once

#include "pkv_internal.h"

namespace pkv {

enum { EPI_F16 = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_ROPE = 3 };

// Epilogues that take output rows in pairs: gate/up (row j and j + n_out) and
// the QKV projection with RoPE (rows i and i + D/2 of one head).
__host__ __device__ constexpr bool epi_pair(int epi) { return epi == EPI_SILU || epi == EPI_ROPE; }
// The epilogues that follow an RMSNorm (QKV, gate/up, LM head); RESID (O and
// down projections) never does.
__host__ __device__ constexpr bool epi_norm(int epi) { return epi != EPI_RESID; }

// What the QKV epilogue needs to rotate q and k at each row's position and to
// store the new token's k and v in the paged cache.  RoPE (rotate-half form)
// is not spelled out by the pages; it is the position encoding of the
// Llama/Qwen2 families the rvLLM post lists as supported.  The angles
// pos * theta^(-2i/D) come from a host-built table (double precision, stored
// as f32 cos/sin), so the device evaluates no trigonometry.
struct RopeArgs {
  const float2* cos_sin;  // [max_positions][D/2] (cos, sin)
  const int32_t* lens;    // [M] context lengths: pos = lens[m] - 1
  const int32_t* bt;      // [M][bt_stride] block tables
  int bt_stride;
  _Float16* q_out;        // [M][Hq][D] rotated queries
  _Float16* k_pool;       // this layer's K pool (tiles [D/8][16][8])
  _Float16* v_pool;       // this layer's V pool (tiles [D][16])
  int hq, hkv, d;
};

// Weight rows of output pair p.
__device__ __forceinline__ int pair_row(int epi_rope, int n_out, int head_dim, int p, int second) {
  if (epi_rope) {
    const int half = head_dim >> 1;
    const int head = p / half, i = p - head * half;
    return head * head_dim + i + (second ? half : 0);
  }
  return p + (second ? n_out : 0);
}

// QKV epilogue for pair p of batch row m: y0, y1 are rows i and i + D/2 of a
// head (norm applied, bias not yet added).
__device__ __forceinline__ void rope_store(const RopeArgs& ra, const _Float16* bias, int m, int p, float y0,
                                           float y1) {
  const int half = ra.d >> 1;
  const int head = p / half, i = p - head * half;
  if (bias) {
    y0 += (float)bias[head * ra.d + i];
    y1 += (float)bias[head * ra.d + half + i];
  }
  const int c = ra.lens[m];
  const int pos = c > 0 ? c - 1 : 0;
  if (head < ra.hq + ra.hkv) {
    const float2 cs = ra.cos_sin[(size_t)pos * half + i];
    const float o0 = y0 * cs.x - y1 * cs.y;
    const float o1 = y1 * cs.x + y0 * cs.y;
    if (head < ra.hq) {
      _Float16* q = ra.q_out + ((size_t)m * ra.hq + head) * ra.d;
      q[i] = (_Float16)o0;
      q[half + i] = (_Float16)o1;
    } else if (c > 0) {  // K tile [D/8][16][8]
      const int blk = ra.bt[(size_t)m * ra.bt_stride + pos / 16];
      _Float16* kp = ra.k_pool + ((size_t)blk * ra.hkv + (head - ra.hq)) * 16 * ra.d + (pos % 16) * 8;
      kp[(i >> 3) * 128 + (i & 7)] = (_Float16)o0;
      kp[((half + i) >> 3) * 128 + ((half + i) & 7)] = (_Float16)o1;
    }
  } else if (c > 0) {  // V tile [D][16]
    const int blk = ra.bt[(size_t)m * ra.bt_stride + pos / 16];
    _Float16* vp = ra.v_pool + ((size_t)blk * ra.hkv + (head - ra.hq - ra.hkv)) * ra.d * 16 + (pos % 16);
    vp[i * 16] = (_Float16)y0;
    vp[(half + i) * 16] = (_Float16)y1;
  }
}

// Batches at or above this size use the MFMA GEMM; smaller ones the GEMV.
constexpr int kMfmaMinBatch = 32;
// Arrival counters available to one split-K GEMM (one per output tile).
constexpr int kGemmMaxCounters = 4096;

struct LinArgs {
  const _Float16* A;     // activations [M][lda] f16
  const _Float16* W;     // weights [rows][K] f16 (rows = n_out, or 2 n_out for EPI_SILU)
  const _Float16* gain;  // RMSNorm gain [K] applied to A (with norm), or null
  const _Float16* bias;  // [n_out] (EPI_F16) or [(Hq + 2 Hkv) D] (EPI_ROPE), or null
  void* out;             // [M][ldo] f16 (unused by EPI_ROPE)
  int M, K, lda, ldo;
  int n_out;             // logical output columns
  int norm;              // scale row m by 1/sqrt(mean_k A[m][k]^2 + eps); needs gain
  float eps;
  RopeArgs rope;         // EPI_ROPE only (n_out = (Hq + 2 Hkv) D / 2 pairs)
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
  RopeArgs rope;
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
