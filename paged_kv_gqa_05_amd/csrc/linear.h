// Fused projection launchers shared by the decode layer and the LM head.
#pragma once

#include "coherent.h"
#include "kvstore.h"
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
  void* k_pool;           // this layer's K pool (f16 or E4M3 tiles, include/pkv.h)
  void* v_pool;           // this layer's V pool
  int hq, hkv, d;
  int fp8;                // E4M3 cache: store codes of f16(x) / scale
  float k_scale, v_scale;
  int num_blocks;         // blocks in the pool: an id outside [0, num_blocks) is never written
  int max_pos;            // rows of cos_sin
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

// The QKV epilogue in three steps, so that a kernel can issue every load of
// its tile before the first store (a load cannot be moved above a store to a
// possibly aliasing pointer, and each such pair would cost a memory round
// trip): the row's context length, then its position's block id and the
// (cos, sin) of each pair, then stores only.
struct RopeRow {
  int c, pos, blk;  // blk -1: nothing stored (inactive row, or no valid slot)
};
__device__ __forceinline__ RopeRow rope_row_len(const RopeArgs& ra, int m) {
  RopeRow r;
  r.c = ra.lens[m];
  r.pos = r.c > 0 ? r.c - 1 : 0;
  r.blk = -1;
  return r;
}
// A length beyond the block table or a block id outside the pool (caller
// errors) stores nothing rather than writing outside the pool.
__device__ __forceinline__ void rope_row_blk(const RopeArgs& ra, int m, RopeRow& r) {
  const int e = r.pos / 16;
  const int blk = (r.c > 0 && e < ra.bt_stride) ? ra.bt[(size_t)m * ra.bt_stride + e] : -1;
  r.blk = (unsigned)blk < (unsigned)ra.num_blocks ? blk : -1;
}
__device__ __forceinline__ float2 rope_cs(const RopeArgs& ra, const RopeRow& r, int p) {
  const int half = ra.d >> 1;
  return ra.cos_sin[(size_t)min(r.pos, ra.max_pos - 1) * half + p % half];
}
// Pair p of batch row m: y0, y1 are rows i and i + D/2 of a head with the
// norm and the bias applied.  Rotates q and k heads at the row's position,
// writes q, and stores the new token's k and v in the paged cache.  COH: q is
// written with agent-scope stores (read by other XCDs in the same kernel).
template <bool COH = false>
__device__ __forceinline__ void rope_put(const RopeArgs& ra, const RopeRow& r, int m, int p, float y0, float y1,
                                         float2 cs) {
  const int half = ra.d >> 1;
  const int head = p / half, i = p - head * half;
  if (head < ra.hq + ra.hkv) {
    const float o0 = y0 * cs.x - y1 * cs.y;
    const float o1 = y1 * cs.x + y0 * cs.y;
    if (head < ra.hq) {
      _Float16* q = ra.q_out + ((size_t)m * ra.hq + head) * ra.d;
      if constexpr (COH) {
        st_agent_h(q + i, (_Float16)o0);
        st_agent_h(q + half + i, (_Float16)o1);
      } else {
        q[i] = (_Float16)o0;
        q[half + i] = (_Float16)o1;
      }
    } else if (r.blk >= 0) {
      const size_t tile = ((size_t)r.blk * ra.hkv + (head - ra.hq)) * 16 * ra.d;
      const int t = r.pos % 16;
      kv_store(ra.k_pool, tile + k_tile_off(ra.fp8, t, i), ra.fp8, ra.k_scale, o0);
      kv_store(ra.k_pool, tile + k_tile_off(ra.fp8, t, half + i), ra.fp8, ra.k_scale, o1);
    }
  } else if (r.blk >= 0) {
    const size_t tile = ((size_t)r.blk * ra.hkv + (head - ra.hq - ra.hkv)) * 16 * ra.d;
    const int t = r.pos % 16;
    kv_store(ra.v_pool, tile + v_tile_off(ra.fp8, t, i), ra.fp8, ra.v_scale, y0);
    kv_store(ra.v_pool, tile + v_tile_off(ra.fp8, t, half + i), ra.fp8, ra.v_scale, y1);
  }
}
// The pair's two bias values (0 without bias).
__device__ __forceinline__ float2 rope_bias(const RopeArgs& ra, const _Float16* bias, int p) {
  if (!bias) return make_float2(0.f, 0.f);
  const int half = ra.d >> 1;
  const int head = p / half, i = p - head * half;
  return make_float2((float)bias[head * ra.d + i], (float)bias[head * ra.d + half + i]);
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

enum { GEMM_32x64 = 0, GEMM_64x128 = 1, GEMM_128x128 = 2, GEMM_128x256 = 3, GEMM_128x128_S3 = 4, GEMM_128x160 = 5,
       GEMM_64x64 = 6, GEMM_256x256 = 7, GEMM_32x96 = 8, GEMM_32x160 = 9, GEMM_64x96 = 10, GEMM_64x160 = 11 };

// Tiles of N-tile columns [0, nt_full) are computed whole; those of columns
// [nt_full, n_nt) are cut into `splits` K ranges of kc_per_split stages.
struct GemmPlan {
  int cfg, mt, nt;
  int n_mt, n_nt, nt_full, splits, kc_per_split;
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
  int n_mt, n_nt, nt_full, splits, kc_per_split;
  int full_per_xcd, per_xcd, split_items;  // workgroups per XCD: whole tiles, then split parts
  int blk_m, nbm;   // > 0: whole tiles in blocks of blk_m x (32 / blk_m) tiles, nbm blocks along M
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

// The GEMV configuration (batch < 32) of an n_out x K projection: lanes per
// output row and chunk steps per lane iteration (the batch-1 bucket).
int gemv_lanes_per_row(int n_out, int K);
void gemv_config(int n_out, int K, int* lanes_per_row, int* steps_per_iter);

// ------------------------------------------------- persistent batch-1 layers

// One layer's weight pointers, kept in device memory for the persistent kernel.
struct PersistLayer {
  const _Float16 *w_in, *w_qkv, *b_qkv, *w_o, *w_post, *w_gu, *w_down;
};

// Every layer of a batch-1 decode step in one persistent kernel (persist.hip).
struct PersistArgs {
  LinArgs qkv, o, gu, down;    // arguments of layer 0 (weights are replaced per layer)
  AttnArgs attn;               // attention of layer 0 (pools and scales replaced per layer)
  AttnPlan plan;
  const PersistLayer* layers;  // device [n_layers]
  size_t pool_stride;          // bytes from one layer's K pool to the next layer's
  size_t v_off;                // bytes from a layer's K pool to its V pool
  const float* k_scales;       // (host) [n_layers], fp8 caches only
  const float* v_scales;
  int n_layers;
  unsigned* barrier;           // 2240 words zero before the launch (word 0 is set
                               // if a barrier timed out)
};
// Whether the shapes fit the kernel's body variants (and the grid can be resident).
bool persistent_config(const PersistArgs& a, int* cfg_hidden, int* cfg_gu);
hipError_t launch_persistent_layers(const PersistArgs& a, hipStream_t s);

// Zero n ints on the stream with a kernel (graph-capturable, no memset node).
hipError_t launch_zero_i32(int* p, int n, hipStream_t s);

}  // namespace pkv
