// Small per-step kernels: embedding gather, greedy argmax and the per-token
// rows of a prefill.
#include <algorithm>

#include "ops.h"

namespace pkv {
namespace {

typedef _Float16 h16;

// Also zeroes zero_n ints at zero_p (the split-K arrival counters of the step).
__global__ void embed_kernel(const h16* __restrict__ table, int rows, const int32_t* __restrict__ tokens,
                             h16* __restrict__ h, int hidden, int* __restrict__ zero_p, int zero_n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < zero_n; i += gridDim.x * blockDim.x) zero_p[i] = 0;
  const int b = blockIdx.x;
  const int tok = tokens[b];
  h16* dst = h + (size_t)b * hidden;
  if (tok < 0 || tok >= rows) {  // outside the table (the argmax's -1 of an inactive row): a zero row
    for (int i = threadIdx.x * 8; i < hidden; i += blockDim.x * 8) *reinterpret_cast<uint4*>(dst + i) = uint4{0, 0, 0, 0};
    return;
  }
  const h16* src = table + (size_t)tok * hidden;
  for (int i = threadIdx.x * 8; i < hidden; i += blockDim.x * 8)
    *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
}

// The first residual add of the (x, residual) layer form: r = f16(r + x) in
// fp32 (the exact sum of two f16 values rounded once more to f16 is the
// correctly rounded f16 sum), then x = 0 (the down projection adds its
// output to it); also zeroes zero_n ints at zero_p (the step's counters).
__global__ void add_clear_kernel(h16* __restrict__ r, h16* __restrict__ x, size_t n, int* __restrict__ zero_p,
                                 int zero_n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = t; i < (size_t)zero_n; i += stride) zero_p[i] = 0;
  for (size_t i = t; i < n; i += stride) {
    r[i] = (h16)((float)r[i] + (float)x[i]);
    x[i] = (h16)0.f;
  }
}

// Lowest index of the largest value per row (-1 for a row whose context
// length is 0 when lengths are given); NaN logits never win.  One
// workgroup of 1024 threads per row; when every row is 16-byte aligned (vec:
// vocab % 8 == 0 and an aligned base) rows are read with 16-byte loads, four
// in flight per thread.
__device__ __forceinline__ void argmax_take(float v, int i, float& best, int& idx) {
  if (v > best || (v == best && i < idx)) {  // NaN compares false: never taken
    best = v;
    idx = i;
  }
}

__global__ void __launch_bounds__(1024) argmax_kernel(const h16* __restrict__ logits, int vocab,
                                                      int32_t* __restrict__ out, int vec,
                                                      const int32_t* __restrict__ lens) {
  const int b = blockIdx.x;
  if (lens && lens[b] == 0) {  // inactive row
    if (threadIdx.x == 0) out[b] = -1;
    return;
  }
  const h16* row = logits + (size_t)b * vocab;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  if (vec) {
    typedef h16 h16x8 __attribute__((ext_vector_type(8)));
    const h16x8* rv = reinterpret_cast<const h16x8*>(row);
    const int nv = vocab / 8;
    int i = threadIdx.x;
    for (; i + 3 * 1024 < nv; i += 4 * 1024) {
      h16x8 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = rv[i + u * 1024];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) argmax_take((float)v[u][e], (i + u * 1024) * 8 + e, best, idx);
    }
    for (; i < nv; i += 1024) {
      const h16x8 v = rv[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) argmax_take((float)v[e], i * 8 + e, best, idx);
    }
  } else {
    for (int i = threadIdx.x; i < vocab; i += 1024) argmax_take((float)row[i], i, best, idx);
  }
  __shared__ float sv[1024 / 64];
  __shared__ int si[1024 / 64];
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    argmax_take(ov, oi, best, idx);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = best;
    si[wave] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 1024 / 64; ++w) argmax_take(sv[w], si[w], best, idx);
    out[b] = idx == 0x7fffffff ? 0 : idx;
  }
}

// Per-token rows of a prefill: new token j of sequence s (tokens
// [seq_starts[s], seq_starts[s+1])) gets context length prior_lens[s] + j + 1
// (0, an inactive row, if that is outside [1, max_context]) and a copy of the
// first stride_tok entries of its sequence's block-table row; last_idx[s] is
// the row of the sequence's last new token.  Offsets are clamped to [0, T], so
// malformed offsets cannot reach outside the buffers.
__global__ void prefill_rows_kernel(const int32_t* __restrict__ seq_starts, const int32_t* __restrict__ prior_lens,
                                    const int32_t* __restrict__ bt, int bt_stride, int n_tokens, int stride_tok,
                                    int max_context, int32_t* __restrict__ lens_tok, int32_t* __restrict__ bt_tok,
                                    int32_t* __restrict__ last_idx) {
  const int s = blockIdx.x;
  const int t0 = min(max(seq_starts[s], 0), n_tokens);
  const int t1 = min(max(seq_starts[s + 1], t0), n_tokens);
  const int n = t1 - t0, prior = prior_lens[s];
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const long long pos1 = (long long)prior + j + 1;
    lens_tok[t0 + j] = (pos1 >= 1 && pos1 <= max_context) ? (int)pos1 : 0;
  }
  const int32_t* src = bt + (size_t)s * bt_stride;
  for (int i = threadIdx.x; i < n * stride_tok; i += blockDim.x) {
    const int j = i / stride_tok, c = i - j * stride_tok;
    bt_tok[(size_t)(t0 + j) * stride_tok + c] = src[c];
  }
  if (threadIdx.x == 0) last_idx[s] = n > 0 ? t1 - 1 : min(t0, n_tokens - 1);
}

}  // namespace

hipError_t launch_prefill_rows(const int32_t* seq_starts, const int32_t* prior_lens, const int32_t* bt,
                               int bt_stride, int n_seqs, int n_tokens, int stride_tok, int max_context,
                               int32_t* lens_tok, int32_t* bt_tok, int32_t* last_idx, hipStream_t s) {
  hipLaunchKernelGGL(prefill_rows_kernel, dim3(n_seqs), dim3(256), 0, s, seq_starts, prior_lens, bt, bt_stride,
                     n_tokens, stride_tok, max_context, lens_tok, bt_tok, last_idx);
  return hipGetLastError();
}

// A plain streaming read, the reference for what one launch of a given size
// can draw from HBM: workgroup w reads its own contiguous range of 16-byte
// units once, eight loads in flight per thread, and folds them with XOR; a
// thread whose fold equals kStreamMagic sets *sink (so the loads cannot be
// dropped, and a test can plant the value).
constexpr uint32_t kStreamMagic = 0x9e3779b9u;

__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ p, size_t n, size_t per_wg,
                                                          int32_t* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_wg, hi = std::min(n, lo + per_wg);
  uint4 acc = uint4{0, 0, 0, 0};
  for (size_t i = lo + threadIdx.x; i < hi; i += 8 * 256) {
    uint4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t j = i + (size_t)u * 256;
      q[u] = j < hi ? p[j] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x ^= q[u].x;
      acc.y ^= q[u].y;
      acc.z ^= q[u].z;
      acc.w ^= q[u].w;
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == kStreamMagic) *sink = 1;
}

hipError_t launch_embed(const void* table, int table_rows, const int32_t* tokens, void* h, int batch, int hidden,
                        int* zero_p, int zero_n, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(batch), dim3(256), 0, s, static_cast<const h16*>(table), table_rows, tokens,
                     static_cast<h16*>(h), hidden, zero_p, zero_n);
  return hipGetLastError();
}

hipError_t launch_add_clear(void* r, void* x, size_t n, int* zero_p, int zero_n, hipStream_t s) {
  const size_t need = (std::max(n, (size_t)zero_n) + 255) / 256;
  const int grid = (int)std::min<size_t>(std::max<size_t>(need, 1), 1024);
  hipLaunchKernelGGL(add_clear_kernel, dim3(grid), dim3(256), 0, s, static_cast<h16*>(r), static_cast<h16*>(x), n,
                     zero_p, zero_n);
  return hipGetLastError();
}

hipError_t launch_argmax(const void* logits, int batch, int vocab, int32_t* tokens, const int32_t* lens,
                         hipStream_t s) {
  const int vec = (vocab % 8 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  hipLaunchKernelGGL(argmax_kernel, dim3(batch), dim3(1024), 0, s, static_cast<const h16*>(logits), vocab,
                     tokens, vec, lens);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* data, size_t bytes, int32_t* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  // about 8 units a thread per workgroup, at most 2048 workgroups
  const size_t grid = std::min<size_t>(std::max<size_t>((n + 2047) / 2048, 1), 2048);
  const size_t per_wg = (n + grid - 1) / grid;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint4*>(data), n,
                     per_wg, sink);
  return hipGetLastError();
}

}  // namespace pkv
