#pragma once

#include "pkv_internal.h"

namespace pkv {

// h[b] = table[tokens[b]] for b < batch (a zero row for an id outside
// [0, table_rows)); also zeroes zero_n ints at zero_p.
hipError_t launch_embed(const void* table, int table_rows, const int32_t* tokens, void* h, int batch, int hidden,
                        int* zero_p, int zero_n, hipStream_t s);
// With counts (int32 [batch][vocab]): penalties applied in place to
// penalized_logits (the same buffer as logits) first, and each active row's
// count of its sampled token incremented at the end.
hipError_t launch_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* uniform, const int32_t* lens, int32_t* tokens,
                         hipStream_t s, void* penalized_logits = nullptr, int32_t* counts = nullptr,
                         const float* repetition = nullptr, const float* frequency = nullptr,
                         const float* presence = nullptr);
hipError_t launch_prefill_rows(const int32_t* seq_starts, const int32_t* prior_lens, const int32_t* bt,
                               int bt_stride, int n_seqs, int n_tokens, int stride_tok, int max_context,
                               int32_t* lens_tok, int32_t* bt_tok, int32_t* last_idx, hipStream_t s);
// Causal attention of a prefill's new tokens over the paged cache (their k and
// v already appended): q and out are [n_tokens][hq][head_dim] f16; items
// (int32 pairs, max_items of them) and n_items are scratch for the work list.
struct PrefillAttnArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  void* out;
  const int32_t* seq_starts;
  const int32_t* prior_lens;
  const int32_t* bt;
  int bt_stride;
  int32_t* items;
  int32_t* n_items;
  int max_items;
  int n_seqs, n_tokens, hq, hkv, head_dim, max_context;
  int num_blocks;  // blocks in the pool (ids outside it are read as block 0)
  bool fp8;
  float scale, k_scale, v_scale;
};
int prefill_max_items(int n_tokens, int n_seqs, int group);
// The (sequence, 16-row chunk) work list, built once per prefill call from
// seq_starts (reads seq_starts, n_seqs, n_tokens, items, n_items, max_items).
hipError_t launch_prefill_items(const PrefillAttnArgs& a, int group, hipStream_t s);
// Attention of every layer, over the work list built above.
hipError_t launch_prefill_attention(const PrefillAttnArgs& a, hipStream_t s);

// One streaming read of `bytes` (a multiple of 16) at 16-byte aligned `data`;
// *sink is set only if the data hold the planted fold value.
hipError_t launch_stream_read(const void* data, size_t bytes, int32_t* sink, hipStream_t s);
hipError_t launch_argmax(const void* logits, int batch, int vocab, int32_t* tokens, const int32_t* lens,
                         hipStream_t s);
// r = f16(r + x), then x = 0, over n f16 elements; zeroes zero_n ints at zero_p.
hipError_t launch_add_clear(void* r, void* x, size_t n, int* zero_p, int zero_n, hipStream_t s);

}  // namespace pkv
