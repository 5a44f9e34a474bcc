#pragma once

#include "pkv_internal.h"

namespace pkv {

hipError_t launch_embed(const void* table, const int32_t* tokens, void* h, int batch, int hidden,
                        int* zero_p, int zero_n, hipStream_t s);
hipError_t launch_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* uniform, const int32_t* lens, int32_t* tokens,
                         hipStream_t s);
hipError_t launch_prefill_rows(const int32_t* seq_starts, const int32_t* prior_lens, const int32_t* bt,
                               int bt_stride, int n_seqs, int n_tokens, int stride_tok, int max_context,
                               int32_t* lens_tok, int32_t* bt_tok, int32_t* last_idx, hipStream_t s);
hipError_t launch_argmax(const void* logits, int batch, int vocab, int32_t* tokens, const int32_t* lens,
                         hipStream_t s);

}  // namespace pkv
