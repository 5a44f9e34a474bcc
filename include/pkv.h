/*
 * pkv.h -- C ABI of the paged-KV GQA decode library for MI355X (gfx950).
 *
 * The library runs the batched f16 decode step of a Llama/Qwen2-style decoder:
 * per layer a fused RMSNorm + QKV projection with RoPE and the KV append into a
 * block-table paged cache, paged GQA decode attention (split over the context
 * plus a merge pass, f16 or FP8 E4M3 KV), the O projection with the residual
 * add, a fused RMSNorm + gate/up projection with SiLU*mul, and the down
 * projection with the residual add; then the final RMSNorm, the LM head and a
 * greedy argmax.  The whole step can be captured once in a hipGraph and
 * replayed on the caller's stream.
 *
 * Sources (rvLLM post on discuss.pytorch.kr, "rvLLM 소개"):
 *   section "CUDA 그래프 리플레이"         -- per-step block tables and context
 *       lengths uploaded before a replay on the caller's stream; the graph holds
 *       the forward only (sampling stays outside);
 *   section "퓨즈드 CUDA 커널"             -- the fused per-layer ops;
 *   section "PagedAttention과 FlashAttention-3" -- block-table KV cache, GQA,
 *       f16 KV by default, FP8 E4M3 KV as an option;
 * zingnex.cn article "rvLLM：用Rust重写vLLM…", section 直接GPU调用 -- f16 GEMMs
 *   for the batched projections.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless a comment says (host).
 *   - Device memory belongs to the caller: the library never frees it.  Objects
 *     made by *_create are freed by the matching *_destroy.
 *   - Work is enqueued on the given stream (a hipStream_t passed as void*) and
 *     the call does not synchronise it.  Host-side argument checks happen
 *     before anything is enqueued; on an error nothing is enqueued.
 *   - Every call returns pkv_status; no C++ exception and no abort crosses the
 *     ABI.  pkv_last_error() returns a message for the calling thread's last
 *     failed call.
 *   - f16 is IEEE binary16; fp8 is OCP E4M3FN (1 sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN, max 448).
 *   - Device-side metadata (context lengths, block ids) is trusted: a context
 *     length above max_context or a block id outside [0, num_blocks) is a
 *     contract violation.  pkv_validate_metadata() checks host copies.
 *
 * Paged KV layout (block size BS = 16, Hkv KV heads, head_dim D in {64, 128}):
 *   For layer l the cache memory holds the K pool, then the V pool, each
 *   [num_blocks][Hkv] tiles of 16 tokens:
 *     K tile, f16: [D/8][BS][8]   element (t, d) at ((d/8)*BS + t)*8 + d%8
 *     K tile, fp8: [D/16][BS][16] element (t, d) at ((d/16)*BS + t)*16 + d%16
 *     V tile, f16: [D][BS]        element (t, d) at d*BS + t
 *     V tile, fp8: [D/64][4][16][4][4]  element (t, d) at
 *                  (((d/64)*4 + t/4)*16 + d%16)*16 + ((d/16)%4)*4 + t%4
 *   (K: 16-byte chunks of one token's dims, so a wave reads a K tile with
 *   contiguous 1 KB loads; f16 V dim-major; fp8 V in 16-byte chunks holding
 *   4 tokens x dims d, d+16, d+32, d+48, again read in contiguous 1 KB
 *   loads).  Element size 2 bytes (f16) or 1 byte (fp8 codes).  Token t of sequence b is in block
 *   block_tables[b * bt_stride + t / BS], slot t % BS.
 *   context_lens[b] counts the cached tokens INCLUDING the token being decoded:
 *   the new token's K/V go to position pos = context_lens[b] - 1 and attention
 *   covers positions [0, context_lens[b]).  context_lens[b] == 0 marks an
 *   inactive row (no append; attention output 0).  Block-table entries at
 *   index >= ceil(context_lens[b] / BS) are never read.
 *   Caller errors in this device metadata (pkv_validate_metadata reports
 *   them on the host) never make a kernel access memory outside the pool,
 *   the tables or the workspace: a block id outside [0, num_blocks) among
 *   the entries a call uses is read as block 0 and an append to it is
 *   dropped; a context length above the call's max_context is taken as
 *   max_context by the attention, and its append is dropped when its slot
 *   lies past the row's table; a token id outside [0, V) embeds as a zero
 *   row.  Such rows' results are unspecified; the call's other rows are
 *   unaffected.
 *
 * Query heads: head h reads KV head h / (Hq / Hkv) (contiguous groups);
 * Hq / Hkv <= 16.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_E_ARG = 1,          /* invalid argument (null pointer, bad size, bad shape) */
  PKV_E_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, block size, dtype) */
  PKV_E_NOMEM = 3,        /* host or device allocation failed */
  PKV_E_CAPACITY = 4,     /* block allocator exhausted */
  PKV_E_HIP = 5,          /* a HIP runtime call failed; message has hipGetErrorString */
  PKV_E_STATE = 6         /* object used in a state that does not allow the call */
} pkv_status;

typedef enum { PKV_KV_F16 = 0, PKV_KV_FP8_E4M3 = 1 } pkv_kv_dtype;

typedef void* pkv_stream_t; /* a hipStream_t; NULL is the null stream */

typedef struct pkv_cache pkv_cache;
typedef struct pkv_model pkv_model;
typedef struct pkv_graph pkv_graph;
typedef struct pkv_alloc pkv_alloc;

/* Message of the calling thread's last failed call ("" if none). */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------ KV cache */

typedef struct {
  int32_t num_layers;   /* >= 1 */
  int32_t num_blocks;   /* physical blocks per layer, >= 1 */
  int32_t block_size;   /* must be 16 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t dtype;        /* pkv_kv_dtype */
} pkv_cache_desc;

/* Bytes of device memory a cache with this description needs (host only).
 * The cache is the paged KV store of the rvLLM post (section
 * "PagedAttention과 FlashAttention-3": keys and values of past tokens kept in
 * a block-table cache) and of the aitrends.kr glossary (용어 해설, the
 * PagedAttention entry: the KV cache split into fixed-size pages); here a page
 * is a block of 16 tokens per KV head, laid out as above. */
pkv_status pkv_cache_bytes(const pkv_cache_desc* desc, size_t* bytes);

/* Wrap caller-owned device memory (>= pkv_cache_bytes, 256-byte aligned) as a
 * paged KV cache (the pages above; rvLLM post, section
 * "PagedAttention과 FlashAttention-3", FP8 E4M3 as the optional cache type).  For fp8 caches k_scales / v_scales (host, [num_layers]) are
 * the per-layer, per-tensor f32 scales (stored value = code value * scale);
 * they must be NULL for f16 caches.  The memory is not initialised. */
pkv_status pkv_kv_cache_create(const pkv_cache_desc* desc, void* dev_mem, size_t bytes,
                               const float* k_scales, const float* v_scales, pkv_cache** out);
void pkv_kv_cache_destroy(pkv_cache* cache);

/* Device addresses of layer `layer`'s K and V pools (tile layouts above).
 * PKV_E_ARG for a NULL argument or a layer outside [0, num_layers); the
 * addresses point into the caller's memory (nothing is allocated). */
pkv_status pkv_kv_cache_layer(const pkv_cache* cache, int layer, void** k_pool, void** v_pool);

/* Append one token per row: k and v are f16 [batch][Hkv][D]; row b is stored
 * at pos = context_lens[b] - 1 of layer `layer` (skipped when the length is 0).
 * f16 caches store the input bytes unchanged.  fp8 caches store the E4M3 code
 * of x / s for each f16 input x, with s the layer's k or v scale: the quotient
 * is formed in float32 (IEEE division), then rounded to the nearest E4M3
 * value with ties to the even code; magnitudes at or above 448 saturate to
 * +-448 and NaN maps to a NaN code (a reading: the rvLLM post names an E4M3
 * cache without a rounding rule).  block_tables: [batch][bt_stride] int32. */
pkv_status pkv_kv_append(pkv_cache* cache, int layer, const void* k, const void* v,
                         const int32_t* block_tables, int bt_stride,
                         const int32_t* context_lens, int batch, pkv_stream_t stream);

/* ----------------------------------------------------------------- attention */

/* Scratch bytes paged_attn_decode needs for this shape (host only).  The
 * workspace must be zero-filled once before its first use (e.g. hipMemset);
 * every call leaves it in a state valid for the next call, of any shape that
 * fits it.  Layout of a workspace of W bytes: the per-(row, KV head) arrival
 * counters sit in a leading region whose size depends on W only (W / 64 in
 * whole 256-byte units, at least 256 bytes), the partial results after it; a
 * call fits W when its batch x Hkv counters fit that region and its partials
 * fit behind it, which every W >= the returned size guarantees.
 * PKV_E_ARG for NULL arguments, sizes below 1 or Hq not a multiple of Hkv;
 * PKV_E_UNSUPPORTED for more than 16 query heads per KV head, max_context
 * above 262144, or batch x Hkv x ceil(max_context / 128) above 2^30 (the
 * attention's grid bound; the same limit holds for every call that plans
 * the decode attention). */
pkv_status pkv_attn_workspace_bytes(const pkv_cache* cache, int batch, int num_q_heads,
                                    int max_context, size_t* bytes);

/* Paged GQA decode attention for one layer (rvLLM post, section
 * "PagedAttention과 FlashAttention-3"):
 *   for query head h of row b, with g = h / (Hq / Hkv) and c = context_lens[b],
 *     s_t = scale * <q[b][h], K_t>    (t < c)
 *     out[b][h] = sum_t softmax(s)_t * V_t
 *   with K_t, V_t read through the block table (fp8 codes are multiplied by the
 *   layer's scales).  Accumulation is fp32; out is f16 [batch][Hq][D]; q is f16
 *   [batch][Hq][D].  lse (nullable, f32 [batch][Hq]) receives max s +
 *   ln(sum exp(s - max s)) (-inf for inactive rows).  The context is split into
 *   partitions processed in parallel; the last partition of a row to finish
 *   merges them all in partition order (so results are deterministic).
 *   workspace (>= pkv_attn_workspace_bytes, 256-byte aligned, zero-filled
 *   before its first use) holds per-(row, KV head) arrival counters, which
 *   every call returns to zero, and the partial results.  Two calls in flight
 *   at once must not share a workspace.  bt_stride >= ceil(max_context / 16);
 *   every context_lens[b] <= max_context <= 262144 (PKV_E_UNSUPPORTED above). */
pkv_status pkv_paged_attn_decode(const pkv_cache* cache, int layer, const void* q, void* out,
                                 float* lse, const int32_t* block_tables, int bt_stride,
                                 const int32_t* context_lens, int batch, int num_q_heads,
                                 int max_context, float scale, void* workspace,
                                 size_t workspace_bytes, pkv_stream_t stream);

/* Allocation-free variant of pkv_paged_attn_decode, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * pkv_paged_attn_decode without the workspace: the arrival counters and the
 * partial results live in a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that each GPU the library runs on holds until the process ends.
 * The call allocates nothing.  PKV_E_ARG when the shape needs more scratch
 * than that (batch x Hkv above 131072 counters, or partials above ~31.5 MiB;
 * the partials take batch x Hq x P x (D + 2) x 4 bytes for P partitions of
 * 512-1024 tokens when a row spans several: e.g. batch 32, Hq 28, contexts up
 * to 32768 need 29.8 MiB).  Every call on one GPU shares that GPU's array and
 * leaves its counters zero; two calls in flight at once on one GPU (two
 * streams, or two host threads) race and give wrong results.  The first call
 * on a device clears the counters with a kernel on the given stream (a call
 * under capture records that kernel; the next uncaptured call clears again). */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status pkv_paged_attn_decode_noalloc(const pkv_cache* cache, int layer, const void* q, void* out,
                                         float* lse, const int32_t* block_tables, int bt_stride,
                                         const int32_t* context_lens, int batch, int num_q_heads,
                                         int max_context, float scale, pkv_stream_t stream);

/* Testing hook for the decode attention's merge (host only, process-wide,
 * takes effect for kernels enqueued or captured later).  Under the 8-wave
 * plans the first partition of a multi-partition row waits up to `ticks` of
 * the 100 MHz device wall clock for the row's other partitions and then
 * merges them with its own partial kept on chip; past the limit it publishes
 * its partial and the last partition to arrive merges.  The default is 10000
 * (100 us); 0 makes it publish at once (the fallback path, for tests).  Both
 * paths give the same bits.  Always PKV_OK. */
pkv_status pkv_debug_attn_merge_wait(unsigned long long ticks);

/* Testing hook for the decode attention's work-list form (host only,
 * process-wide, default 1).  A call with long rows (8 or more 512-token
 * partitions at max_context) whose partitions would span several rounds of
 * the device runs in work-list form: a grid of resident workgroups takes
 * only the partitions inside each row's context, longest rows first, so no
 * workgroup is spent on partitions past a shorter row's context and the rows
 * with the most partials to merge merge early.  With 0 such calls run the
 * direct grid of the same partitions.  Both forms give the same bits.
 * Always PKV_OK. */
pkv_status pkv_debug_attn_worklist(int enable);

/* --------------------------------------------------------------------- model */

typedef struct {
  int32_t hidden;        /* H */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t ffn;           /* F */
  int32_t vocab;         /* V */
  int32_t num_layers;    /* L */
  int32_t max_positions; /* RoPE table length: positions [0, max_positions) */
  float rms_eps;
  float rope_theta;
} pkv_model_desc;

/* Device pointers to one layer's f16 weights, matrices row-major [out][in]:
 *   w_in [H]                    RMSNorm gain before attention
 *   w_qkv [(Hq + 2 Hkv) D][H]   rows: q heads, then k heads, then v heads
 *   b_qkv [(Hq + 2 Hkv) D]      QKV bias, nullable
 *   w_o [H][Hq D]
 *   w_post [H]                  RMSNorm gain before the MLP
 *   w_gate_up [2F][H]           rows: gate (F rows), then up (F rows)
 *   w_down [H][F] */
typedef struct {
  const void* w_in;
  const void* w_qkv;
  const void* b_qkv;
  const void* w_o;
  const void* w_post;
  const void* w_gate_up;
  const void* w_down;
} pkv_layer_weights;

/* Describe a model whose weights live in caller-owned device memory (borrowed,
 * not copied; they must outlive the model).  embed [V][H], w_final_norm [H],
 * w_lm_head [V][H] (untied).  layers: (host) array of num_layers entries.
 * The model owns only a device RoPE table (cos, sin of pos * theta^(-2i/D),
 * computed in double precision on the host).  Synchronous. */
pkv_status pkv_model_create(const pkv_model_desc* desc, const void* embed,
                            const pkv_layer_weights* layers, const void* w_final_norm,
                            const void* w_lm_head, pkv_model** out);
void pkv_model_destroy(pkv_model* model);

/* Model options (host only; take effect for steps enqueued or captured later):
 *   PKV_OPT_PERSISTENT_BATCH1 (default 0): with 1, a decode step of batch 1
 *   runs all layers in one persistent kernel (a grid of resident workgroups
 *   walks the five fused ops of every layer with a grid-wide barrier between
 *   them; the rvLLM post's optimisation history: fewer launches, cross-layer
 *   fusion) when the model's shapes fit it (head_dim 128 and the batch-1
 *   projection plans of the 1.5B / 7B-class shapes); otherwise, or with 0,
 *   one kernel per fused op.  Both give the same bits.  Off by default because
 *   on an MI355X it is the slower of the two (1.5B shape: 1.90 against
 *   1.01 ms per step; 7B: 4.40 against 2.82 ms): its phases read the
 *   activations with L2-bypassing loads and run at two workgroups per CU.
 * PKV_E_ARG for an unknown option or value. */
enum { PKV_OPT_PERSISTENT_BATCH1 = 0 };
pkv_status pkv_model_set_option(pkv_model* model, int option, int value);

/* Scratch bytes decode_layer / decode_step / graph_capture need (host only):
 * the per-step buffers of the fused layer (rvLLM post, section "퓨즈드 CUDA
 * 커널": q, the attention output and the SiLU*mul activation), the split-K
 * partial tiles of the projections and the attention partials.  Contents
 * need no initialisation (the step zeroes its arrival counters in its first
 * kernel, the memset removal of the post's optimisation history).
 * PKV_E_ARG for NULL arguments or sizes below 1; PKV_E_UNSUPPORTED for
 * max_context above 262144 or batch x Hkv x ceil(max_context / 128) above
 * 2^30. */
pkv_status pkv_step_workspace_bytes(const pkv_model* model, const pkv_cache* cache, int batch,
                                    int max_context, size_t* bytes);

/* One decoder layer for `batch` single-token rows (the pre-norm Llama/Qwen2
 * layer; rvLLM post, section "퓨즈드 CUDA 커널"):
 *   a = RMSNorm(h) * w_in; q,k,v = split(W_qkv a + b_qkv); q,k = RoPE(., pos)
 *   append k, v at pos = context_lens[b] - 1; o = paged attention(q)
 *   h1 = h + W_o o;  m = RMSNorm(h1) * w_post;  g,u = split(W_gate_up m)
 *   h  = h1 + W_down (silu(g) * u)
 * hidden: f16 [batch][H], updated in place.  The cache (f16, or fp8 with the
 * appended k and v quantised as pkv_kv_append does, from their f16 values)
 * must have the model's Hkv and head_dim and at least layer+1 layers. */
pkv_status pkv_decode_layer(const pkv_model* model, pkv_cache* cache, int layer, void* hidden,
                            const int32_t* block_tables, int bt_stride,
                            const int32_t* context_lens, int batch, int max_context,
                            void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* The same layer in the (x, residual) form of the fused "Add + RMSNorm"
 * kernels (rvLLM post, section "퓨즈드 CUDA 커널": the residual add of a
 * sub-block's output happens inside the next fused op):
 *   h = f16(residual + x)   (correctly rounded)
 *   the layer above on h up to h1 = h + W_o o
 *   residual = h1;  x = f16(W_down (silu(g) * u))   (not yet added)
 * x: f16 [batch][H], in: the previous layer's x (the embedding rows for
 * layer 0), out: this layer's MLP output.  residual: f16 [batch][H], in/out
 * (zero for layer 0).  Distinct buffers (PKV_E_ARG otherwise).  The final
 * hidden state after the last layer is f16(residual + x).  Workspace, cache
 * and metadata as for pkv_decode_layer. */
pkv_status pkv_decode_layer_xr(const pkv_model* model, pkv_cache* cache, int layer, void* x, void* residual,
                               const int32_t* block_tables, int bt_stride, const int32_t* context_lens,
                               int batch, int max_context, void* ws, size_t ws_bytes, pkv_stream_t stream);

/* One of the five fused ops of a decoder layer (rvLLM post, section
 * "퓨즈드 CUDA 커널"), run alone; in the order below they are exactly
 * pkv_decode_layer (bit for bit), passing q, the attention output and the
 * SiLU*mul activation through the workspace:
 *   PKV_OP_QKV      RMSNorm(hidden) * w_in, QKV projection + bias, RoPE of q
 *                   and k, q into the workspace, the new k and v into the cache
 *   PKV_OP_ATTN     paged GQA attention of that q (split + merge)
 *   PKV_OP_O        hidden += W_o o
 *   PKV_OP_GATE_UP  RMSNorm(hidden) * w_post, gate/up projection, SiLU(g) * u
 *                   into the workspace
 *   PKV_OP_DOWN     hidden += W_down act
 * Arguments as pkv_decode_layer, with the same batch, max_context and
 * workspace for the ops of one layer step.  The workspace must be zero-filled
 * before its first use by this call (its arrival counters must start at
 * zero; every call, and every decode step or prefill, leaves them zero).
 * PKV_E_ARG for an op outside the list.  Meant for profiling and testing a
 * single fused kernel; the decode step runs all five in one graph. */
enum { PKV_OP_QKV = 0, PKV_OP_ATTN = 1, PKV_OP_O = 2, PKV_OP_GATE_UP = 3, PKV_OP_DOWN = 4 };
pkv_status pkv_layer_op(const pkv_model* model, pkv_cache* cache, int layer, int op, void* hidden,
                        const int32_t* block_tables, int bt_stride, const int32_t* context_lens, int batch,
                        int max_context, void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* One decode step: h = embed[token_ids[b]], every layer, then
 * logits = W_lm RMSNorm(h) * w_final_norm.  token_ids int32 [batch]; an id
 * outside [0, V) (such as the -1 pkv_argmax gives an inactive row) embeds as
 * a zero row and is never read from the table (the same in pkv_prefill);
 * logits f16 [batch][V]; hidden_out (nullable) f16 [batch][H] gets the final
 * pre-norm hidden state.  Appends each row's token to the cache at
 * pos = context_lens[b] - 1 in every layer (f16 or fp8 caches, as
 * pkv_decode_layer). */
pkv_status pkv_decode_step(const pkv_model* model, pkv_cache* cache, const int32_t* token_ids,
                           const int32_t* block_tables, int bt_stride,
                           const int32_t* context_lens, int batch, int max_context,
                           void* logits, void* hidden_out, void* workspace,
                           size_t workspace_bytes, pkv_stream_t stream);

/* Batched, chunked prefill (the step before decode; rvLLM post, section
 * "PagedAttention과 FlashAttention-3": causal multi-token attention over the
 * paged cache).  Sequence s brings the new tokens
 * token_ids[seq_starts[s] .. seq_starts[s+1]) at positions prior_lens[s],
 * prior_lens[s] + 1, ... (prior_lens[s] tokens already cached, 0 for a whole
 * prompt).  In every layer the k and v of all new tokens are appended, then
 * new token j of sequence s attends over positions [0, prior_lens[s] + j] of
 * its sequence: the layer of pkv_decode_layer with each new token as a row of
 * its own.  Device arrays: token_ids int32 [n_tokens]; seq_starts int32
 * [n_seqs + 1], ascending from 0 to n_tokens, every sequence with at least
 * one new token; prior_lens int32 [n_seqs]; block_tables int32
 * [n_seqs][bt_stride] covering each sequence's first prior + new tokens;
 * logits f16 [n_seqs][V] gets the logits of each sequence's last new token.
 * max_context bounds prior_lens[s] + (new tokens of s); a token beyond it is
 * not appended and attends to nothing (its row is inactive).  f16 or fp8
 * caches as pkv_decode_layer.  workspace: pkv_prefill_workspace_bytes, 256-byte
 * aligned, contents irrelevant (the arrival counters are zeroed on entry). */
pkv_status pkv_prefill_workspace_bytes(const pkv_model* model, const pkv_cache* cache, int n_tokens, int n_seqs,
                                       int max_context, size_t* bytes);
pkv_status pkv_prefill(const pkv_model* model, pkv_cache* cache, const int32_t* token_ids,
                       const int32_t* seq_starts, const int32_t* prior_lens, int n_seqs, int n_tokens,
                       const int32_t* block_tables, int bt_stride, int max_context, void* logits,
                       void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* Greedy token per row: the lowest index of the largest f16 logit
 * (zingnex.cn article, section 支持的参数: temperature 0 decodes greedily);
 * NaN logits never win.  logits f16 [batch][vocab]; tokens int32 [batch].
 * context_lens (nullable, int32 [batch]): a row whose length is 0 is inactive
 * and gets token -1. */
pkv_status pkv_argmax(const void* logits, int batch, int vocab, int32_t* tokens, const int32_t* context_lens,
                      pkv_stream_t stream);

/* Measurement reference (not a step of the path): one plain streaming read
 * of `bytes` of device memory at `data` (16-byte aligned, bytes a positive
 * multiple of 16), 16-byte loads, each workgroup over its own contiguous
 * range.  Its time is what one launch of that many cold bytes can draw from
 * HBM on this device, against which the attention's achieved GB/s is also
 * reported (the rvLLM post, section "PagedAttention과 FlashAttention-3",
 * states attention as bound by the KV bytes it reads).  sink: a device int32
 * that is written (with 1) only if the XOR of every 32-bit word of some
 * thread's share of the data equals 0x9e3779b9 (tests plant such a word).
 * PKV_E_ARG for NULL pointers, a misaligned `data` or a bad size; nothing is
 * enqueued then. */
pkv_status pkv_stream_read(const void* data, size_t bytes, int32_t* sink, pkv_stream_t stream);

/* Sampled token per row, after the forward pass (zingnex.cn article, section
 * 支持的参数: temperature (0 = greedy), top_p, top_k (-1 = disabled)).  All
 * per-row arrays are device memory, [batch]: temperature f32, top_k int32,
 * top_p f32, uniform f32 in [0, 1) (the caller's random numbers; values
 * outside, and NaN, are clamped into [0, 1 - 2^-24]).  For row b with
 * T = temperature[b] and m its largest finite logit:
 *   T <= 0 (or NaN): the greedy token, as pkv_argmax;
 *   every finite logit x weighs W(x) = floor(2^40 E((x - m) * (1/T))), where
 *   1/T and the product are float32 and E is this float32 exponential, each
 *   operation rounded on its own: n = floor(y * log2(e) + 0.5),
 *   r = (y - n * 0.693359375) - n * (-2.12194440e-4), e^r by the degree-7
 *   Taylor polynomial 1 + r(1 + r(1/2 + r(1/6 + ... + r/5040))) in Horner
 *   form, times 2^n; E = 0 below -30 (W(m) = 2^40);
 *   top_k > 0 keeps every token whose logit is at or above the k-th largest
 *   (ties at the boundary kept);
 *   top_p < 1 keeps the tokens whose logit is at or above the largest value t
 *   for which the kept tokens at or above t sum to at least
 *   ceil(max(top_p, 0) * sum W) (in double; ties kept; top_p <= 0 keeps the
 *   largest logit and its ties);
 *   the result is the first kept token, in index order, whose running sum of
 *   W exceeds floor(u24 * Z / 2^24), Z the kept sum, u24 = floor(u * 2^24).
 * Every sum is an exact 64-bit integer, so the token is a function of the
 * inputs alone.  Non-finite logits are never kept; a row with none finite
 * gets 0.  context_lens (nullable): rows of length 0 get -1.  vocab <= 2^24. */
pkv_status pkv_sample(const void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* uniform, int32_t* tokens, const int32_t* context_lens,
                      pkv_stream_t stream);

/* pkv_sample after repetition, frequency and presence penalties (zingnex.cn
 * article, section CPU操作优化: the three penalties applied together).
 * counts: int32 [batch][vocab] (device, caller-owned, in/out), how many times
 * each token was already sampled for the row (the caller zeroes a row when a
 * sequence starts).  Per active row, for every token with c = counts > 0,
 * in float32 with each operation rounded on its own:
 *   x = x > 0 ? x / repetition : x * repetition;  x = (x - frequency * c) - presence
 * and the result is written back into logits as f16 (logits are in/out; rows
 * with repetition 1, frequency 0 and presence 0, and inactive rows, are left
 * untouched).  Then the row is sampled as pkv_sample does, and counts of the
 * sampled token is incremented (active rows only).  repetition, frequency,
 * presence: f32 [batch]; repetition must be > 0 and finite. */
pkv_status pkv_sample_penalized(void* logits, int batch, int vocab, const float* temperature, const int32_t* top_k,
                                const float* top_p, const float* repetition, const float* frequency,
                                const float* presence, const float* uniform, int32_t* counts, int32_t* tokens,
                                const int32_t* context_lens, pkv_stream_t stream);

/* ------------------------------------------------------------- graph replay */

/* Capture one pkv_decode_step (same arguments) into a hipGraph on
 * capture_stream (not the null stream).  Every pointer is baked into the
 * graph: before each replay the caller rewrites the CONTENTS of token_ids,
 * block_tables and context_lens (ordered on the replay stream, rvLLM post
 * section "CUDA 그래프 리플레이").  Nothing is allocated inside the captured
 * region.  The model, the cache and every buffer passed here must outlive the
 * graph: a replay uses them as captured (options such as
 * PKV_OPT_PERSISTENT_BATCH1 are read at capture time). */
pkv_status pkv_graph_capture(const pkv_model* model, pkv_cache* cache, const int32_t* token_ids,
                             const int32_t* block_tables, int bt_stride,
                             const int32_t* context_lens, int batch, int max_context,
                             void* logits, void* hidden_out, void* workspace,
                             size_t workspace_bytes, pkv_stream_t capture_stream,
                             pkv_graph** out);
/* Launch the captured step on the caller's stream. */
pkv_status pkv_graph_replay(pkv_graph* graph, pkv_stream_t stream);
void pkv_graph_destroy(pkv_graph* graph);

/* Batch-size buckets (rvLLM post, section "CUDA 그래프 리플레이": graphs are
 * captured for a set of batch sizes and a step runs the smallest one that
 * holds its rows).  Captures one pkv_decode_step per bucket (host array,
 * strictly ascending, 1 to 64 entries) over the same buffers, each sized for
 * the largest bucket; workspace_bytes must cover pkv_step_workspace_bytes of
 * every bucket.  token_ids and context_lens are written by the library on
 * replay, so they are not const. */
typedef struct pkv_graph_set pkv_graph_set;
pkv_status pkv_graph_set_capture(const pkv_model* model, pkv_cache* cache, const int32_t* buckets,
                                 int n_buckets, int32_t* token_ids, const int32_t* block_tables, int bt_stride,
                                 int32_t* context_lens, int max_context, void* logits, void* hidden_out,
                                 void* workspace, size_t workspace_bytes, pkv_stream_t capture_stream,
                                 pkv_graph_set** out);
/* Runs the step for rows [0, batch): replays the smallest bucket >= batch on
 * `stream`, first setting context_lens and token_ids of the padding rows
 * [batch, bucket) to 0 on that stream (inactive rows: no append, attention
 * output 0, pkv_argmax with context_lens gives -1).  *bucket_out (host,
 * nullable) receives the bucket used.  PKV_E_ARG if batch exceeds the largest
 * bucket. */
pkv_status pkv_graph_set_replay(pkv_graph_set* set, int batch, pkv_stream_t stream, int* bucket_out);
void pkv_graph_set_destroy(pkv_graph_set* set);

/* ----------------------------------------------------- host block allocator */

/* The block allocator of a paged cache (aitrends.kr glossary, 용어 해설,
 * PagedAttention entry: the cache is split into fixed-size pages, so memory
 * is handed out page by page and not reserved per sequence; rvLLM post,
 * section "CUDA 그래프 리플레이": block tables are host metadata uploaded
 * before each step).  Host memory only; no device call.
 * Free list of num_blocks physical block ids.  seed 0 hands ids out in
 * ascending order; any other seed shuffles the free list once (deterministic
 * for a given seed), which tests use to scatter a sequence's blocks. */
pkv_status pkv_alloc_create(int num_blocks, uint64_t seed, pkv_alloc** out);
/* Grow a (host) block-table row from old_len to new_len tokens: fills entries
 * [ceil(old_len/16), ceil(new_len/16)) with fresh ids.  PKV_E_CAPACITY (row
 * and allocator unchanged) when not enough blocks are free; PKV_E_ARG when
 * new_len < old_len or the row is too short. */
pkv_status pkv_alloc_grow(pkv_alloc* alloc, int32_t* row, int bt_stride, int old_len, int new_len);
/* Return the ceil(len/16) blocks of a (host) row to the free list. */
pkv_status pkv_alloc_release(pkv_alloc* alloc, const int32_t* row, int len);
int pkv_alloc_free_blocks(const pkv_alloc* alloc);
void pkv_alloc_destroy(pkv_alloc* alloc);

/* Check (host) metadata: every length in [0, max_context], every needed block
 * id in [0, num_blocks), no block used twice across rows, and
 * bt_stride >= ceil(max_context / 16).  PKV_E_ARG with a message otherwise.
 * These are the per-step block tables and context lengths of the rvLLM post
 * (section "CUDA 그래프 리플레이"), which the device path trusts; this check is
 * for callers and tests that hold host copies. */
pkv_status pkv_validate_metadata(const int32_t* block_tables, int bt_stride,
                                 const int32_t* context_lens, int batch, int num_blocks,
                                 int max_context);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
