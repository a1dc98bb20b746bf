/*
 * mla.h -- C ABI of libmla: multi-head latent attention (MLA) for AMD Instinct MI355X (gfx950).
 *
 * Three entry points follow the hot path of DeepSeek/Kimi-style MLA:
 *   mla_query_path  RMSNorm of the query latent (fp32, learned gain) -> wq_b up-projection to
 *                   H heads of 128 content + 64 rotary features -> RoPE on the rotary part.
 *                   Source: "DeepSeek-V3.2-Exp · Query heads" (equations, in/out shapes, query code
 *                   excerpt) and "DeepSeek V4.1 · Query RMSNorm" (equation, RMSNorm excerpt).
 *   mla_decode      absorbed decode of one new token per sequence over the cached latent:
 *                   q_nope folded through the key half of wkv_b, scores = 512-wide latent dot +
 *                   64-wide rotary dot, scaled softmax, weighted latent sum projected out through
 *                   the value half of wkv_b.
 *                   Source: "DeepSeek-V3.2-Exp · Attention update", mla-decode (MQA decode) excerpt;
 *                   "Kimi-K2 · value_states" (value reconstruction shapes).
 *   mla_prefill     non-absorbed causal prefill: latent expanded through wkv_b to per-head k_nope
 *                   and values, keys joined with the shared rotary key, causal softmax attention.
 *                   Source: "Kimi-K2 · value_states", mla-prefill excerpt.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers. bf16 tensors are passed as uint16_t (raw bf16 bits).
 *     Every tensor is dense, row-major, with the layout stated at its argument. Every base
 *     pointer must be 16-byte aligned.
 *   - The caller owns all memory. The library never allocates or frees device memory and never
 *     synchronises: a call validates its arguments on the host, enqueues its kernels on `stream`
 *     and returns. Outputs must not alias inputs. Calls on one stream are ordered; the library
 *     keeps no mutable state besides a cached device-property record, so different streams may
 *     call concurrently if their workspaces differ.
 *   - Errors: host validation runs before any HIP call and returns MLA_ERR_* with nothing
 *     enqueued: a NULL required pointer -> MLA_ERR_INVALID_ARG; model widths the kernels are not
 *     built for -> MLA_ERR_UNSUPPORTED; negative or out-of-range sizes -> MLA_ERR_SHAPE;
 *     misaligned pointers -> MLA_ERR_ALIGNMENT; a workspace smaller than *_workspace_size
 *     reports -> MLA_ERR_WORKSPACE. A launch failure reports MLA_ERR_HIP. Faults inside kernels
 *     surface at the caller's next synchronisation. The library never aborts or prints.
 *   - Sizes of zero (n_tokens = 0, batch = 0, seqlen = 0) are valid and enqueue nothing.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_SHAPE = 3,
  MLA_ERR_ALIGNMENT = 4,
  MLA_ERR_WORKSPACE = 5,
  MLA_ERR_HIP = 6
} mla_status_t;

/* Model widths. The kernels are built for q_lora_rank 1536, kv_lora_rank 512, qk_nope_dim 128,
 * qk_rope_dim 64, v_head_dim 128 (DeepSeek-V3.2-Exp / Kimi-K2: "DeepSeek-V3.2-Exp · Query heads",
 * MLA __init__ excerpt; "Kimi-K2 · value_states", mla-init excerpt) and n_heads in {16, 32, 64, 128}
 * (one GPU's share of the heads). softmax_scale is (qk_nope_dim + qk_rope_dim)^-0.5 = 192^-0.5 in
 * the pages' configuration; rms_eps is 1e-6 (RMSNorm code default). Both are used as given. */
typedef struct {
  int32_t n_heads;
  int32_t q_lora_rank;
  int32_t kv_lora_rank;
  int32_t qk_nope_dim;
  int32_t qk_rope_dim;
  int32_t v_head_dim;
  float softmax_scale;
  float rms_eps;
} mla_dims_t;

/* Fill *dims with the pages' widths for n_heads heads, scale 192^-0.5 and eps 1e-6. */
mla_status_t mla_dims_default(int32_t n_heads, mla_dims_t* dims);

/* Bytes of device workspace mla_query_path needs for n_tokens tokens: 0 for n_tokens <= 32 (the
 * decode sizes), n_tokens * (1536 * 2 + 4) rounded up to 256-byte pieces otherwise (the normalised
 * activation and the row statistics). Host-only; no HIP call. */
mla_status_t mla_query_path_workspace_size(const mla_dims_t* dims, int64_t n_tokens, size_t* bytes);

/* Query path ("DeepSeek-V3.2-Exp · Query heads": q^C = c^Q W_UQ, q^pe = c^Q W_QR,
 * Q^R = RoPE(Q^pe, R), Q = [Q^C; Q^R]; c^Q = RMSNorm(q latent) per "DeepSeek V4.1 · Query RMSNorm").
 *   n_tokens  0 .. 8,388,480
 *   q_latent  bf16 [n_tokens, q_lora_rank]           query latent (output of wq_a)
 *   q_norm_w  fp32 [q_lora_rank]                      RMSNorm gain
 *   wq_b      bf16 [q_lora_rank, n_heads*192]         input x output; head h owns columns
 *                                                     h*192 .. h*192+191 (128 content, then 64 rotary)
 *   rope_cs   fp32 [n_tokens, 32, 2]                  R row of each token: (cos, sin) of each pair
 *   q_out     bf16 [n_tokens, n_heads, 192]           token-major query heads
 *   inv_rms   fp32 [n_tokens] or NULL                 1/sqrt(mean(x^2) + eps) of each token
 *   workspace >= mla_query_path_workspace_size bytes; may be NULL when that size is 0
 * Arithmetic: inv_rms in fp32; y = bf16(gain * x * inv_rms) (rounded before the product, as the
 * RMSNorm excerpt casts back to the input dtype); q = bf16(y @ wq_b) with fp32 accumulation; rotary
 * pairs (2i, 2i+1) of each head rotate as (a,b) -> (a cos - b sin, a sin + b cos) from the bf16
 * product and are rounded to bf16 again.
 * Errors: MLA_ERR_WORKSPACE when workspace_bytes is below the size query; MLA_ERR_INVALID_ARG for a
 * NULL workspace when one is needed. */
mla_status_t mla_query_path(const mla_dims_t* dims, int64_t n_tokens,
                            const uint16_t* q_latent, const float* q_norm_w, const uint16_t* wq_b,
                            const float* rope_cs, uint16_t* q_out, float* inv_rms,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Query weights in the decode-friendly layout (the same values, rearranged once when the weights
 * are loaded; "DeepSeek-V3.2-Exp · Query heads": wq_b maps the 1536 query-latent features to the
 * n_heads*192 query features):
 *   wq_b         bf16 [q_lora_rank, n_heads*192]           as mla_query_path takes it
 *   wq_b_packed  bf16 [n_heads*192/32, q_lora_rank, 32]    output: wq_b_packed[g][k][j] = wq_b[k][32g + j],
 *                                                          the same number of bytes as wq_b
 * Each group of 32 output columns then holds its 1536 input rows back to back, so that the column
 * slices the query products stream are a few contiguous runs instead of short pieces of every row.
 * Pure data movement: bit-exact; not in place. Errors: MLA_ERR_INVALID_ARG for a NULL pointer or
 * for byte ranges of wq_b and wq_b_packed that overlap, MLA_ERR_ALIGNMENT, MLA_ERR_UNSUPPORTED for
 * other widths. */
mla_status_t mla_wq_b_pack(const mla_dims_t* dims, const uint16_t* wq_b, uint16_t* wq_b_packed, hipStream_t stream);

/* mla_query_path on the packed weights of mla_wq_b_pack: the same arguments, sizes, workspace and
 * errors, wq_b_packed in place of wq_b, and bit-identical outputs (the products read the same
 * weight tiles in the same order; only where they come from in memory differs). */
mla_status_t mla_query_path_packed(const mla_dims_t* dims, int64_t n_tokens,
                                   const uint16_t* q_latent, const float* q_norm_w, const uint16_t* wq_b_packed,
                                   const float* rope_cs, uint16_t* q_out, float* inv_rms,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace mla_decode needs for `batch` sequences of at most max_seqlen cached
 * rows each. Host-only; no HIP call. */
mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t max_seqlen,
                                       size_t* bytes);

/* Absorbed decode ("DeepSeek-V3.2-Exp · Attention update", mla-decode excerpt), one query token
 * per sequence, dense over all cached rows of the sequence:
 *   q_lat[b,h,:] = bf16(q_nope[b,h,:] . W_UK[h])                     (W_UK[h] = wkv_b rows h*256 .. +127)
 *   s[b,h,t]     = scale * (q_lat[b,h,:] . kv[t,:] + q_pe[b,h,:] . pe[t,:]),   t < L_b
 *   o_lat[b,h,:] = sum_t softmax_t(s) kv[t,:]                         (fp32 softmax and sums)
 *   out[b,h,d]   = bf16(sum_c o_lat[b,h,c] W_UV[h,d,c])              (W_UV[h] = wkv_b rows h*256+128 .. +255)
 *   lse[b,h]     = ln sum_t exp(s[b,h,t])
 *   q                 bf16 [batch, n_heads, 192]   query heads of the new token (mla_query_path output)
 *   wkv_b             bf16 [n_heads*256, 512]      output x input
 *   kv_cache          bf16 rows of 512             cached (normalised) latent
 *   pe_cache          bf16 rows of 64              cached rotated rotary key
 *   cache_row_offset  int64 [batch] or NULL        first cache row of sequence b; NULL = b*max_seqlen
 *   cache_seqlens     int32 [batch]                L_b (device); values are clamped to [0, max_seqlen]
 *   max_seqlen        host upper bound on L_b, 0 .. 2,097,152 (2^21)
 *   workspace         >= mla_decode_workspace_size bytes of device memory (contents need not be
 *                     initialised; overwritten by the call)
 *   out               bf16 [batch, n_heads, 128]
 *   lse               fp32 [batch, n_heads] or NULL
 * A sequence with L_b = 0 gets out = 0 and lse = -inf. Rows beyond L_b are never read. */
mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                        const uint16_t* kv_cache, const uint16_t* pe_cache,
                        const int64_t* cache_row_offset, const int32_t* cache_seqlens, int64_t max_seqlen,
                        void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                        hipStream_t stream);

/* mla_decode without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * computation and results as mla_decode; the scratch memory mla_decode takes from `workspace`
 * (run plan, absorbed queries, split partials) comes instead from a fixed device array of
 * MLA_DECODE_NOALLOC_SCRATCH_BYTES inside the library, of which every GPU the library runs on holds
 * its own copy until the process ends (its address is looked up on the first call on a device).
 * The call allocates and frees nothing. A batch whose mla_decode_workspace_size exceeds that size
 * returns MLA_ERR_WORKSPACE with nothing enqueued (at 128 heads: up to 128 sequences of any length
 * up to 2^21). Every call on one GPU uses the same array and leaves its contents behind (nothing in
 * it has to start at zero): calls that overlap on one GPU -- on different streams, or from
 * different threads without ordering -- race and give undefined results. */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                                const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                                const int32_t* cache_seqlens, int64_t max_seqlen, uint16_t* out, float* lse,
                                hipStream_t stream);

/* Bytes of device workspace mla_prefill needs (holds the expanded per-head k_nope and values).
 * Host-only; no HIP call. batch in [0, 65535] and batch * seqlen <= 2^23 key positions, else
 * MLA_ERR_SHAPE (the same limits hold for mla_prefill and, with kv_len, mla_prefill_with_prefix). */
mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t seqlen, size_t* bytes);

/* Non-absorbed causal prefill ("Kimi-K2 · value_states", mla-prefill excerpt), start position 0:
 *   k_nope[b,t,h,:] = bf16(W_UK[h] kv_latent[b,t,:]),  v[b,t,h,:] = bf16(W_UV[h] kv_latent[b,t,:])
 *   key[b,t,h] = [k_nope[b,t,h,:] ; k_pe[b,t,:]]       (the rotary key is shared by every head)
 *   s = scale * q . key, keys t' <= t only; fp32 online softmax; out = bf16(sum_t' p v)
 *   q          bf16 [batch, seqlen, n_heads, 192]   query heads (mla_query_path output)
 *   kv_latent  bf16 [batch, seqlen, 512]            normalised latent, as it would be cached
 *   k_pe       bf16 [batch, seqlen, 64]             rotated rotary key, as it would be cached
 *   wkv_b      bf16 [n_heads*256, 512]
 *   workspace  >= mla_prefill_workspace_size bytes
 *   out        bf16 [batch, seqlen, n_heads, 128]
 *   lse        fp32 [batch, n_heads, seqlen] or NULL
 * batch > 65535 or batch * seqlen > 2^23 -> MLA_ERR_SHAPE. */
mla_status_t mla_prefill(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* q,
                         const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b,
                         void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                         hipStream_t stream);

/* Bytes of device workspace mla_decode_sparse needs for `batch` sequences and lists of `topk`
 * entries (host-only, no HIP calls). topk in [0, 2^21]. */
mla_status_t mla_decode_sparse_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t max_seqlen,
                                              int32_t topk, size_t* bytes);

/* Absorbed decode restricted to each sequence's top-k positions ("DeepSeek-V3.2-Exp · Attention
 * update", mla-decode excerpt: the indexer's top-k positions give a mask of 0 at those positions and
 * -inf elsewhere, added to the scores before the softmax). Same computation and arguments as
 * mla_decode, over the rows of sequence b at the positions topk_indices[b, :] names:
 *   topk_indices  int32 [batch, topk], device: positions within sequence b (0-based, as cache rows
 *                 cache_row_offset[b] + position). Entries outside [0, L_b) name no position (e.g.
 *                 -1 padding of a list longer than the sequence). A position listed more than once
 *                 is attended once, as the excerpt's scattered mask counts it. For max_seqlen up
 *                 to 491,520 the named positions are attended in ascending order; beyond, in the
 *                 order of their first entries (and for lists longer than 2048 entries the
 *                 workspace then holds a table of about 16 bytes per entry).
 *   topk          entries per list, 0 .. 2^21
 *   workspace     >= mla_decode_sparse_workspace_size(dims, batch, max_seqlen, topk) bytes
 * The order of a list does not matter beyond floating-point summation order. A sequence with no
 * valid entry gets out = 0, lse = -inf. */
mla_status_t mla_decode_sparse(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                               const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                               const int32_t* cache_seqlens, int64_t max_seqlen, const int32_t* topk_indices,
                               int32_t topk, void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                               hipStream_t stream);

/* Causal prefill of new tokens over a cached prefix ("Kimi-K2 · value_states", mla-prefill excerpt:
 * once past keys join the new ones the weights and mask are (q_len, kv_seq_len)). The sequence has
 * kv_len positions; the queries are its last q_len (q_len <= kv_len), query i at position
 * kv_len - q_len + i, and see keys 0 .. kv_len - q_len + i. q_len = kv_len is mla_prefill.
 *   q          bf16 [batch, q_len, n_heads, 192]
 *   kv_latent  bf16 [batch, kv_len, 512]    normalised latent of every position (cached prefix, then
 *                                           the new tokens' own rows, e.g. as mla_kv_append wrote them)
 *   k_pe       bf16 [batch, kv_len, 64]     rotated rotary key of every position
 *   wkv_b      bf16 [n_heads*256, 512]
 *   workspace  >= mla_prefill_workspace_size(dims, batch, kv_len) bytes
 *   out        bf16 [batch, q_len, n_heads, 128]
 *   lse        fp32 [batch, n_heads, q_len] or NULL
 * kv_len < q_len, batch > 65535 or batch * kv_len > 2^23 -> MLA_ERR_SHAPE; q_len = 0 enqueues nothing. */
mla_status_t mla_prefill_with_prefix(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t kv_len,
                                     const uint16_t* q, const uint16_t* kv_latent, const uint16_t* k_pe,
                                     const uint16_t* wkv_b, void* workspace, size_t workspace_bytes,
                                     uint16_t* out, float* lse, hipStream_t stream);

/* Key/value side of new tokens and their cache rows ("DeepSeek-V3.2-Exp · Query heads", MLA __init__:
 * wkv_a gives kv_lora_rank + qk_rope_dim = 576 features per token and kv_norm normalises the latent;
 * "Kimi-K2 · value_states", mla-init and mla-prefill excerpts: the rotary key is rotated like q_pe;
 * "DeepSeek-V3.2-Exp · Attention update", mla-decode excerpt: cache rows are positions). For new
 * token t of sequence b, at position p = start_pos[b] + t:
 *   latent = bf16(kv_norm_w * x / sqrt(mean(x^2) + rms_eps)),  x = kv_a[b,t,0:512]  (fp32 math)
 *   rotary = bf16(RoPE(kv_a[b,t,512:576], rope_cs[b,t]))  interleaved pairs (2i, 2i+1),
 *            (a, b) -> (a cos - b sin, a sin + b cos)
 *   kv_cache[row] = latent, pe_cache[row] = rotary,  row = cache_row_offset[b] + p
 *   kv_a              bf16 [batch, seqlen, 576]   wkv_a output: latent (512) then rotary key (64)
 *   kv_norm_w         fp32 [512]                  kv_norm gain
 *   rope_cs           fp32 [batch, seqlen, 32, 2] (cos, sin) of each token's own position
 *   start_pos         int32 [batch], device       position of each sequence's first new token
 *   cache_row_offset  int64 [batch], device, or NULL for b * max_seqlen (a padded [batch, max_seqlen]
 *                     cache)
 *   kv_cache, pe_cache bf16 rows of 512 / 64, written in place (the caches mla_decode reads)
 * Positions outside [0, max_seqlen) are not written (a caller error that never writes out of
 * bounds). No other row is touched. Tokens must not map to the same row. */
mla_status_t mla_kv_append(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* kv_a,
                           const float* kv_norm_w, const float* rope_cs, const int32_t* start_pos,
                           const int64_t* cache_row_offset, int64_t max_seqlen, uint16_t* kv_cache,
                           uint16_t* pe_cache, hipStream_t stream);

/* Bytes of device workspace mla_output_proj needs (host-only, no HIP calls). */
mla_status_t mla_output_proj_workspace_size(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, size_t* bytes);

/* Output projection ("DeepSeek-V3.2-Exp · Attention update", mla-output excerpt and the update's
 * shape [B, 1, 7168]; "DeepSeek-V3.2-Exp · Query heads", MLA __init__: wo maps n_heads * v_head_dim
 * features to the model width):
 *   y[m, j] = bf16(sum_f x[m, f] wo[j, f]),  f = h*128 + d  (the head outputs flattened head-major)
 *   x     bf16 [n_tokens, n_heads*128]   attention outputs, e.g. mla_decode / mla_prefill `out`
 *   wo    bf16 [dim, n_heads*128]        output x input, as a Linear stores its weight
 *   y     bf16 [n_tokens, dim]
 *   dim   model width, a positive multiple of 64 (7168 for DeepSeek-V3.2)
 *   workspace >= mla_output_proj_workspace_size bytes (NULL allowed when that is 0)
 * n_tokens * n_heads * 128 and dim * n_heads * 128 must stay below 2^31 (else MLA_ERR_SHAPE). */
mla_status_t mla_output_proj(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, const uint16_t* x,
                             const uint16_t* wo, void* workspace, size_t workspace_bytes, uint16_t* y,
                             hipStream_t stream);

/* Instrumented variants: identical work, plus hipEventRecord of caller-created events on `stream`
 * at the boundaries of the library's kernel stages, so a caller can time each stage on the stream
 * it runs on. stage_events is NULL or an array of (number of stages + 1) events, any of which may be
 * NULL: event i is recorded before stage i and the last after the final stage.
 *   mla_query_path_ex, mla_query_path_packed_ex: 2 stages (RMSNorm pass -- empty when fused into
 *                      the product, 32 tokens or fewer --, product + RoPE)
 *   mla_decode_ex:     3 stages (absorb + run plan, split-KV attention, log-sum-exp combine + value projection)
 *   mla_decode_sparse_ex: the same 3 stages, the first also compacting the top-k lists
 *   mla_output_proj_ex: 2 stages (product, sum of the K-slice partials -- empty above 64 tokens)
 *   mla_prefill_ex, mla_prefill_with_prefix_ex: 2 stages (latent expansion, causal attention) */
mla_status_t mla_query_path_ex(const mla_dims_t* dims, int64_t n_tokens,
                               const uint16_t* q_latent, const float* q_norm_w, const uint16_t* wq_b,
                               const float* rope_cs, uint16_t* q_out, float* inv_rms,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_query_path_packed_ex(const mla_dims_t* dims, int64_t n_tokens,
                                      const uint16_t* q_latent, const float* q_norm_w, const uint16_t* wq_b_packed,
                                      const float* rope_cs, uint16_t* q_out, float* inv_rms,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_decode_ex(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                           const uint16_t* kv_cache, const uint16_t* pe_cache,
                           const int64_t* cache_row_offset, const int32_t* cache_seqlens, int64_t max_seqlen,
                           void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                           hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_prefill_ex(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* q,
                            const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b,
                            void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                            hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_decode_sparse_ex(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                                  const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                                  const int32_t* cache_seqlens, int64_t max_seqlen, const int32_t* topk_indices,
                                  int32_t topk, void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                                  hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_output_proj_ex(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, const uint16_t* x,
                                const uint16_t* wo, void* workspace, size_t workspace_bytes, uint16_t* y,
                                hipStream_t stream, hipEvent_t* stage_events);
mla_status_t mla_prefill_with_prefix_ex(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t kv_len,
                                        const uint16_t* q, const uint16_t* kv_latent, const uint16_t* k_pe,
                                        const uint16_t* wkv_b, void* workspace, size_t workspace_bytes,
                                        uint16_t* out, float* lse, hipStream_t stream, hipEvent_t* stage_events);

/* Static description of a status code. */
const char* mla_status_string(mla_status_t status);

/* Library version, "major.minor.patch". */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
