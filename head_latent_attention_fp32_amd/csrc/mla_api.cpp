// C ABI of libmla: host-side argument validation, workspace sizing and kernel dispatch.
// Validation runs before any HIP call; a rejected call enqueues nothing.
#include <math.h>

#include "../../include/mla.h"
#include "mla_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status_t check_dims(const mla_dims_t* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->q_lora_rank != 1536 || d->kv_lora_rank != 512 || d->qk_nope_dim != 128 || d->qk_rope_dim != 64 ||
      d->v_head_dim != 128)
    return MLA_ERR_UNSUPPORTED;
  if (d->n_heads != 16 && d->n_heads != 32 && d->n_heads != 64 && d->n_heads != 128) return MLA_ERR_UNSUPPORTED;
  if (!isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (!isfinite(d->rms_eps) || d->rms_eps < 0.f) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// The largest decode batch: the combine kernel's grid x and the int32 sequence index.
constexpr int64_t kMaxBatch = 1 << 24;
// The longest decode cache: the attention kernel addresses the rows of a sequence, and one tile
// past them, through buffer descriptors with 32-bit byte ranges (rows of 1 KiB).
constexpr int64_t kMaxSeqlen = int64_t(1) << 21;
// The largest query-path token count: the product's grid has ceil(n / 128) blocks in y (at most
// 65535).
constexpr int64_t kMaxTokens = int64_t(65535) * 128;
// Output projection: the token and weight matrices are addressed through buffer descriptors with
// 32-bit byte ranges (elements of 2 bytes).
constexpr int64_t kMaxOutElems = (int64_t(1) << 31) - 1;
// The longest top-k list of one sequence (a list of one sequence's positions).
constexpr int32_t kMaxTopk = 1 << 21;
// Prefill: at most 2^23 key positions over the batch (batch x kv_len), so that the expansion's and
// the attention's grids fit their 32-bit block counts with room to spare, and every workspace index
// stays far inside int64.
constexpr int64_t kMaxPrefillTokens = int64_t(1) << 23;
constexpr int32_t kMaxPrefillBatch = 65535;

mla_status_t check_prefill_sizes(int32_t batch, int32_t q_len, int32_t kv_len) {
  if (batch < 0 || batch > kMaxPrefillBatch || q_len < 0 || kv_len < q_len) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * kv_len > kMaxPrefillTokens) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_dims_default(int32_t n_heads, mla_dims_t* dims) {
  if (!dims) return MLA_ERR_INVALID_ARG;
  dims->n_heads = n_heads;
  dims->q_lora_rank = 1536;
  dims->kv_lora_rank = 512;
  dims->qk_nope_dim = 128;
  dims->qk_rope_dim = 64;
  dims->v_head_dim = 128;
  dims->softmax_scale = 1.0f / sqrtf(192.0f);
  dims->rms_eps = 1e-6f;
  return check_dims(dims);
}

mla_status_t mla_query_path_workspace_size(const mla_dims_t* dims, int64_t n_tokens, size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > kMaxTokens) return MLA_ERR_SHAPE;
  *bytes = mla::query_layout(dims->n_heads, n_tokens).total;
  return MLA_OK;
}

}  // extern "C"

namespace {

mla_status_t query_path_impl(const mla_dims_t* dims, int64_t n_tokens, const uint16_t* q_latent,
                             const float* q_norm_w, const uint16_t* wq_b, bool packed, const float* rope_cs,
                             uint16_t* q_out, float* inv_rms, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || n_tokens > kMaxTokens) return MLA_ERR_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!q_latent || !q_norm_w || !wq_b || !rope_cs || !q_out) return MLA_ERR_INVALID_ARG;
  const mla::QueryLayout lay = mla::query_layout(dims->n_heads, n_tokens);
  if (lay.total > 0 && !workspace) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_latent) || !aligned16(q_norm_w) || !aligned16(wq_b) || !aligned16(rope_cs) ||
      !aligned16(q_out) || (inv_rms && !aligned16(inv_rms)) || (workspace && !aligned16(workspace)))
    return MLA_ERR_ALIGNMENT;
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_query_path(dims->n_heads, n_tokens, q_latent, q_norm_w, wq_b, packed, rope_cs, q_out,
                                        inv_rms, workspace, lay, dims->rms_eps, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status_t mla_query_path_ex(const mla_dims_t* dims, int64_t n_tokens, const uint16_t* q_latent,
                               const float* q_norm_w, const uint16_t* wq_b, const float* rope_cs, uint16_t* q_out,
                               float* inv_rms, void* workspace, size_t workspace_bytes, hipStream_t stream,
                               hipEvent_t* stage_events) {
  return query_path_impl(dims, n_tokens, q_latent, q_norm_w, wq_b, false, rope_cs, q_out, inv_rms, workspace,
                         workspace_bytes, stream, stage_events);
}

mla_status_t mla_query_path(const mla_dims_t* dims, int64_t n_tokens, const uint16_t* q_latent,
                            const float* q_norm_w, const uint16_t* wq_b, const float* rope_cs, uint16_t* q_out,
                            float* inv_rms, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return query_path_impl(dims, n_tokens, q_latent, q_norm_w, wq_b, false, rope_cs, q_out, inv_rms, workspace,
                         workspace_bytes, stream, nullptr);
}

mla_status_t mla_wq_b_pack(const mla_dims_t* dims, const uint16_t* wq_b, uint16_t* wq_b_packed, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!wq_b || !wq_b_packed) return MLA_ERR_INVALID_ARG;
  if (!aligned16(wq_b) || !aligned16(wq_b_packed)) return MLA_ERR_ALIGNMENT;
  // the rearrangement cannot run in place: the two byte ranges must not overlap
  const uintptr_t a = reinterpret_cast<uintptr_t>(wq_b), b = reinterpret_cast<uintptr_t>(wq_b_packed);
  const uintptr_t bytes = static_cast<uintptr_t>(dims->q_lora_rank) * dims->n_heads *
                          (dims->qk_nope_dim + dims->qk_rope_dim) * sizeof(uint16_t);
  if (a < b + bytes && b < a + bytes) return MLA_ERR_INVALID_ARG;
  hipError_t e = mla::launch_pack_wq_b(dims->n_heads, wq_b, wq_b_packed, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_query_path_packed_ex(const mla_dims_t* dims, int64_t n_tokens, const uint16_t* q_latent,
                                      const float* q_norm_w, const uint16_t* wq_b_packed, const float* rope_cs,
                                      uint16_t* q_out, float* inv_rms, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, hipEvent_t* stage_events) {
  return query_path_impl(dims, n_tokens, q_latent, q_norm_w, wq_b_packed, true, rope_cs, q_out, inv_rms, workspace,
                         workspace_bytes, stream, stage_events);
}

mla_status_t mla_query_path_packed(const mla_dims_t* dims, int64_t n_tokens, const uint16_t* q_latent,
                                   const float* q_norm_w, const uint16_t* wq_b_packed, const float* rope_cs,
                                   uint16_t* q_out, float* inv_rms, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return query_path_impl(dims, n_tokens, q_latent, q_norm_w, wq_b_packed, true, rope_cs, q_out, inv_rms, workspace,
                         workspace_bytes, stream, nullptr);
}

mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t max_seqlen, size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  if (batch < 0 || batch > kMaxBatch || max_seqlen < 0 || max_seqlen > kMaxSeqlen) return MLA_ERR_SHAPE;
  *bytes = batch == 0 ? 0 : mla::decode_layout(dims->n_heads, batch, max_seqlen).total;
  return MLA_OK;
}

mla_status_t mla_decode_ex(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                           const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                           const int32_t* cache_seqlens, int64_t max_seqlen, void* workspace,
                           size_t workspace_bytes, uint16_t* out, float* lse, hipStream_t stream,
                           hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || max_seqlen < 0 || max_seqlen > kMaxSeqlen) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q || !wkv_b || !kv_cache || !pe_cache || !cache_seqlens || !workspace || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(wkv_b) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
      !aligned16(cache_seqlens) || !aligned16(workspace) || !aligned16(out) ||
      (cache_row_offset && !aligned16(cache_row_offset)) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGNMENT;
  const mla::DecodeLayout lay = mla::decode_layout(dims->n_heads, batch, max_seqlen);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_decode(dims->n_heads, batch, q, wkv_b, kv_cache, pe_cache, cache_row_offset,
                                    cache_seqlens, max_seqlen, nullptr, -1, workspace, lay, out, lse,
                                    dims->softmax_scale, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

static_assert(MLA_DECODE_NOALLOC_SCRATCH_BYTES == mla::kDecodeScratchBytes, "scratch size of mla.h and the library");

mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                                const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                                const int32_t* cache_seqlens, int64_t max_seqlen, uint16_t* out, float* lse,
                                hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || max_seqlen < 0 || max_seqlen > kMaxSeqlen) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q || !wkv_b || !kv_cache || !pe_cache || !cache_seqlens || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(wkv_b) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
      !aligned16(cache_seqlens) || !aligned16(out) || (cache_row_offset && !aligned16(cache_row_offset)) ||
      (lse && !aligned16(lse)))
    return MLA_ERR_ALIGNMENT;
  const mla::DecodeLayout lay = mla::decode_layout(dims->n_heads, batch, max_seqlen);
  if (lay.total > mla::kDecodeScratchBytes) return MLA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (mla::decode_scratch(&scratch) != hipSuccess) return MLA_ERR_HIP;
  hipError_t e = mla::launch_decode(dims->n_heads, batch, q, wkv_b, kv_cache, pe_cache, cache_row_offset,
                                    cache_seqlens, max_seqlen, nullptr, -1, scratch, lay, out, lse,
                                    dims->softmax_scale, stream, nullptr);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_decode_sparse_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t max_seqlen,
                                              int32_t topk, size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  if (batch < 0 || batch > kMaxBatch || max_seqlen < 0 || max_seqlen > kMaxSeqlen || topk < 0 || topk > kMaxTopk)
    return MLA_ERR_SHAPE;
  *bytes = batch == 0 ? 0 : mla::decode_layout(dims->n_heads, batch, max_seqlen, topk).total;
  return MLA_OK;
}

mla_status_t mla_decode_sparse_ex(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                                  const uint16_t* kv_cache, const uint16_t* pe_cache,
                                  const int64_t* cache_row_offset, const int32_t* cache_seqlens, int64_t max_seqlen,
                                  const int32_t* topk_indices, int32_t topk, void* workspace, size_t workspace_bytes,
                                  uint16_t* out, float* lse, hipStream_t stream, hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || max_seqlen < 0 || max_seqlen > kMaxSeqlen || topk < 0 || topk > kMaxTopk)
    return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q || !wkv_b || !kv_cache || !pe_cache || !cache_seqlens || !workspace || !out || (topk > 0 && !topk_indices))
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(wkv_b) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
      !aligned16(cache_seqlens) || !aligned16(workspace) || !aligned16(out) || (topk > 0 && !aligned16(topk_indices)) ||
      (cache_row_offset && !aligned16(cache_row_offset)) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGNMENT;
  const mla::DecodeLayout lay = mla::decode_layout(dims->n_heads, batch, max_seqlen, topk);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_decode(dims->n_heads, batch, q, wkv_b, kv_cache, pe_cache, cache_row_offset,
                                    cache_seqlens, max_seqlen, topk_indices, topk, workspace, lay, out, lse,
                                    dims->softmax_scale, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_decode_sparse(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                               const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                               const int32_t* cache_seqlens, int64_t max_seqlen, const int32_t* topk_indices,
                               int32_t topk, void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                               hipStream_t stream) {
  return mla_decode_sparse_ex(dims, batch, q, wkv_b, kv_cache, pe_cache, cache_row_offset, cache_seqlens, max_seqlen,
                              topk_indices, topk, workspace, workspace_bytes, out, lse, stream, nullptr);
}

mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch, const uint16_t* q, const uint16_t* wkv_b,
                        const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* cache_row_offset,
                        const int32_t* cache_seqlens, int64_t max_seqlen, void* workspace, size_t workspace_bytes,
                        uint16_t* out, float* lse, hipStream_t stream) {
  return mla_decode_ex(dims, batch, q, wkv_b, kv_cache, pe_cache, cache_row_offset, cache_seqlens, max_seqlen,
                       workspace, workspace_bytes, out, lse, stream, nullptr);
}

mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t seqlen, size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  if ((st = check_prefill_sizes(batch, 0, seqlen)) != MLA_OK) return st;
  *bytes = (batch == 0 || seqlen == 0) ? 0 : mla::prefill_layout(dims->n_heads, batch, seqlen).total;
  return MLA_OK;
}

mla_status_t mla_prefill_ex(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* q,
                            const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b, void* workspace,
                            size_t workspace_bytes, uint16_t* out, float* lse, hipStream_t stream,
                            hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_prefill_sizes(batch, seqlen, seqlen)) != MLA_OK) return st;
  if (batch == 0 || seqlen == 0) return MLA_OK;
  if (!q || !kv_latent || !k_pe || !wkv_b || !workspace || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_latent) || !aligned16(k_pe) || !aligned16(wkv_b) || !aligned16(workspace) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGNMENT;
  const mla::PrefillLayout lay = mla::prefill_layout(dims->n_heads, batch, seqlen);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_prefill(dims->n_heads, batch, seqlen, seqlen, q, kv_latent, k_pe, wkv_b, workspace, lay,
                                     out, lse, dims->softmax_scale, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_prefill_with_prefix_ex(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t kv_len,
                                        const uint16_t* q, const uint16_t* kv_latent, const uint16_t* k_pe,
                                        const uint16_t* wkv_b, void* workspace, size_t workspace_bytes, uint16_t* out,
                                        float* lse, hipStream_t stream, hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_prefill_sizes(batch, q_len, kv_len)) != MLA_OK) return st;
  if (batch == 0 || q_len == 0) return MLA_OK;
  if (!q || !kv_latent || !k_pe || !wkv_b || !workspace || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_latent) || !aligned16(k_pe) || !aligned16(wkv_b) || !aligned16(workspace) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return MLA_ERR_ALIGNMENT;
  const mla::PrefillLayout lay = mla::prefill_layout(dims->n_heads, batch, kv_len);
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_prefill(dims->n_heads, batch, q_len, kv_len, q, kv_latent, k_pe, wkv_b, workspace, lay,
                                     out, lse, dims->softmax_scale, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_prefill_with_prefix(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t kv_len,
                                     const uint16_t* q, const uint16_t* kv_latent, const uint16_t* k_pe,
                                     const uint16_t* wkv_b, void* workspace, size_t workspace_bytes, uint16_t* out,
                                     float* lse, hipStream_t stream) {
  return mla_prefill_with_prefix_ex(dims, batch, q_len, kv_len, q, kv_latent, k_pe, wkv_b, workspace,
                                    workspace_bytes, out, lse, stream, nullptr);
}

mla_status_t mla_kv_append(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* kv_a,
                           const float* kv_norm_w, const float* rope_cs, const int32_t* start_pos,
                           const int64_t* cache_row_offset, int64_t max_seqlen, uint16_t* kv_cache,
                           uint16_t* pe_cache, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || seqlen < 0 || max_seqlen < 0 || max_seqlen > kMaxSeqlen ||
      static_cast<int64_t>(batch) * seqlen > kMaxTokens)
    return MLA_ERR_SHAPE;
  if (batch == 0 || seqlen == 0) return MLA_OK;
  if (!kv_a || !kv_norm_w || !rope_cs || !start_pos || !kv_cache || !pe_cache) return MLA_ERR_INVALID_ARG;
  if (!aligned16(kv_a) || !aligned16(kv_norm_w) || !aligned16(rope_cs) || !aligned16(start_pos) ||
      !aligned16(kv_cache) || !aligned16(pe_cache) || (cache_row_offset && !aligned16(cache_row_offset)))
    return MLA_ERR_ALIGNMENT;
  hipError_t e = mla::launch_kv_append(batch, seqlen, kv_a, kv_norm_w, rope_cs, start_pos, cache_row_offset,
                                       max_seqlen, dims->rms_eps, kv_cache, pe_cache, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_prefill(const mla_dims_t* dims, int32_t batch, int32_t seqlen, const uint16_t* q,
                         const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b, void* workspace,
                         size_t workspace_bytes, uint16_t* out, float* lse, hipStream_t stream) {
  return mla_prefill_ex(dims, batch, seqlen, q, kv_latent, k_pe, wkv_b, workspace, workspace_bytes, out, lse, stream,
                        nullptr);
}

mla_status_t mla_output_proj_workspace_size(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  const int64_t K = static_cast<int64_t>(dims->n_heads) * dims->v_head_dim;
  if (n_tokens < 0 || dim <= 0 || dim % 64 != 0 || n_tokens * K > kMaxOutElems || dim * K > kMaxOutElems)
    return MLA_ERR_SHAPE;
  *bytes = n_tokens == 0 ? 0 : mla::out_proj_layout(dims->n_heads, n_tokens, dim).total;
  return MLA_OK;
}

mla_status_t mla_output_proj_ex(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, const uint16_t* x,
                                const uint16_t* wo, void* workspace, size_t workspace_bytes, uint16_t* y,
                                hipStream_t stream, hipEvent_t* stage_events) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  const int64_t K = static_cast<int64_t>(dims->n_heads) * dims->v_head_dim;
  if (n_tokens < 0 || dim <= 0 || dim % 64 != 0 || n_tokens * K > kMaxOutElems || dim * K > kMaxOutElems)
    return MLA_ERR_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!x || !wo || !y) return MLA_ERR_INVALID_ARG;
  const mla::OutProjLayout lay = mla::out_proj_layout(dims->n_heads, n_tokens, dim);
  if (lay.total > 0 && !workspace) return MLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wo) || !aligned16(y) || (workspace && !aligned16(workspace)))
    return MLA_ERR_ALIGNMENT;
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE;
  hipError_t e = mla::launch_out_proj(dims->n_heads, n_tokens, dim, x, wo, workspace, lay, y, stream, stage_events);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_output_proj(const mla_dims_t* dims, int64_t n_tokens, int32_t dim, const uint16_t* x,
                             const uint16_t* wo, void* workspace, size_t workspace_bytes, uint16_t* y,
                             hipStream_t stream) {
  return mla_output_proj_ex(dims, n_tokens, dim, x, wo, workspace, workspace_bytes, y, stream, nullptr);
}

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: a required pointer is NULL or a parameter is invalid";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: model widths or head count the kernels are not built for";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is negative or out of range";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT: a tensor base pointer is not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace smaller than the *_workspace_size query reports";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a kernel launch failed";
  }
  return "unknown mla_status_t";
}

const char* mla_version(void) { return "0.1.0"; }

}  // extern "C"
