// Host-side internals of libmla: workspace layouts and kernel launchers (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Records stage-boundary event i (if the caller supplied one) on the stream.
inline void mark(hipEvent_t* ev, int i, hipStream_t stream) {
  if (ev && ev[i]) (void)hipEventRecord(ev[i], stream);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Split-KV decode. The cached tokens of all sequences, taken back to back, are cut into at most
// `units` equal runs; one workgroup attends one run (which may span several sequences) and writes
// one partial result per (run, sequence) pair it touches, in slot run + sequence.
// Top-k mode (topk >= 0) attends, per sequence, only the positions its list names: the list is
// first compacted (list_off, count_off) and the runs cover the compacted positions.
struct DecodeLayout {
  int units;            // workgroups launched for the split attention
  int min_unit_tokens;  // fewer tokens than this per run are not worth a partial
  int topk_slots;       // top-k mode: slots of each sequence's first-entry table
  size_t plan_off, cum_off, runs_off, qlat_off, part_o_off, part_s_off, part_l_off, list_off, count_off, table_off,
      total;
};
DecodeLayout decode_layout(int n_heads, int batch, int64_t max_seqlen, int topk = -1);

struct PrefillLayout {
  int64_t t_pad;        // sequence length padded to the key tile
  size_t knope_off, vt_off;
  size_t bound_off;     // fp32: per-head max row L1 norm of W_UV [H], then max |latent| per slot [256]
  size_t vexp_off;      // int32 [H]: the power of two the stored values are divided by
  size_t total;
};
PrefillLayout prefill_layout(int n_heads, int batch, int seqlen);

// Query path for more than 32 tokens: the normalised activation y [n][1536] bf16 (row-major for
// many tokens, `large`, else in the mid-size product's LDS-image order) and, when the caller passes
// no inv_rms, the per-token statistics. Empty for 32 tokens or fewer.
struct QueryLayout {
  bool large;
  size_t y_off, inv_off, total;
};
QueryLayout query_layout(int n_heads, int64_t n_tokens);

// wq_b as stored ([1536][H*192]) or, packed, in 32-column groups ([H*192/32][1536][32]).
hipError_t launch_query_path(int n_heads, int64_t n_tokens, const uint16_t* q_latent, const float* gamma,
                             const uint16_t* wq_b, bool packed, const float* rope_cs, uint16_t* q_out,
                             float* inv_rms, void* workspace, const QueryLayout& lay, float eps, hipStream_t stream,
                             hipEvent_t* ev);
hipError_t launch_pack_wq_b(int n_heads, const uint16_t* wq_b, uint16_t* packed, hipStream_t stream);

// Decode on a fixed device array instead of a caller workspace (for callers that cannot allocate):
// its size, and the array's device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);

// topk < 0: dense decode; else top-k mode over int32 [batch, topk] positions topk_indices.
hipError_t launch_decode(int n_heads, int batch, const uint16_t* q, const uint16_t* wkv_b,
                         const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* row_offset,
                         const int32_t* seqlens, int64_t max_seqlen, const int32_t* topk_indices, int topk,
                         void* workspace, const DecodeLayout& lay, uint16_t* out, float* lse, float scale,
                         hipStream_t stream, hipEvent_t* ev);

// Causal prefill of the last q_len of kv_len positions (q_len <= kv_len); the workspace layout is
// prefill_layout(n_heads, batch, kv_len).
hipError_t launch_prefill(int n_heads, int batch, int q_len, int kv_len, const uint16_t* q,
                          const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b, void* workspace,
                          const PrefillLayout& lay, uint16_t* out, float* lse, float scale,
                          hipStream_t stream, hipEvent_t* ev);

// Output projection: up to kOutSmallTokens tokens stream wo, more use the tiled GEMM; either runs
// in `slices` K-slices whose fp32 partials (workspace, slices > 1) a second kernel sums.
constexpr int kOutSmallTokens = 64;
struct OutProjLayout {
  int slices;
  size_t total;
};
OutProjLayout out_proj_layout(int n_heads, int64_t n_tokens, int dim);
hipError_t launch_out_proj(int n_heads, int64_t n_tokens, int dim, const uint16_t* x, const uint16_t* wo,
                           void* workspace, const OutProjLayout& lay, uint16_t* y, hipStream_t stream,
                           hipEvent_t* ev);

hipError_t launch_kv_append(int batch, int seqlen, const uint16_t* kv_a, const float* kv_norm_w,
                            const float* rope_cs, const int32_t* start_pos, const int64_t* row_offset,
                            int64_t max_seqlen, float eps, uint16_t* kv_cache, uint16_t* pe_cache,
                            hipStream_t stream);

}  // namespace mla
