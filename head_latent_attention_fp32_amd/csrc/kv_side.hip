// Key/value side of new tokens on gfx950: split of the joint down-projection's output, latent
// RMSNorm, rotary key, and the write into the decode caches.
//
// Follows "DeepSeek-V3.2-Exp · Query heads", MLA __init__ excerpt (wkv_a gives kv_lora + rope
// features per token; kv_norm normalises the latent) and "Kimi-K2 · value_states", mla-init and
// mla-prefill excerpts (kv_a_proj_with_mqa, kv_a_layernorm; the rotary key is rotated together
// with q_pe); the caches hold one row per position, as the mla-decode excerpt of
// "DeepSeek-V3.2-Exp · Attention update" reads them (kv_cache[:bsz, :end_pos]).
//
// One wave per token, HBM-bound (1152 bytes in, 1152 out): lane l holds latent features
// 8l .. 8l+7 (one 16-byte load), sums their squares, and after a wave reduction writes
// bf16(gain * x * inv_rms) to the latent cache row; lanes 0-7 also hold rotary features 8l .. 8l+7
// (4 interleaved pairs) and write them rotated by their (cos, sin) to the rotary cache row.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ kv_a, const float* __restrict__ gamma, const float* __restrict__ rope_cs,
    int batch, int seqlen, const int32_t* __restrict__ start_pos, const int64_t* __restrict__ row_offset,
    int64_t max_seqlen, float eps, uint16_t* __restrict__ kv_cache, uint16_t* __restrict__ pe_cache) {
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= static_cast<int64_t>(batch) * seqlen) return;
  const int b = static_cast<int>(tok / seqlen);
  const int t = static_cast<int>(tok - static_cast<int64_t>(b) * seqlen);
  const int64_t pos = static_cast<int64_t>(start_pos[b]) + t;
  if (pos < 0 || pos >= max_seqlen) return;   // positions outside the cache are not stored
  const int64_t row = (row_offset ? row_offset[b] : static_cast<int64_t>(b) * max_seqlen) + pos;
  const uint16_t* src = kv_a + tok * kLat;

  const bf16x8 v = as_bf16x8(ldg16(src + lane * 8));
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = static_cast<float>(v[e]);
    s += f * f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  const float iv = 1.f / sqrtf(s * (1.f / kKvLora) + eps);
  const float4 g0 = *reinterpret_cast<const float4*>(gamma + lane * 8);
  const float4 g1 = *reinterpret_cast<const float4*>(gamma + lane * 8 + 4);
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = g[e] * (static_cast<float>(v[e]) * iv);
  *reinterpret_cast<bf16x8*>(kv_cache + row * kKvLora + lane * 8) = bf16x8_from_f32(o);

  if (lane < kRope / 8) {
    const bf16x8 p = as_bf16x8(ldg16(src + kKvLora + lane * 8));
    const float* cs = rope_cs + tok * kRope + lane * 8;   // (cos, sin) of pairs 4 lane .. 4 lane + 3
    const float4 c0 = *reinterpret_cast<const float4*>(cs);
    const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = static_cast<float>(p[2 * i]), bb = static_cast<float>(p[2 * i + 1]);
      const float cc = c[2 * i], sn = c[2 * i + 1];
      r[2 * i] = a * cc - bb * sn;
      r[2 * i + 1] = a * sn + bb * cc;
    }
    *reinterpret_cast<bf16x8*>(pe_cache + row * kRope + lane * 8) = bf16x8_from_f32(r);
  }
}

}  // namespace

hipError_t launch_kv_append(int batch, int seqlen, const uint16_t* kv_a, const float* kv_norm_w,
                            const float* rope_cs, const int32_t* start_pos, const int64_t* row_offset,
                            int64_t max_seqlen, float eps, uint16_t* kv_cache, uint16_t* pe_cache,
                            hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(batch) * seqlen;
  kv_append_kernel<<<static_cast<unsigned>((n + 3) / 4), 256, 0, stream>>>(
      kv_a, kv_norm_w, rope_cs, batch, seqlen, start_pos, row_offset, max_seqlen, eps, kv_cache, pe_cache);
  return hipGetLastError();
}

}  // namespace mla
