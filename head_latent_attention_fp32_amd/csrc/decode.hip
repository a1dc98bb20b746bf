// Absorbed MLA decode on gfx950: one new query token per sequence, dense over its cached latent.
//
// Follows "DeepSeek-V3.2-Exp · Attention update", mla-decode (MQA decode) excerpt: the query's
// content part is absorbed through the key half of wkv_b, scores are the 512-wide latent dot plus
// the 64-wide rotary dot times the softmax scale, the softmax-weighted sum of cached latents is
// projected out through the value half of wkv_b ("Kimi-K2 · value_states": [B,1,512] -> [B,H,1,128]).
//
// Four kernels, enqueued back to back on the caller's stream:
//   1. absorb_plan   q_lat = bf16(q_nope . W_UK) per head (MFMA), and (block 0) the run plan:
//                    prefix sums of the clamped lengths and the number of runs.
//   2. attend        split-KV attention: the tokens of all sequences, back to back, are cut into
//                    equal runs; a workgroup streams its run's kv/pe rows through LDS 32 at a
//                    time, computes S^T = [kv|pe] . [q_lat|q_pe]^T and O^T += kv^T . P^T on MFMA
//                    with an fp32 online softmax, and writes one normalised partial (o, lse) per
//                    sequence it touches.
//   3. combine       log-sum-exp merge of the partials of each (sequence, head) -> o_lat (bf16), lse.
//   4. value_proj    out = bf16(o_lat . W_UV^T) per head (MFMA).
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

constexpr int kTileTok = 32;                     // cached rows per LDS tile
constexpr int kTileStride = kLat + 8;            // padded LDS row (bf16): conflict-free 16-B reads
constexpr int kChunksPerRow = kLat / 8;          // 72 sixteen-byte chunks per cached row
constexpr int kTileChunks = kTileTok * kChunksPerRow;

struct Plan {
  int64_t total_tokens;   // N = sum of clamped lengths
  int32_t runs;           // G = number of non-empty runs (<= launched units)
  int32_t pad;
};

__device__ __forceinline__ int64_t run_start(int64_t g, int64_t N, int64_t G) { return g * N / G; }
// Run containing global token x (0 <= x < N).
__device__ __forceinline__ int64_t run_of(int64_t x, int64_t N, int64_t G) { return ((x + 1) * G - 1) / N; }

// ---------------------------------------------------------------------------------------------
// 1. q_lat[b,h,c] = bf16(sum_d q[b,h,d] W_UK[h,d,c]); block (h, 64-column slice of c).
//    W_UK[h] rows are stored with c contiguous, so the slice is transposed into LDS ([c][d]) to
//    give the MFMA B operand eight consecutive d per lane. Block (0,0) also builds the plan.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_plan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ wkv_b, int batch, int n_heads,
    uint16_t* __restrict__ q_lat, const int32_t* __restrict__ seqlens, int64_t max_seqlen,
    int units, int min_unit_tokens, Plan* __restrict__ plan, int64_t* __restrict__ cum) {
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 64;

  __shared__ uint16_t wt[64][kNope + 8];
  __shared__ int64_t scan[256];

  if (blockIdx.x == 0 && blockIdx.y == 0) {
    // cum[b] = sum_{b' < b} clamp(L_b', 0, max_seqlen); each thread owns a contiguous chunk.
    const int per = (batch + 255) / 256;
    const int b0 = min(batch, tid * per), b1 = min(batch, b0 + per);
    int64_t s = 0;
    for (int b = b0; b < b1; ++b) s += min<int64_t>(max<int64_t>(seqlens[b], 0), max_seqlen);
    scan[tid] = s;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int64_t v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int64_t run = scan[tid] - s;
    for (int b = b0; b < b1; ++b) {
      cum[b] = run;
      run += min<int64_t>(max<int64_t>(seqlens[b], 0), max_seqlen);
    }
    if (tid == 255) {
      const int64_t N = scan[255];
      cum[batch] = N;
      int64_t G = (N + min_unit_tokens - 1) / min_unit_tokens;
      G = min<int64_t>(G, units);
      plan->total_tokens = N;
      plan->runs = static_cast<int32_t>(N > 0 ? max<int64_t>(G, 1) : 0);
      plan->pad = 0;
    }
  }

  // Transposed W_UK[h][0:128][c0:c0+64] -> wt[c][d].
  const uint16_t* wk = wkv_b + static_cast<int64_t>(h) * kKvRows * kKvLora + c0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int d = idx >> 3, ch = idx & 7;
    const uint4 v = ldg16(wk + static_cast<int64_t>(d) * kKvLora + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) wt[ch * 8 + e][d] = u4_elem(v, e);
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  bf16x8 bw[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    bw[ks] = *reinterpret_cast<const bf16x8*>(&wt[wave * 16 + r][ks * 32 + grp * 8]);

  for (int b0 = 0; b0 < batch; b0 += 16) {
    const int b = b0 + r;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* qrow = q + (static_cast<int64_t>(min(b, batch - 1)) * n_heads + h) * kQk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a = as_bf16x8(ldg16(qrow + ks * 32 + grp * 8));
      acc = mfma16x16x32(a, bw[ks], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bb = b0 + grp * 4 + j;
      if (bb < batch)
        q_lat[(static_cast<int64_t>(bb) * n_heads + h) * kKvLora + c0 + wave * 16 + r] = f32_to_bf16_bits(acc[j]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 2. Split-KV attention over runs. NW waves, wave w owns heads 16w .. 16w+15 (H = 16 NW).
// ---------------------------------------------------------------------------------------------
template <int NW>
__global__ __launch_bounds__(NW * 64) void attend_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ pe, const int64_t* __restrict__ row_offset, int64_t max_seqlen,
    const Plan* __restrict__ plan, const int64_t* __restrict__ cum, int batch, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_l) {
  constexpr int H = 16 * NW;
  constexpr int NT = NW * 64;
  constexpr int CH = (kTileChunks + NT - 1) / NT;

  const int64_t N = plan->total_tokens;
  const int64_t G = plan->runs;
  const int64_t g = blockIdx.x;
  if (g >= G) return;

  __shared__ __attribute__((aligned(16))) uint16_t tile[kTileTok * kTileStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int head = wave * 16 + r;

  int64_t start = run_start(g, N, G);
  const int64_t end = run_start(g + 1, N, G);
  // First sequence whose rows reach past `start`.
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid + 1] > start) hi = mid; else lo = mid + 1;
  }
  int b = lo;

  while (start < end) {
    const int64_t seq0 = cum[b];
    const int64_t seg_end = min(end, cum[b + 1]);
    const int64_t t0 = start - seq0, t1 = seg_end - seq0;
    const int64_t base_row = row_offset ? row_offset[b] : static_cast<int64_t>(b) * max_seqlen;

    // Query of (b, head) as MFMA B operand: 16 k-steps of the absorbed latent, 2 of the rotary part.
    bf16x8 qf[18];
    {
      const uint16_t* ql = q_lat + (static_cast<int64_t>(b) * H + head) * kKvLora + grp * 8;
      const uint16_t* qp = q + (static_cast<int64_t>(b) * H + head) * kQk + kNope + grp * 8;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = as_bf16x8(ldg16(ql + ks * 32));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) qf[16 + ks] = as_bf16x8(ldg16(qp + ks * 32));
    }

    float m = -INFINITY, lsum = 0.f;
    f32x4 o[32];
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 pf[CH];
    auto fetch = [&](int64_t tt0) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int i = tid + k * NT;
        if (i < kTileChunks) {
          const int row = i / kChunksPerRow, ch = i - row * kChunksPerRow;
          const int64_t t = min(tt0 + row, t1 - 1);   // tail rows re-read the last valid row
          const int64_t cr = base_row + t;
          pf[k] = ch < 64 ? ldg16(kv + cr * kKvLora + ch * 8) : ldg16(pe + cr * kRope + (ch - 64) * 8);
        }
      }
    };
    auto stash = [&]() {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int i = tid + k * NT;
        if (i < kTileChunks) {
          const int row = i / kChunksPerRow, ch = i - row * kChunksPerRow;
          *reinterpret_cast<uint4*>(&tile[row * kTileStride + ch * 8]) = pf[k];
        }
      }
    };

    const int n_tiles = static_cast<int>((t1 - t0 + kTileTok - 1) / kTileTok);
    fetch(t0);
    for (int it = 0; it < n_tiles; ++it) {
      __syncthreads();
      stash();
      __syncthreads();
      const int64_t tt0 = t0 + static_cast<int64_t>(it) * kTileTok;
      if (it + 1 < n_tiles) fetch(tt0 + kTileTok);

      // S^T[token][head] for the 32 tokens of the tile: two 16-token blocks.
      f32x4 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* arow = &tile[(mb * 16 + r) * kTileStride + grp * 8];
#pragma unroll
        for (int ks = 0; ks < 18; ++ks)
          acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(arow + ks * 32), qf[ks], acc);
        s[mb] = acc;
      }
      const int64_t valid = t1 - tt0;   // tokens of this tile that belong to the run
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (mb * 16 + grp * 4 + j >= valid) s[mb][j] = -INFINITY;
          mx = fmaxf(mx, s[mb][j]);
        }
      mx = max_over_rows(mx);
      const float m_new = fmaxf(m, mx);
      const float alpha = exp2f((m - m_new) * scale_log2);
      const float mref = m_new * scale_log2;
      float p[8];
      float ps = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[mb * 4 + j] = exp2f(s[mb][j] * scale_log2 - mref);
          ps += p[mb * 4 + j];
        }
      lsum = lsum * alpha + ps;
      m = m_new;
      const bf16x8 pb = bf16x8_from_f32(p);

      // O^T[c][head] += kv^T[c][token] . P^T[token][head]; k index e of lane group grp is token
      // (e/4)*16 + 4*grp + e%4, matching where P^T's values sit.
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        const uint16_t* col = &tile[(grp * 4) * kTileStride + cb * 16 + r];
        uint4 u;
        u.x = static_cast<uint32_t>(col[0]) | (static_cast<uint32_t>(col[kTileStride]) << 16);
        u.y = static_cast<uint32_t>(col[2 * kTileStride]) | (static_cast<uint32_t>(col[3 * kTileStride]) << 16);
        u.z = static_cast<uint32_t>(col[16 * kTileStride]) | (static_cast<uint32_t>(col[17 * kTileStride]) << 16);
        u.w = static_cast<uint32_t>(col[18 * kTileStride]) | (static_cast<uint32_t>(col[19 * kTileStride]) << 16);
        o[cb] = o[cb] * alpha;
        o[cb] = mfma16x16x32(as_bf16x8(u), pb, o[cb]);
      }
    }

    const float ltot = sum_over_rows(lsum);
    const float inv = 1.f / ltot;
    const int64_t slot = g + b;
    float* po = part_o + (slot * H + head) * kKvLora + grp * 4;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float4 v = make_float4(o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv);
      *reinterpret_cast<float4*>(po + cb * 16) = v;
    }
    if (grp == 0) part_l[slot * H + head] = (m * scale_log2 + __log2f(ltot)) * kLn2;

    start = seg_end;
    ++b;
    while (b < batch && cum[b + 1] <= start) ++b;
  }
}

// ---------------------------------------------------------------------------------------------
// 3. Merge the partials of (b, 16 heads): thread = (head, 32 consecutive latent columns).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(
    const Plan* __restrict__ plan, const int64_t* __restrict__ cum, int n_heads,
    const float* __restrict__ part_o, const float* __restrict__ part_l, uint16_t* __restrict__ o_lat,
    float* __restrict__ lse) {
  const int b = blockIdx.x;
  const int h = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int c0 = (threadIdx.x & 15) * 32;
  const int64_t N = plan->total_tokens, G = plan->runs;
  const int64_t x0 = cum[b], x1 = cum[b + 1];
  uint16_t* dst = o_lat + (static_cast<int64_t>(b) * n_heads + h) * kKvLora + c0;
  if (x1 <= x0) {
#pragma unroll
    for (int i = 0; i < 32; i += 8) *reinterpret_cast<uint4*>(dst + i) = make_uint4(0, 0, 0, 0);
    if (lse && (threadIdx.x & 15) == 0) lse[static_cast<int64_t>(b) * n_heads + h] = -INFINITY;
    return;
  }
  const int64_t g0 = run_of(x0, N, G), g1 = run_of(x1 - 1, N, G);
  float M = -INFINITY;
  for (int64_t g = g0; g <= g1; ++g) M = fmaxf(M, part_l[(g + b) * n_heads + h]);
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  for (int64_t g = g0; g <= g1; ++g) {
    const int64_t slot = g + b;
    const float w = __expf(part_l[slot * n_heads + h] - M);
    wsum += w;
    const float4* src = reinterpret_cast<const float4*>(part_o + (slot * n_heads + h) * kKvLora + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      acc[4 * i + 0] += w * v.x;
      acc[4 * i + 1] += w * v.y;
      acc[4 * i + 2] += w * v.z;
      acc[4 * i + 3] += w * v.w;
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    uint4 u;
    u.x = pack_bf16x2(acc[i + 0] * inv, acc[i + 1] * inv);
    u.y = pack_bf16x2(acc[i + 2] * inv, acc[i + 3] * inv);
    u.z = pack_bf16x2(acc[i + 4] * inv, acc[i + 5] * inv);
    u.w = pack_bf16x2(acc[i + 6] * inv, acc[i + 7] * inv);
    *reinterpret_cast<uint4*>(dst + i) = u;
  }
  if (lse && (threadIdx.x & 15) == 0) lse[static_cast<int64_t>(b) * n_heads + h] = M + __logf(wsum);
}

// ---------------------------------------------------------------------------------------------
// 4. out[b,h,d] = bf16(sum_c o_lat[b,h,c] W_UV[h,d,c]); block (h, 64 values of d), wave = 16 d.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void value_proj_kernel(
    const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ wkv_b, int batch, int n_heads,
    uint16_t* __restrict__ out) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int d = blockIdx.y * 64 + wave * 16 + r;
  const uint16_t* wrow = wkv_b + (static_cast<int64_t>(h) * kKvRows + kNope + d) * kKvLora + grp * 8;
  bf16x8 bw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) bw[ks] = as_bf16x8(ldg16(wrow + ks * 32));
  for (int b0 = 0; b0 < batch; b0 += 16) {
    const int b = min(b0 + r, batch - 1);
    const uint16_t* arow = o_lat + (static_cast<int64_t>(b) * n_heads + h) * kKvLora + grp * 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) acc = mfma16x16x32(as_bf16x8(ldg16(arow + ks * 32)), bw[ks], acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bb = b0 + grp * 4 + j;
      if (bb < batch) out[(static_cast<int64_t>(bb) * n_heads + h) * kVDim + blockIdx.y * 64 + wave * 16 + r] =
          f32_to_bf16_bits(acc[j]);
    }
  }
}

}  // namespace

DecodeLayout decode_layout(int n_heads, int batch, int64_t max_seqlen) {
  DecodeLayout L{};
  L.min_unit_tokens = 256;
  const int64_t upper = static_cast<int64_t>(batch) * max_seqlen;
  int64_t units = (upper + L.min_unit_tokens - 1) / L.min_unit_tokens;
  units = units < 1 ? 1 : (units > 256 ? 256 : units);
  L.units = static_cast<int>(units);
  const size_t B = static_cast<size_t>(batch), H = static_cast<size_t>(n_heads);
  const size_t slots = static_cast<size_t>(L.units) + B;
  size_t off = 0;
  L.plan_off = off;   off = align_up(off + sizeof(Plan));
  L.cum_off = off;    off = align_up(off + (B + 1) * sizeof(int64_t));
  L.qlat_off = off;   off = align_up(off + B * H * kKvLora * sizeof(uint16_t));
  L.part_o_off = off; off = align_up(off + slots * H * kKvLora * sizeof(float));
  L.part_l_off = off; off = align_up(off + slots * H * sizeof(float));
  L.olat_off = off;   off = align_up(off + B * H * kKvLora * sizeof(uint16_t));
  L.total = off;
  return L;
}

hipError_t launch_decode(int n_heads, int batch, const uint16_t* q, const uint16_t* wkv_b,
                         const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* row_offset,
                         const int32_t* seqlens, int64_t max_seqlen, void* workspace,
                         const DecodeLayout& lay, uint16_t* out, float* lse, float scale,
                         hipStream_t stream, hipEvent_t* ev) {
  char* ws = static_cast<char*>(workspace);
  Plan* plan = reinterpret_cast<Plan*>(ws + lay.plan_off);
  int64_t* cum = reinterpret_cast<int64_t*>(ws + lay.cum_off);
  uint16_t* q_lat = reinterpret_cast<uint16_t*>(ws + lay.qlat_off);
  float* part_o = reinterpret_cast<float*>(ws + lay.part_o_off);
  float* part_l = reinterpret_cast<float*>(ws + lay.part_l_off);
  uint16_t* o_lat = reinterpret_cast<uint16_t*>(ws + lay.olat_off);
  const float scale_log2 = scale * kLog2e;

  mark(ev, 0, stream);
  absorb_plan_kernel<<<dim3(n_heads, kKvLora / 64), 256, 0, stream>>>(
      q, wkv_b, batch, n_heads, q_lat, seqlens, max_seqlen, lay.units, lay.min_unit_tokens, plan, cum);
  mark(ev, 1, stream);
  switch (n_heads) {
    case 16: attend_kernel<1><<<lay.units, 64, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen,
                                                            plan, cum, batch, scale_log2, part_o, part_l); break;
    case 32: attend_kernel<2><<<lay.units, 128, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen,
                                                             plan, cum, batch, scale_log2, part_o, part_l); break;
    case 64: attend_kernel<4><<<lay.units, 256, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen,
                                                             plan, cum, batch, scale_log2, part_o, part_l); break;
    case 128: attend_kernel<8><<<lay.units, 512, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen,
                                                              plan, cum, batch, scale_log2, part_o, part_l); break;
    default: return hipErrorInvalidValue;
  }
  mark(ev, 2, stream);
  combine_kernel<<<dim3(batch, n_heads / 16), 256, 0, stream>>>(plan, cum, n_heads, part_o, part_l, o_lat, lse);
  mark(ev, 3, stream);
  value_proj_kernel<<<dim3(n_heads, kVDim / 64), 256, 0, stream>>>(o_lat, wkv_b, batch, n_heads, out);
  mark(ev, 4, stream);
  return hipGetLastError();
}

}  // namespace mla
