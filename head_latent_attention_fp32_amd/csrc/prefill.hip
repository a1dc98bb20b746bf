// Non-absorbed causal MLA prefill on gfx950.
//
// Follows "Kimi-K2 · value_states", mla-prefill excerpt: the cached latent is expanded through
// kv_b_proj (wkv_b) into per-head k_nope and value states; each head's key joins its k_nope with
// the rotary key shared by every head; scores are scaled, causally masked, softmaxed in fp32 and
// used to mix the values. Start position 0: query t sees keys 0..t.
//
// Two kernels:
//   1. expand   [k_nope | v] = latent . wkv_b^T per head (MFMA GEMM, bf16 outputs as the bf16
//               Linear of the excerpt). k_nope is written [b][h][t][128] and v transposed,
//               [b][h][128][t], so that the attention kernel's P.V operand reads runs of keys.
//   2. attend   flash-style causal attention: block = (b, h, 64 queries), wave = 16 queries;
//               S^T = K . Q^T and O^T += V^T . P^T on MFMA with an fp32 online softmax; the
//               score matrix never leaves registers.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

constexpr int kQBlk = 64;     // queries per block
constexpr int kKBlk = 64;     // keys per LDS tile
constexpr int kKStride = kQk + 8;       // K tile row: 128 k_nope + 64 k_pe (+ pad)
constexpr int kVStride = kKBlk + 8;     // V^T tile row: 64 keys (+ pad)

// ---------------------------------------------------------------------------------------------
// 1. Expansion: rows = B*T tokens, columns = H*256 (k_nope then v per head), K = 512.
//    Block tile 64 tokens x 64 columns; wave (wt, wc) owns 32 x 32.
// ---------------------------------------------------------------------------------------------
constexpr int EX_BT = 64, EX_BC = 64, EX_BK = 64, EX_LD = EX_BK + 8;

__global__ __launch_bounds__(256) void expand_kernel(const uint16_t* __restrict__ lat, const uint16_t* __restrict__ wkv_b,
                                                     int n_heads, int seqlen, int64_t t_pad, int64_t n_rows,
                                                     uint16_t* __restrict__ knope, uint16_t* __restrict__ vt) {
  __shared__ __attribute__((aligned(16))) uint16_t as[EX_BT * EX_LD];
  __shared__ __attribute__((aligned(16))) uint16_t bs[EX_BC * EX_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * EX_BT;
  const int col0 = blockIdx.y * EX_BC;

  uint4 areg[2], breg[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int rr = idx >> 3, ch = idx & 7;
      areg[i] = ldg16(lat + min(row0 + rr, n_rows - 1) * kKvLora + k0 + ch * 8);
      breg[i] = ldg16(wkv_b + static_cast<int64_t>(col0 + rr) * kKvLora + k0 + ch * 8);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int rr = idx >> 3, ch = idx & 7;
      *reinterpret_cast<uint4*>(&as[rr * EX_LD + ch * 8]) = areg[i];
      *reinterpret_cast<uint4*>(&bs[rr * EX_LD + ch * 8]) = breg[i];
    }
  };

  const int wt = wave >> 1, wc = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int k0 = 0; k0 < kKvLora; k0 += EX_BK) {
    __syncthreads();
    stash();
    __syncthreads();
    if (k0 + EX_BK < kKvLora) fetch(k0 + EX_BK);
#pragma unroll
    for (int kk = 0; kk < EX_BK; kk += 32) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(&as[(wt * 32 + i * 16 + r) * EX_LD + kk + grp * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(&bs[(wc * 32 + j * 16 + r) * EX_LD + kk + grp * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
  }

  // lane holds D[token row0 + wt*32 + i*16 + 4*grp + e][column col0 + wc*32 + j*16 + r]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + wc * 32 + j * 16 + r;
    const int h = col / kKvRows, jj = col % kKvRows;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t tok0 = row0 + wt * 32 + i * 16 + grp * 4;
      if (tok0 >= n_rows) continue;
      const int64_t b = tok0 / seqlen;
      const int64_t t = tok0 - b * seqlen;   // 4 consecutive tokens stay in one sequence when seqlen % 4 == 0
      const int64_t bh = b * n_heads + h;
      if (jj < kNope) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t tk = tok0 + e;
          if (tk >= n_rows) break;
          const int64_t bb = tk / seqlen, tt = tk - bb * seqlen;
          knope[((bb * n_heads + h) * t_pad + tt) * kNope + jj] = f32_to_bf16_bits(acc[i][j][e]);
        }
      } else if (seqlen % 4 == 0) {
        uint2 u;
        u.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        u.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(&vt[(bh * kVDim + (jj - kNope)) * t_pad + t]) = u;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t tk = tok0 + e;
          if (tk >= n_rows) break;
          const int64_t bb = tk / seqlen, tt = tk - bb * seqlen;
          vt[((bb * n_heads + h) * kVDim + (jj - kNope)) * t_pad + tt] = f32_to_bf16_bits(acc[i][j][e]);
        }
      }
    }
  }
}

// Zero V^T columns seqlen .. t_pad-1: they sit inside the last key tile, where P is exactly 0, and
// must hold finite values (0 * NaN would poison the product).
__global__ __launch_bounds__(256) void zero_vt_tail_kernel(uint16_t* __restrict__ vt, int64_t rows, int seqlen,
                                                           int64_t t_pad) {
  const int64_t w = t_pad - seqlen;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * w) return;
  const int64_t row = i / w;
  vt[row * t_pad + seqlen + (i - row * w)] = 0;
}

// ---------------------------------------------------------------------------------------------
// 2. Causal flash attention for one (b, h, 64-query block); 4 waves x 16 queries.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ knope, const uint16_t* __restrict__ vt,
    const uint16_t* __restrict__ k_pe, int n_heads, int seqlen, int64_t t_pad, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_[kKBlk * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vs_[kVDim * kVStride];

  const int n_qb = gridDim.x;
  const int qb = n_qb - 1 - blockIdx.x;          // longest rows first
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int q0 = qb * kQBlk;
  const int tq = q0 + wave * 16 + r;             // this lane's query (B-operand column)
  const int tq_c = min(tq, seqlen - 1);

  bf16x8 qf[6];
  {
    const uint16_t* qp = q + ((b * seqlen + tq_c) * n_heads + h) * kQk + grp * 8;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[ks] = as_bf16x8(ldg16(qp + ks * 32));
  }
  const uint16_t* kn = knope + (b * n_heads + h) * t_pad * kNope;
  const uint16_t* vh = vt + (b * n_heads + h) * kVDim * t_pad;
  const uint16_t* pe = k_pe + b * static_cast<int64_t>(seqlen) * kRope;

  // Per tile: 64 rows x 16 chunks of k_nope, 64 x 8 of k_pe, 128 x 8 of V^T = 2560 chunks.
  constexpr int kChunks = kKBlk * 16 + kKBlk * 8 + kVDim * 8;
  constexpr int CH = kChunks / 256;
  uint4 pf[CH];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = tid + 256 * c;
      if (i < kKBlk * 16) {
        const int row = i >> 4, ch = i & 15;
        const int t = min(k0 + row, seqlen - 1);
        pf[c] = ldg16(kn + static_cast<int64_t>(t) * kNope + ch * 8);
      } else if (i < kKBlk * 24) {
        const int j = i - kKBlk * 16;
        const int row = j >> 3, ch = j & 7;
        const int t = min(k0 + row, seqlen - 1);
        pf[c] = ldg16(pe + static_cast<int64_t>(t) * kRope + ch * 8);
      } else {
        const int j = i - kKBlk * 24;
        const int d = j >> 3, ch = j & 7;
        pf[c] = ldg16(vh + static_cast<int64_t>(d) * t_pad + k0 + ch * 8);   // t_pad covers the tile
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = tid + 256 * c;
      if (i < kKBlk * 16) {
        const int row = i >> 4, ch = i & 15;
        *reinterpret_cast<uint4*>(&ks_[row * kKStride + ch * 8]) = pf[c];
      } else if (i < kKBlk * 24) {
        const int j = i - kKBlk * 16;
        const int row = j >> 3, ch = j & 7;
        *reinterpret_cast<uint4*>(&ks_[row * kKStride + kNope + ch * 8]) = pf[c];
      } else {
        const int j = i - kKBlk * 24;
        const int d = j >> 3, ch = j & 7;
        *reinterpret_cast<uint4*>(&vs_[d * kVStride + ch * 8]) = pf[c];
      }
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_kt = min(qb + 1, (seqlen + kKBlk - 1) / kKBlk);
  fetch(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kt + 1 < n_kt) fetch((kt + 1) * kKBlk);
    const int k0 = kt * kKBlk;

    f32x4 s[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = &ks_[(mb * 16 + r) * kKStride + grp * 8];
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) acc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(arow + ks * 32), qf[ks], acc);
      s[mb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + mb * 16 + grp * 4 + j;
        if (key > tq || key >= seqlen) s[mb][j] = -INFINITY;
        mx = fmaxf(mx, s[mb][j]);
      }
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f((m - m_new) * scale_log2);
    const float mref = m_new * scale_log2;
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[mb * 4 + j] = exp2f(s[mb][j] * scale_log2 - mref);
        ps += p[mb * 4 + j];
      }
    lsum = lsum * alpha + ps;
    m = m_new;
    const bf16x8 pb0 = bf16x8_from_f32(p), pb1 = bf16x8_from_f32(p + 8);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* vrow = &vs_[(db * 16 + r) * kVStride + grp * 4];
      uint4 u0, u1;
      const uint2 a0 = *reinterpret_cast<const uint2*>(vrow);
      const uint2 a1 = *reinterpret_cast<const uint2*>(vrow + 16);
      const uint2 a2 = *reinterpret_cast<const uint2*>(vrow + 32);
      const uint2 a3 = *reinterpret_cast<const uint2*>(vrow + 48);
      u0 = make_uint4(a0.x, a0.y, a1.x, a1.y);
      u1 = make_uint4(a2.x, a2.y, a3.x, a3.y);
      o[db] = o[db] * alpha;
      o[db] = mfma16x16x32(as_bf16x8(u0), pb0, o[db]);
      o[db] = mfma16x16x32(as_bf16x8(u1), pb1, o[db]);
    }
  }

  const float ltot = sum_over_rows(lsum);
  if (tq < seqlen) {
    const float inv = 1.f / ltot;
    uint16_t* dst = out + ((b * seqlen + tq) * n_heads + h) * kVDim + grp * 4;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 u;
      u.x = pack_bf16x2(o[db][0] * inv, o[db][1] * inv);
      u.y = pack_bf16x2(o[db][2] * inv, o[db][3] * inv);
      *reinterpret_cast<uint2*>(dst + db * 16) = u;
    }
    if (lse && grp == 0) lse[(b * n_heads + h) * seqlen + tq] = (m * scale_log2 + __log2f(ltot)) * kLn2;
  }
}

}  // namespace

PrefillLayout prefill_layout(int n_heads, int batch, int seqlen) {
  PrefillLayout L{};
  L.t_pad = (static_cast<int64_t>(seqlen) + kKBlk - 1) / kKBlk * kKBlk;
  const size_t per = static_cast<size_t>(batch) * n_heads * static_cast<size_t>(L.t_pad) * 128 * sizeof(uint16_t);
  L.knope_off = 0;
  L.vt_off = align_up(per);
  L.total = align_up(L.vt_off + per);
  return L;
}

hipError_t launch_prefill(int n_heads, int batch, int seqlen, const uint16_t* q, const uint16_t* kv_latent,
                          const uint16_t* k_pe, const uint16_t* wkv_b, void* workspace,
                          const PrefillLayout& lay, uint16_t* out, float* lse, float scale,
                          hipStream_t stream, hipEvent_t* ev) {
  char* ws = static_cast<char*>(workspace);
  uint16_t* knope = reinterpret_cast<uint16_t*>(ws + lay.knope_off);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + lay.vt_off);
  const int64_t n_rows = static_cast<int64_t>(batch) * seqlen;
  mark(ev, 0, stream);
  if (lay.t_pad != seqlen) {
    const int64_t rows = static_cast<int64_t>(batch) * n_heads * kVDim;
    const int64_t n = rows * (lay.t_pad - seqlen);
    zero_vt_tail_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(vt, rows, seqlen, lay.t_pad);
  }
  const dim3 g1(static_cast<unsigned>((n_rows + EX_BT - 1) / EX_BT), n_heads * kKvRows / EX_BC);
  expand_kernel<<<g1, 256, 0, stream>>>(kv_latent, wkv_b, n_heads, seqlen, lay.t_pad, n_rows, knope, vt);
  mark(ev, 1, stream);
  const dim3 g2(static_cast<unsigned>((seqlen + kQBlk - 1) / kQBlk), n_heads, batch);
  attend_kernel<<<g2, 256, 0, stream>>>(q, knope, vt, k_pe, n_heads, seqlen, lay.t_pad, scale * kLog2e, out, lse);
  mark(ev, 2, stream);
  return hipGetLastError();
}

}  // namespace mla
