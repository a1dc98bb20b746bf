// MLA query path on gfx950: RMSNorm of the query latent -> wq_b up-projection -> RoPE.
//
// Follows "DeepSeek V4.1 · Query RMSNorm" (equation; RMSNorm excerpt: fp32 statistics, learned
// gain, cast back to the input dtype) and "DeepSeek-V3.2-Exp · Query heads" (q^C = c^Q W_UQ,
// q^pe = c^Q W_QR from one matrix wq_b, split per head into 128 content + 64 rotary features,
// Q^R = RoPE(Q^pe, R)).
//
// The GEMM is computed transposed, q^T[n][m] = sum_k wq_b[k][n] y[m][k]: weight columns n are the
// MFMA rows, so every lane ends with four consecutive output columns of one token -- both halves
// of two rotary pairs -- and RoPE runs in registers in the epilogue. wq_b is stored input x
// output (n contiguous), so its tiles are transposed into LDS ([n][k]) on the way in; the
// activation tile is normalised, multiplied by the gain and rounded to bf16 on the way in,
// which keeps the rounding point of the RMSNorm excerpt ahead of the product.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

constexpr int BN = 64;    // weight columns per block
constexpr int BM = 64;    // tokens per block
constexpr int BK = 64;    // reduction slice per LDS stage
constexpr int LDK = BK + 8;

// inv_rms[m] = 1/sqrt(mean_k x[m,k]^2 + eps); one wave per token.
__global__ __launch_bounds__(256) void row_stats_kernel(const uint16_t* __restrict__ x, int64_t n_tokens,
                                                        float eps, float* __restrict__ inv_rms) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= n_tokens) return;
  const uint16_t* row = x + m * kQLora;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kQLora / (64 * 8); ++i) {
    const uint4 v = ldg16(row + (i * 64 + lane) * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf16_bits_to_f32(u4_elem(v, e));
      s += f * f;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) inv_rms[m] = 1.f / sqrtf(s * (1.f / kQLora) + eps);
}

// FUSED: the block computes the statistics of its own BM tokens first (used when the tokens fit
// one block column, i.e. decode); otherwise inv_rms was written by row_stats_kernel.
template <bool FUSED>
__global__ __launch_bounds__(256) void query_gemm_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gamma, const uint16_t* __restrict__ wq_b,
    const float* __restrict__ rope_cs, int64_t n_tokens, int n_cols, float eps,
    float* __restrict__ inv_rms, uint16_t* __restrict__ q_out) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[BN * LDK];   // [n][k]
  __shared__ __attribute__((aligned(16))) uint16_t ys[BM * LDK];   // [m][k]
  __shared__ float rinv[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;

  if (FUSED) {
    // wave w: tokens m0 + w, m0 + w + 4, ...
    for (int mi = wave; mi < BM; mi += 4) {
      if (m0 + mi >= n_tokens) {
        if (lane == 0) rinv[mi] = 0.f;
        continue;
      }
      const int64_t m = m0 + mi;
      const uint16_t* row = x + m * kQLora;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < kQLora / 512; ++i) {
        const uint4 v = ldg16(row + (i * 64 + lane) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = bf16_bits_to_f32(u4_elem(v, e));
          s += f * f;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      const float iv = 1.f / sqrtf(s * (1.f / kQLora) + eps);
      if (lane == 0) {
        rinv[mi] = iv;
        if (inv_rms && blockIdx.x == 0 && m0 + mi < n_tokens) inv_rms[m0 + mi] = iv;
      }
    }
  } else {
    if (tid < BM) rinv[tid] = inv_rms[min(m0 + tid, n_tokens - 1)];
  }

  // Per-thread load assignment: 2 weight chunks (8 n of one k) and 2 activation chunks (8 k of one m).
  uint4 wreg[2], xreg[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int kk = idx >> 3, nch = idx & 7;
      wreg[i] = ldg16(wq_b + static_cast<int64_t>(k0 + kk) * n_cols + n0 + nch * 8);
      const int mm = idx >> 3, kch = idx & 7;
      xreg[i] = ldg16(x + min(m0 + mm, n_tokens - 1) * kQLora + k0 + kch * 8);
    }
  };
  auto stash = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int kk = idx >> 3, nch = idx & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) ws[(nch * 8 + e) * LDK + kk] = u4_elem(wreg[i], e);
      const int mm = idx >> 3, kch = idx & 7;
      const float sc = rinv[mm];
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        y[e] = gamma[k0 + kch * 8 + e] * (bf16_bits_to_f32(u4_elem(xreg[i], e)) * sc);
      *reinterpret_cast<bf16x8*>(&ys[mm * LDK + kch * 8]) = bf16x8_from_f32(y);
    }
  };

  // wave (wn, wm) computes weight columns wn*32 .. +32 x tokens wm*32 .. +32.
  const int wn = wave >> 1, wm = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  __syncthreads();   // rinv visible
  for (int k0 = 0; k0 < kQLora; k0 += BK) {
    __syncthreads();
    stash(k0);
    __syncthreads();
    if (k0 + BK < kQLora) fetch(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&ws[(wn * 32 + i * 16 + r) * LDK + kk + grp * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&ys[(wm * 32 + j * 16 + r) * LDK + kk + grp * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
  }

  // Epilogue: lane holds q[m][n .. n+3], m = m0 + wm*32 + j*16 + r, n = n0 + wn*32 + i*16 + 4*grp.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + wm * 32 + j * 16 + r;
    if (m >= n_tokens) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + wn * 32 + i * 16 + grp * 4;
      const int hd = n % kQk;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = round_bf16(acc[i][j][e]);   // bf16 Linear output
      if (hd >= kNope) {
        const int pair = (hd - kNope) >> 1;
        const float4 cs = *reinterpret_cast<const float4*>(rope_cs + (m * (kRope / 2) + pair) * 2);
        const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
        v[0] = a0 * cs.x - b0 * cs.y;
        v[1] = a0 * cs.y + b0 * cs.x;
        v[2] = a1 * cs.z - b1 * cs.w;
        v[3] = a1 * cs.w + b1 * cs.z;
      }
      uint2 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(q_out + m * n_cols + n) = u;
    }
  }
}

}  // namespace

hipError_t launch_query_path(int n_heads, int64_t n_tokens, const uint16_t* q_latent, const float* gamma,
                             const uint16_t* wq_b, const float* rope_cs, uint16_t* q_out, float* inv_rms,
                             float eps, hipStream_t stream, hipEvent_t* ev) {
  const int n_cols = n_heads * kQk;
  const int64_t m_blocks = (n_tokens + BM - 1) / BM;
  const dim3 grid(n_cols / BN, static_cast<unsigned>(m_blocks));
  mark(ev, 0, stream);
  if (m_blocks == 1 || inv_rms == nullptr) {
    mark(ev, 1, stream);
    query_gemm_kernel<true><<<grid, 256, 0, stream>>>(q_latent, gamma, wq_b, rope_cs, n_tokens, n_cols, eps,
                                                      inv_rms, q_out);
  } else {
    row_stats_kernel<<<static_cast<unsigned>((n_tokens + 3) / 4), 256, 0, stream>>>(q_latent, n_tokens, eps, inv_rms);
    mark(ev, 1, stream);
    query_gemm_kernel<false><<<grid, 256, 0, stream>>>(q_latent, gamma, wq_b, rope_cs, n_tokens, n_cols, eps,
                                                       inv_rms, q_out);
  }
  mark(ev, 2, stream);
  return hipGetLastError();
}

}  // namespace mla
