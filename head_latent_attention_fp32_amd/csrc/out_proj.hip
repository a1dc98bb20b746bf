// Output projection wo on gfx950: y[m, :] = bf16(x[m, :] . wo^T), x the flattened head outputs.
//
// Follows "DeepSeek-V3.2-Exp · Attention update", mla-output excerpt (the head outputs are flattened
// and projected back to the model width, the attention update [B, 1, 7168]) and
// "DeepSeek-V3.2-Exp · Query heads", MLA __init__ (wo maps n_heads * v_head_dim features to dim).
// wo is stored as a Linear stores it, [dim][K = H*128], so both operands are K-contiguous.
//
// Two kernels:
//   small  (n <= 64 tokens, decode): the weight matrix dominates, so it is streamed once, straight
//          into registers (each lane reads 64 contiguous bytes of a weight row per 128-k chunk,
//          two chunks in flight). Block = 64 output columns x one K-slice; its 4 waves take
//          consecutive quarters of the slice with the same columns, and their partial sums meet in
//          LDS. Several K-slices per column tile fill the chip; their fp32 partials are summed in
//          a fixed order by the reduce kernel (deterministic).
//   big    (prefill): the tiled MFMA product of gemm_nt.hpp (256 x 256 output tiles, direct-to-LDS
//          operand stages), split along K when the tiles alone are too few to fill the chip.
// In both, the MFMA A operand is a weight row (output column) and B a token, so a lane ends with
// four consecutive output columns of one token: one 8-byte store.
// The k order inside a 128-k chunk of the small kernel is permuted (lane group g holds k
// 32 g .. 32 g + 31 for its four k-steps) identically for both operands, which leaves the sum
// unchanged and makes each lane's loads contiguous.
#include "gemm_nt.hpp"
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

// ---------------------------------------------------------------------------------------------
// Small token counts.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallCols = 64;     // output columns per block
constexpr int kChunk = 128;        // k per chunk (four MFMA k-steps)

template <int MT>   // 16-token blocks
__global__ __launch_bounds__(256, 1) void out_proj_small_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wo, int n_tokens, int K, int dim,
    int k_per_block, float* __restrict__ part, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) f32x4 red[4][4][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * kSmallCols;
  const int kw = k_per_block / 4;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_per_block + wave * kw + 32 * grp;
  const int n_chunks = kw / kChunk;

  const uint16_t* wp[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) wp[cb] = wo + static_cast<int64_t>(n0 + 16 * cb + r) * K + kbeg;
  const uint16_t* xp[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) xp[mb] = x + static_cast<int64_t>(min(16 * mb + r, n_tokens - 1)) * K + kbeg;

  f32x4 acc[4][MT];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[cb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wf[2][4][4], xf[2][MT][4];
  auto load = [&](int c, int buf) {
    const int64_t o = static_cast<int64_t>(c) * kChunk;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[buf][cb][i] = as_bf16x8(ldg16(wp[cb] + o + 8 * i));
#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[buf][mb][i] = as_bf16x8(ldg16(xp[mb] + o + 8 * i));
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) acc[cb][mb] = mfma16x16x32(wf[buf][cb][i], xf[buf][mb][i], acc[cb][mb]);
  };
  load(0, 0);
  for (int c = 0; c < n_chunks; c += 2) {
    if (c + 1 < n_chunks) load(c + 1, 1);
    compute(0);
    if (c + 1 < n_chunks) {
      if (c + 2 < n_chunks) load(c + 2, 0);
      compute(1);
    }
  }

#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) red[wave][cb][mb][lane] = acc[cb][mb];
  __syncthreads();
  // wave w sums column block w over the four waves; lane holds columns n0 + 16 w + 4 grp .. +3 of
  // token 16 mb + r
  const int n = n0 + 16 * wave + 4 * grp;
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) {
    const int m = 16 * mb + r;
    f32x4 s = red[0][wave][mb][lane];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) s += red[wv][wave][mb][lane];
    if (m >= n_tokens) continue;
    if (gridDim.y == 1) {
      uint2 u;
      u.x = pack_bf16x2(s[0], s[1]);
      u.y = pack_bf16x2(s[2], s[3]);
      *reinterpret_cast<uint2*>(y + static_cast<int64_t>(m) * dim + n) = u;
    } else {
      *reinterpret_cast<float4*>(part + (static_cast<int64_t>(blockIdx.y) * n_tokens + m) * dim + n) =
          make_float4(s[0], s[1], s[2], s[3]);
    }
  }
}

// y = bf16(sum over the K-slices of their partials), four outputs per thread.
__global__ __launch_bounds__(256) void out_proj_reduce_kernel(const float* __restrict__ part, int slices,
                                                              int64_t n_out, uint16_t* __restrict__ y) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n_out) return;
  float4 s = *reinterpret_cast<const float4*>(part + i);
  for (int k = 1; k < slices; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(part + k * n_out + i);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  uint2 u;
  u.x = pack_bf16x2(s.x, s.y);
  u.y = pack_bf16x2(s.z, s.w);
  *reinterpret_cast<uint2*>(y + i) = u;
}

// ---------------------------------------------------------------------------------------------
// Many tokens: the tiled product of gemm_nt.hpp; blockIdx.y = K-slice of k_per_block. With more
// than one slice (gridDim.y > 1) the fp32 partial of the slice goes to part[slice][m][n] for the
// reduce kernel.
// ---------------------------------------------------------------------------------------------
struct OutEpi {
  uint16_t* y;
  float* part;
  int64_t n_tokens;
  int dim, slice, slices;
  __device__ bool transposed(int) const { return false; }
  __device__ void store(int64_t m, int n, f32x4 v, bool) const {
    if (slices > 1) {
      *reinterpret_cast<f32x4*>(part + (static_cast<int64_t>(slice) * n_tokens + m) * dim + n) = v;
      return;
    }
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(y + m * dim + n) = u;
  }
};

__global__ __launch_bounds__(512, 1) void out_proj_big_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wo, int n_tokens, int K,
                                                              int dim, int k_per_block, float* __restrict__ part,
                                                              uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[2 * gemm::kStageBytes];
  const int n_tiles = (dim + gemm::kBN - 1) / gemm::kBN;
  const int nt = blockIdx.x % n_tiles, mt = blockIdx.x / n_tiles;
  const OutEpi epi{y, part, n_tokens, dim, static_cast<int>(blockIdx.y), static_cast<int>(gridDim.y)};
  gemm::nt_tile(wo, dim, x, n_tokens, K, nt * gemm::kBN, static_cast<int64_t>(mt) * gemm::kBM,
                blockIdx.y * k_per_block, k_per_block, stage, epi);
}

// K-slices of the small kernel: enough blocks to give every SIMD about two waves, each wave at
// least one 128-k chunk.
int small_slices(int K, int dim) {
  const int col_tiles = dim / kSmallCols;
  int s = 1;
  while (col_tiles * s * 4 < 2048 && K / (s * 2) >= 4 * kChunk && (K / (s * 2)) % (4 * kChunk) == 0) s *= 2;
  return s;
}

// K-slices of the big kernel: one when the output tiles alone give the chip about one block per
// compute unit; else enough (at most 8) to reach that, each slice at least 16 k-steps.
int big_slices(int K, int dim, int64_t n_tokens) {
  const int64_t tiles = static_cast<int64_t>((dim + gemm::kBN - 1) / gemm::kBN) * ((n_tokens + gemm::kBM - 1) / gemm::kBM);
  int s = 1;
  while (tiles * s < 200 && s < 8 && (K / (2 * s)) % gemm::kBK == 0 && K / (2 * s) >= 16 * gemm::kBK) s *= 2;
  return s;
}

}  // namespace

OutProjLayout out_proj_layout(int n_heads, int64_t n_tokens, int dim) {
  OutProjLayout L{};
  const int K = n_heads * kVDim;
  L.slices = n_tokens <= kOutSmallTokens ? small_slices(K, dim) : big_slices(K, dim, n_tokens);
  L.total = L.slices > 1 ? align_up(static_cast<size_t>(L.slices) * n_tokens * dim * sizeof(float)) : 0;
  return L;
}

hipError_t launch_out_proj(int n_heads, int64_t n_tokens, int dim, const uint16_t* x, const uint16_t* wo,
                           void* workspace, const OutProjLayout& lay, uint16_t* y, hipStream_t stream,
                           hipEvent_t* ev) {
  const int K = n_heads * kVDim;
  mark(ev, 0, stream);
  if (n_tokens <= kOutSmallTokens) {
    const dim3 grid(dim / kSmallCols, lay.slices);
    const int kpb = K / lay.slices;
    float* part = static_cast<float*>(workspace);
    const int n = static_cast<int>(n_tokens);
    if (n <= 16) out_proj_small_kernel<1><<<grid, 256, 0, stream>>>(x, wo, n, K, dim, kpb, part, y);
    else if (n <= 32) out_proj_small_kernel<2><<<grid, 256, 0, stream>>>(x, wo, n, K, dim, kpb, part, y);
    else if (n <= 48) out_proj_small_kernel<3><<<grid, 256, 0, stream>>>(x, wo, n, K, dim, kpb, part, y);
    else out_proj_small_kernel<4><<<grid, 256, 0, stream>>>(x, wo, n, K, dim, kpb, part, y);
    mark(ev, 1, stream);
    if (lay.slices > 1) {
      const int64_t n_out = n_tokens * dim;
      out_proj_reduce_kernel<<<static_cast<unsigned>((n_out / 4 + 255) / 256), 256, 0, stream>>>(part, lay.slices,
                                                                                              n_out, y);
    }
  } else {
    const int64_t tiles =
        static_cast<int64_t>((dim + gemm::kBN - 1) / gemm::kBN) * ((n_tokens + gemm::kBM - 1) / gemm::kBM);
    float* part = static_cast<float*>(workspace);
    out_proj_big_kernel<<<dim3(static_cast<unsigned>(tiles), lay.slices), 512, 0, stream>>>(
        x, wo, static_cast<int>(n_tokens), K, dim, K / lay.slices, part, y);
    mark(ev, 1, stream);
    if (lay.slices > 1) {
      const int64_t n_out = n_tokens * dim;
      out_proj_reduce_kernel<<<static_cast<unsigned>((n_out / 4 + 255) / 256), 256, 0, stream>>>(part, lay.slices,
                                                                                              n_out, y);
    }
  }
  mark(ev, 2, stream);
  return hipGetLastError();
}

}  // namespace mla
