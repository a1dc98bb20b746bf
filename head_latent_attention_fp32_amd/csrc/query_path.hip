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
// output (n contiguous): its tiles go to LDS as stored ([k][n]) and the transposing LDS read
// (ds_read_b64_tr_b16) gives the MFMA operand, eight consecutive k per lane. The activation is
// normalised, multiplied by the gain and rounded to bf16 before the product, which keeps the
// rounding point of the RMSNorm excerpt ahead of it.
#include "gemm_nt.hpp"
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

// ---------------------------------------------------------------------------------------------
// Many tokens: the RMSNorm runs once per token, ahead of the product.
// One wave per token: inv_rms = 1/sqrt(mean x^2 + eps) in fp32, then y = bf16(gain * (x * inv_rms))
// (the rounding point of the RMSNorm excerpt) into the workspace. For the mid-size product
// (kTiled) y is laid out as the LDS image of its activation stages: [24 k-stages of 64][tiles of
// 128 tokens][128 rows][128 B], 16-byte chunk c of row r at c ^ ((r >> 1) & 7), so that a stage of
// a block is one contiguous run, loaded 1 KB per instruction; rows past the last token are written
// as zeros. For the large product y is row-major [n][1536].
// ---------------------------------------------------------------------------------------------
constexpr int kYTile = 128;   // tokens per activation tile

// Activation tiles: an even count, so that a block of 256 tokens never reads past the last one.
__host__ __device__ inline int64_t y_tiles(int64_t n_tokens) { return (n_tokens + 2 * kYTile - 1) / (2 * kYTile) * 2; }

__device__ __forceinline__ int64_t y_chunk_offset(int64_t m, int k, int64_t n_tiles) {
  // element offset of the 8 activations k .. k+7 (k a multiple of 8) of token m
  const int ks = k >> 6, c = (k >> 3) & 7;
  const int r = static_cast<int>(m & (kYTile - 1));
  return (((static_cast<int64_t>(ks) * n_tiles + (m >> 7)) * kYTile + r) * 64) + ((c ^ ((r >> 1) & 7)) << 3);
}

template <bool kTiled>
__global__ __launch_bounds__(256) void normalize_kernel(const uint16_t* __restrict__ x, const float* __restrict__ gamma,
                                                        int64_t n_tokens, int64_t n_tiles, float eps,
                                                        float* __restrict__ inv_rms, uint16_t* __restrict__ y) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= (kTiled ? n_tiles * kYTile : n_tokens)) return;
  auto at = [&](int k) { return kTiled ? y_chunk_offset(m, k, n_tiles) : m * kQLora + k; };
  constexpr int kPer = kQLora / (64 * 8);   // 3 chunks of 8 per lane
  if (m >= n_tokens) {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) *reinterpret_cast<uint4*>(y + at((i * 64 + lane) * 8)) = z;
    return;
  }
  const uint16_t* row = x + m * kQLora;
  bf16x8 v[kPer];
  float4 gl[kPer][2];   // the gain, loaded with the activation rather than after the reduction
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    v[i] = as_bf16x8(ldg16(row + (i * 64 + lane) * 8));
    gl[i][0] = *reinterpret_cast<const float4*>(gamma + (i * 64 + lane) * 8);
    gl[i][1] = *reinterpret_cast<const float4*>(gamma + (i * 64 + lane) * 8 + 4);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = static_cast<float>(v[i][e]);
      s += f * f;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  const float iv = 1.f / sqrtf(s * (1.f / kQLora) + eps);
  if (lane == 0) inv_rms[m] = iv;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int k = (i * 64 + lane) * 8;
    const float4 g0 = gl[i][0], g1 = gl[i][1];
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = g[e] * (static_cast<float>(v[i][e]) * iv);
    *reinterpret_cast<bf16x8*>(y + at(k)) = bf16x8_from_f32(o);
  }
}

// ---------------------------------------------------------------------------------------------
// Small token counts (decode, n <= 32): the weights dominate (1536 x 192 H bf16), so the kernel
// streams them at full width and keeps the activation in registers.
//
// One block of 4 waves per CU works on column slices of 16 NB columns (NB n-blocks of 16): 64
// columns (128 B of each weight row) when the slices outnumber the CUs, persistent over a list of
// them; otherwise 128 columns (256 B per row, which HBM streams faster), one slice per block.
// Wave w owns the k-range [384 w, 384 w + 384) in 12 steps of 32: it holds x for its k-range and
// both 16-token m-blocks in VGPRs (loaded once per block), takes the row statistics from those
// registers (sums of squares exchanged through LDS), and streams the weight rows of its slices
// through a private LDS ring (6 steps of 4 KB, or 4 of 8 KB) with direct-to-LDS loads, without a
// barrier in the k loop. The MFMA A operand (W^T: 16 columns x 8 consecutive k) comes from the ring
// with ds_read_b64_tr_b16, the transposing LDS read; B is y = bf16(gamma x inv_rms) from
// registers. After each slice the four partial sums are added through LDS (the ring itself when a
// block has one slice) and the epilogue rounds the Linear output to bf16, rotates the rotary pairs
// and stores bf16.
// Ring step layout [32 k rows][16 NB columns], so that the 8 rows of a half-wave's transposing read
// (two groups of 4 consecutive rows) fall into distinct 32-byte bank groups:
//   NB = 4: 16-byte chunk c of row k at c ^ 2 gx(k), gx(k) = ((k >> 1) & 1) | (((k >> 3) & 1) << 1);
//   NB = 6: 32-byte group g of row k at g ^ ((k >> 3) & 1) (192-byte rows: four consecutive rows
//           start at four different quarters of the 256-byte bank line, and the flip moves rows
//           8..11 to the other half of each quarter);
//   NB = 8: 32-byte group g of row k at g ^ f(k), f(k) = (k & 3) | ((k >> 1) & 4).
// With 128 heads, 96-column slices make exactly 256 of them: one per CU.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallM = 32;          // largest token count of the small kernel

// NW waves per block, each owning kQLora / NW rows of K (4 waves: 384 rows in 12 steps of 32;
// 8 waves: 192 rows in 6 steps), each with a ring of kRing steps.
template <int NB, int NW>
struct SmallCfg {
  static_assert(NB == 4 || NB == 6 || NB == 8, "slices of 64, 96 or 128 columns");
  static_assert(NW == 4 || (NW == 8 && NB != 4), "8 waves only with one slice per block");
  static constexpr int kWaveK = kQLora / NW;                   // 384 or 192
  static constexpr int kSteps = kWaveK / 32;                   // 12 or 6 k-steps per slice
  static constexpr int kCols = 16 * NB;                        // columns per slice
  static constexpr int kRowBytes = kCols * 2;                  // 128, 192 or 256
  static constexpr int kStepBytes = 32 * kRowBytes;            // 4, 6 or 8 KB
  static constexpr int kLoads = kStepBytes / 1024;             // loads per wave and step
  static constexpr int kRing = NW == 8 ? (NB == 8 ? 2 : 3) : (NB == 8 ? 4 : 6);   // steps in a wave's ring
  static constexpr int kRingBytes = NW * kRing * kStepBytes;   // 96, 144 or 128 KB
  static constexpr int kRedBytes = NW * 2 * NB * 64 * 16;      // NW x 2 NB KB
  static constexpr bool kOneSlice = NB != 4;                   // one slice per block, reduction in the ring
  static constexpr int kLdsBytes = kOneSlice ? kRingBytes : kRingBytes + kRedBytes;
  static_assert(!kOneSlice || kRedBytes <= kRingBytes, "the reduction reuses the ring");
};

// Slice t of XCD x's list: x, x + 8, x + 16, ... For 96-column slices, whose 192-byte row pieces
// share 128-byte lines with their neighbours, pairs of neighbours instead: 2 (x + 8 (t/2)) + t%2,
// so that a line is fetched into one XCD's L2 only.
template <int NB>
__device__ __forceinline__ int slice_of(int x, int t) {
  return NB == 6 ? 2 * (x + 8 * (t >> 1)) + (t & 1) : x + 8 * t;
}
__device__ __forceinline__ int gx(int k) { return ((k >> 1) & 1) | (((k >> 3) & 1) << 1); }
__device__ __forceinline__ int wswz(int k) { return (k & 3) | ((k >> 1) & 4); }

template <int NB, int NW, bool kPacked>
__global__ __launch_bounds__(64 * NW, 1) void query_gemm_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gamma, const uint16_t* __restrict__ wq_b,
    const float* __restrict__ rope_cs, int n_tokens, int n_cols, float eps, float* __restrict__ inv_rms,
    uint16_t* __restrict__ q_out) {
  using C = SmallCfg<NB, NW>;
  constexpr int kWaveK = C::kWaveK, kSteps = C::kSteps;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLdsBytes];
  __shared__ float ss_s[NW][kSmallM];
  float4* red = reinterpret_cast<float4*>(lds + (C::kOneSlice ? 0 : C::kRingBytes));   // [NW][2 NB][64]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int k0 = wave * kWaveK;
  // this block's slices: entries i, i + per, i + 2 per, ... of its XCD's list
  const int xcd = blockIdx.x & 7, i0 = blockIdx.x >> 3, per = gridDim.x >> 3;
  const int list_len = n_cols / C::kCols / 8;
  const int n_mine = i0 < list_len ? (list_len - i0 + per - 1) / per : 0;
  const int total_steps = n_mine * kSteps;

  // Weight rows k0 .. k0 + kWaveK - 1 of the whole matrix through one descriptor (packed: the whole
  // packed matrix); global step g is slice g / kSteps of this block, k-step g % kSteps: kLoads
  // loads of 1 KB.
  const uint16_t* wbase = kPacked ? wq_b : wq_b + static_cast<int64_t>(k0) * n_cols;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wbase, static_cast<uint32_t>(kPacked ? kQLora : kWaveK) * static_cast<uint32_t>(n_cols) * 2u);
  uint8_t* ring = lds + wave * C::kRing * C::kStepBytes;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)ring));
  uint32_t w_voff[C::kLoads];
#pragma unroll
  for (int d = 0; d < C::kLoads; ++d) {
    // step row and logical 16-byte chunk (of the slice's row) that this lane's 16 bytes fill
    int row, lc;
    if constexpr (NB == 4) {
      row = 8 * d + (lane >> 3);
      lc = (lane & 7) ^ (2 * gx(row));
    } else if constexpr (NB == 6) {
      // LDS bytes 1024 d + 16 lane of the step: row P / 192, physical 16-byte chunk (P % 192) / 16
      const int pos = 1024 * d + 16 * lane;
      row = pos / 192;
      const int pc = (pos % 192) >> 4;
      lc = (((pc >> 1) ^ ((row >> 3) & 1)) << 1) | (pc & 1);
    } else {
      row = 4 * d + (lane >> 4);
      const int pc = lane & 15;
      lc = (((pc >> 1) ^ wswz(row)) << 1) | (pc & 1);
    }
    w_voff[d] = kPacked ? gemm::packed_lane_off(kQLora, row, lc) : static_cast<uint32_t>(row * n_cols * 2 + lc * 16);
  }
  auto issue = [&](int g) {
    const int sl = slice_of<NB>(xcd, i0 + per * (g / kSteps));
    const uint32_t off =
        kPacked ? static_cast<uint32_t>(sl * (C::kCols / gemm::kPackCols)) * (kQLora * gemm::kPackCols * 2u) +
                      static_cast<uint32_t>(k0 + (g % kSteps) * 32) * (gemm::kPackCols * 2u)
                : static_cast<uint32_t>(g % kSteps) * 32u * n_cols * 2u + sl * C::kRowBytes;
    const uint32_t dst = ring_lds + (g % C::kRing) * C::kStepBytes;
#pragma unroll
    for (int d = 0; d < C::kLoads; ++d) dma16(rw, dst + d * 1024, w_voff[d] + off);
  };
  // Activation of tokens 16 mb + r (clamped to the last token), k-group grp of each step. Its loads
  // go out ahead of the weight ring (they are waited for first).
  bf16x8 xf[2][kSteps];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = min(16 * mb + r, n_tokens - 1);
    const uint16_t* row = x + static_cast<int64_t>(m) * kQLora + k0 + grp * 8;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) xf[mb][st] = as_bf16x8(ldg16(row + st * 32));
  }
  // With 8 waves (6 k-steps each, registers to spare) the gain goes out with the activation instead
  // of after the row statistics
  constexpr int kGainAhead = NW == 8 ? kSteps : 1;
  float4 gl[kGainAhead][2];
  if constexpr (NW == 8) {
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      gl[st][0] = *reinterpret_cast<const float4*>(gamma + k0 + st * 32 + grp * 8);
      gl[st][1] = *reinterpret_cast<const float4*>(gamma + k0 + st * 32 + grp * 8 + 4);
    }
  }
  int issued = 0;
  while (issued < C::kRing && issued < total_steps) issue(issued++);
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = static_cast<float>(xf[mb][st][e]);
        ss[mb] += f * f;
      }
    }
    ss[mb] = sum_over_rows(ss[mb]);
  }
  if (grp == 0) {
    ss_s[wave][r] = ss[0];
    ss_s[wave][16 + r] = ss[1];
  }
  __syncthreads();
  float inv[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int mm = 16 * mb + r;
    float t = (ss_s[0][mm] + ss_s[1][mm]) + (ss_s[2][mm] + ss_s[3][mm]);
    if constexpr (NW == 8) t += (ss_s[4][mm] + ss_s[5][mm]) + (ss_s[6][mm] + ss_s[7][mm]);
    inv[mb] = 1.f / sqrtf(t * (1.f / kQLora) + eps);
    if (inv_rms && blockIdx.x == 0 && wave == 0 && grp == 0 && mm < n_tokens) inv_rms[mm] = inv[mb];
  }
  // y = bf16(gamma * (x * inv_rms)), in place
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const float4 g0 = NW == 8 ? gl[st % kGainAhead][0] : *reinterpret_cast<const float4*>(gamma + k0 + st * 32 + grp * 8);
    const float4 g1 =
        NW == 8 ? gl[st % kGainAhead][1] : *reinterpret_cast<const float4*>(gamma + k0 + st * 32 + grp * 8 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = g[e] * (static_cast<float>(xf[mb][st][e]) * inv[mb]);
      xf[mb][st] = bf16x8_from_f32(y);
    }
  }

  // A operand of n-block nb, k rows 8 grp + 4 h .. +3 of a step: source lane j of a 16-lane group
  // reads row 8 grp + 4 h + j/4 at columns 16 nb + 4 (j%4) .. +3.
  int a_off[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * grp + 4 * h + (r >> 2);
      if constexpr (NB == 4) {
        const int c = 2 * nb + ((r & 3) >> 1);
        a_off[nb][h] = row * 128 + ((c ^ (2 * gx(row))) << 4) + 8 * (r & 1);
      } else if constexpr (NB == 6) {
        a_off[nb][h] = row * 192 + ((nb ^ ((row >> 3) & 1)) << 5) + 8 * (r & 3);
      } else {
        a_off[nb][h] = row * 256 + ((nb ^ wswz(row)) << 5) + 8 * (r & 3);
      }
    }

  for (int j = 0; j < n_mine; ++j) {
    f32x4 acc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int g = j * kSteps + st;
      // loads of up to kRing - 1 later steps may stay in flight
      const int after = issued - 1 - g;
      constexpr int L = C::kLoads;
      if (C::kRing == 6 && after >= 5) wait_vm<5 * L>();
      else if (C::kRing == 6 && after == 4) wait_vm<4 * L>();
      else if (after >= 3) wait_vm<3 * L>();
      else if (after == 2) wait_vm<2 * L>();
      else if (after == 1) wait_vm<L>();
      else wait_vm<0>();
      const uint8_t* base = ring + (g % C::kRing) * C::kStepBytes;
      bf16x8 af[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + a_off[nb][0]));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(base + a_off[nb][1]));
        af[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      if (issued < total_steps) {
        // the stage is refilled only after this wave's reads of it have completed
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
        issue(issued++);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma16x16x32(af[nb], xf[mb][st], acc[nb][mb]);
    }

    // Sum of the NW waves' partials (in wave order): wave w finalises the (n-block, m-block) pairs
    // p = nb 2 + mb with p = w (mod NW).
    if (C::kOneSlice) __syncthreads();   // every wave's ring reads are done before it is overwritten
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const f32x4 v = acc[nb][mb];
        red[(wave * 2 * NB + nb * 2 + mb) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
    __syncthreads();
    constexpr int kOwn = (2 * NB + NW - 1) / NW;   // pairs finalised per wave, at most
    float vv[kOwn][4];
#pragma unroll
    for (int o = 0; o < kOwn; ++o) {
      const int pr = wave + NW * o;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[o][e] = 0.f;
      if (pr < 2 * NB) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float4 u = red[(w * 2 * NB + pr) * 64 + lane];
          vv[o][0] += u.x;
          vv[o][1] += u.y;
          vv[o][2] += u.z;
          vv[o][3] += u.w;
        }
      }
    }
    if (!C::kOneSlice) __syncthreads();   // red is rewritten for the next slice
#pragma unroll
    for (int o = 0; o < kOwn; ++o) {
      {   // lane holds q[m][n .. n+3], m = 16 mb + r, n = slice start + 16 nb + 4 grp
        const int pr = wave + NW * o, nb = pr >> 1, mb = pr & 1;
        float* v = vv[o];
        const int m = 16 * mb + r;
        if (pr < 2 * NB && m < n_tokens) {
          const int n = slice_of<NB>(xcd, i0 + per * j) * C::kCols + 16 * nb + 4 * grp;
          const int hd = n % kQk;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = round_bf16(v[e]);   // bf16 Linear output
          if (hd >= kNope) {
            const int pair = (hd - kNope) >> 1;
            const float4 cs =
                *reinterpret_cast<const float4*>(rope_cs + (static_cast<int64_t>(m) * (kRope / 2) + pair) * 2);
            const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
            v[0] = a0 * cs.x - b0 * cs.y;
            v[1] = a0 * cs.y + b0 * cs.x;
            v[2] = a1 * cs.z - b1 * cs.w;
            v[3] = a1 * cs.w + b1 * cs.z;
          }
          uint2 u;
          u.x = pack_bf16x2(v[0], v[1]);
          u.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(q_out + static_cast<int64_t>(m) * n_cols + n) = u;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Mid-size token counts (33 .. 1023): large-tile MFMA GEMM on the normalised activation y
// (normalize_kernel), q^T = W^T . y^T per block tile of BN output columns x BM tokens (BN = 96 at
// 128 heads: 256 column tiles, one per CU; else 128), 4 waves as 2 x 2, each wave
// (BN/2) x (BM/2). The W operand (the transposing read, half the LDS rate of a plain read) is reused
// across the wave's BM/32 token blocks. K advances 64 at a time through three LDS stages (two in flight), filled
// by direct-to-LDS loads, so the main loop holds no conversion work:
//   W stage [64 k][BN] bf16: 32-byte column group g of row k at g ^ f(k), f(k) = (k & 3) |
//     ((k >> 1) & 4) (BN = 96: (k >> 3) & 1), so the 8 rows of a half-wave's transposing read
//     (ds_read_b64_tr_b16: 16 columns x 8 consecutive k, the A operand) hit 8 distinct 32-byte bank
//     groups;
//   Y stage [BM tokens][64 k] bf16: 16-byte chunk c of row m at c ^ ((m >> 1) & 7).
// The epilogue rounds the Linear output to bf16 and rotates the rotary pairs in registers.
// ---------------------------------------------------------------------------------------------
constexpr int kBigStages = 3;   // LDS stages of 64 k; two in flight ahead of the one in use

// W stage swizzle: 32-byte group g of row k at g ^ big_swz(k); 96-column (192-byte) rows flip
// rows 8..15 of every 16 (the same reasoning as the small kernel's 96-column slices)
template <int BN>
__device__ __forceinline__ int big_swz(int k) { return BN == 96 ? (k >> 3) & 1 : wswz(k); }

template <int BN, int BM>
struct BigTile {
  static constexpr int kWN = BN / 2 / 16;            // n-blocks per wave
  static constexpr int kWM = BM / 2 / 16;            // m-blocks per wave
  static constexpr int kWBytes = 64 * BN * 2;        // W stage
  static constexpr int kYBytes = BM * 64 * 2;        // Y stage
  static constexpr int kWLoads = kWBytes / 1024 / 4; // direct-to-LDS loads per wave per stage
  static constexpr int kYLoads = kYBytes / 1024 / 4;
};

template <int BN, int BM, bool kPacked>
__global__ __launch_bounds__(256, 1) void query_gemm_big_kernel(
    const uint16_t* __restrict__ y, const uint16_t* __restrict__ wq_b, const float* __restrict__ rope_cs,
    int64_t n_tokens, int n_cols, uint16_t* __restrict__ q_out) {
  using T = BigTile<BN, BM>;
  __shared__ __attribute__((aligned(1024))) uint8_t wst[kBigStages][T::kWBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t yst[kBigStages][T::kYBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int wn = wave >> 1, wm = wave & 1;
  // 96-column tiles (exactly 256 at 128 heads): neighbours, whose 192-byte row pieces share
  // 128-byte lines, paired on one XCD as in the small kernel
  const int nt = BN == 96 ? 2 * ((blockIdx.x & 7) + 8 * (blockIdx.x >> 4)) + ((blockIdx.x >> 3) & 1) : blockIdx.x;
  const int n0 = nt * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;

  // W loads: stage rows k0 .. k0+63, columns n0 .. n0+BN-1 of wq_b (row pitch n_cols); load li
  // covers 1 KB = 1024 / (2 BN) rows; lane l -> row, physical 16-byte chunk.
  uint32_t w_voff[T::kWLoads];
#pragma unroll
  for (int e = 0; e < T::kWLoads; ++e) {
    const int li = wave + 4 * e;
    // byte 1024 li + 16 lane of the stage: row and physical 16-byte chunk
    const int pos = 1024 * li + 16 * lane;
    const int row = pos / (BN * 2), pc = (pos % (BN * 2)) >> 4;
    const int lc = (((pc >> 1) ^ big_swz<BN>(row)) << 1) | (pc & 1);
    w_voff[e] = kPacked ? gemm::packed_lane_off(kQLora, row, lc) : static_cast<uint32_t>(row * n_cols * 2 + lc * 16);
  }
  // Y loads: the block's BM tokens of a stage are BM / 128 consecutive tiles of the workspace
  // (already in LDS order): contiguous 1 KB loads.
  const int64_t n_tiles = y_tiles(n_tokens);
  const uint16_t* y_blk = y + (m0 / kYTile) * kYTile * 64;   // stage 0 of this block's first tile
  const uint32_t y_stage_pitch = static_cast<uint32_t>(n_tiles * kYTile * 128);   // bytes per k-stage
  const uint32_t y_bytes = y_stage_pitch * (kQLora / 64) - static_cast<uint32_t>(m0 / kYTile) * kYTile * 128;
  const uint32_t w_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)&wst[0][0]));
  const uint32_t y_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)&yst[0][0]));
  auto issue = [&](int kt) {
    // descriptors rebuilt per stage (scalar work): kept short-lived, they stay in SGPRs
    // (packed: the tile's BN / 32 column groups)
    const __amdgpu_buffer_rsrc_t rw =
        kPacked ? make_rsrc(wq_b + static_cast<int64_t>(n0) * kQLora, static_cast<uint32_t>(kQLora) * BN * 2u)
                : make_rsrc(wq_b + n0, static_cast<uint32_t>(kQLora) * n_cols * 2u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y_blk, y_bytes);
    const uint32_t wk = static_cast<uint32_t>(kt) * 64u * (kPacked ? gemm::kPackCols * 2u : n_cols * 2u);
    const uint32_t yk = static_cast<uint32_t>(kt) * y_stage_pitch;
#pragma unroll
    for (int e = 0; e < T::kWLoads; ++e)
      dma16(rw, w_lds + (kt % kBigStages) * T::kWBytes + (wave + 4 * e) * 1024, w_voff[e] + wk);
#pragma unroll
    for (int e = 0; e < T::kYLoads; ++e)
      dma16(ry, y_lds + (kt % kBigStages) * T::kYBytes + (wave + 4 * e) * 1024, yk + (wave + 4 * e) * 1024 + lane * 16);
  };

  // Operand offsets. A (W^T, n-block nb of the wave, k rows 8 grp + 4 h .. +3 of k-step ks):
  // source lane j of a 16-lane group reads row 32 ks + 8 grp + 4 h + j/4 at columns
  // 16 (wn kWN + nb) + 4 (j%4) .. +3. B (y, m-block mb): row 16 (wm kWM + mb) + r, chunk 4 ks + grp.
  int b_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int row = wm * (BM / 2) + r;                  // + 16 mb leaves (row >> 1) & 7 unchanged
    b_off[ks] = row * 128 + (((4 * ks + grp) ^ ((row >> 1) & 7)) << 4);
  }

  f32x4 acc[T::kWN][T::kWM];
#pragma unroll
  for (int i = 0; i < T::kWN; ++i)
#pragma unroll
    for (int j = 0; j < T::kWM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int n_kt = kQLora / 64;   // 24
  constexpr int kLoads = T::kWLoads + T::kYLoads;
  issue(0);
  issue(1);
  for (int kt = 0; kt < n_kt; ++kt) {
    // this wave's loads of stage kt (those of kt+1 may stay in flight)
    if (kt + 1 < n_kt) wait_vm<kLoads>();
    else wait_vm<0>();
    __syncthreads();         // everyone's; the stage of kt-1 is free
    if (kt + 2 < n_kt) issue(kt + 2);
    const uint8_t* wb = &wst[kt % kBigStages][0];
    const uint8_t* yb = &yst[kt % kBigStages][0];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[T::kWN], bfm[T::kWM];
#pragma unroll
      for (int nb = 0; nb < T::kWN; ++nb) {
        const int g = wn * T::kWN + nb;                   // 32-byte column group
        i16x4 half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * ks + 8 * grp + 4 * h + (r >> 2);
          const int byte = row * (BN * 2) + ((g ^ big_swz<BN>(row)) << 5) + 8 * (r & 3);
          half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(wb + byte));
        }
        af[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mb = 0; mb < T::kWM; ++mb) bfm[mb] = *reinterpret_cast<const bf16x8*>(yb + b_off[ks] + mb * 16 * 128);
#pragma unroll
      for (int nb = 0; nb < T::kWN; ++nb)
#pragma unroll
        for (int mb = 0; mb < T::kWM; ++mb) acc[nb][mb] = mfma16x16x32(af[nb], bfm[mb], acc[nb][mb]);
    }
  }

  // lane holds q[m][n .. n+3], m = m0 + wm BM/2 + 16 mb + r, n = n0 + wn BN/2 + 16 nb + 4 grp
#pragma unroll
  for (int mb = 0; mb < T::kWM; ++mb) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * mb + r;
    if (m >= n_tokens) continue;
#pragma unroll
    for (int nb = 0; nb < T::kWN; ++nb) {
      const int n = n0 + wn * (BN / 2) + 16 * nb + 4 * grp;
      const int hd = n % kQk;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = round_bf16(acc[nb][mb][e]);   // bf16 Linear output
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

// ---------------------------------------------------------------------------------------------
// Large token counts (prefill, >= kNtTokens): the tiled product of gemm_nt.hpp (256 x 256 tiles)
// on the row-major y and on wq_b as it is stored, its weight stages [64 k][256 n] read with the
// transposing LDS read. The epilogue is the one above: bf16 rounding of the Linear output, RoPE of
// the rotary pairs in registers, one 8-byte store per lane.
// ---------------------------------------------------------------------------------------------
constexpr int64_t kNtTokens = 1024;

struct QueryEpi {
  const float* rope_cs;
  uint16_t* q_out;
  int n_cols;
  int64_t n_tokens, m0;
  int n0;
  __device__ bool transposed(int) const { return false; }
  // Final values of q[m][n .. n+3]: the bf16 Linear output, rotary pairs rotated, packed.
  __device__ uint2 finish(int64_t m, int n, f32x4 acc) const {
    const int hd = n % kQk;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = round_bf16(acc[e]);   // bf16 Linear output
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
    return u;
  }
  // A whole 256 x 256 tile goes out through LDS: [256 tokens][256 features] bf16 (the two 64 KB
  // stages), 16-byte chunk c of token row m at c ^ (m & 15), so that the 16 tokens of a lane group
  // write 16 distinct bank groups; then each token's 512 bytes are copied out in 16-byte pieces.
  static constexpr bool kStaged = true;
  __device__ bool can_stage() const { return m0 + 256 <= n_tokens; }
  __device__ void stage_store(uint8_t* lds, int ml, int nl, f32x4 acc, bool) const {
    const int c = nl >> 3;
    *reinterpret_cast<uint2*>(lds + ml * 512 + ((c ^ (ml & 15)) << 4) + 8 * ((nl >> 2) & 1)) =
        finish(m0 + ml, n0 + nl, acc);
  }
  __device__ void copy_out(const uint8_t* lds) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = tid + 512 * i, m = q >> 5, c = q & 31;
      *reinterpret_cast<uint4*>(q_out + (m0 + m) * n_cols + n0 + 8 * c) =
          *reinterpret_cast<const uint4*>(lds + m * 512 + ((c ^ (m & 15)) << 4));
    }
  }
  __device__ void store(int64_t m, int n, f32x4 acc, bool) const {
    *reinterpret_cast<uint2*>(q_out + m * n_cols + n) = finish(m, n, acc);
  }
};

// wq_b read as it is stored (input x output), or packed in 32-column groups: the product's weight
// operand through the transposing LDS read (n_cols is a multiple of 256 for every supported head
// count).
template <bool kPacked>
__global__ __launch_bounds__(512, 1) void query_gemm_nt_kernel(const uint16_t* __restrict__ wq_b,
                                                               const uint16_t* __restrict__ y,
                                                               const float* __restrict__ rope_cs, int64_t n_tokens,
                                                               int n_cols, uint16_t* __restrict__ q_out) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[2 * gemm::kStageBytes];
  const int n_tiles = n_cols / gemm::kBN;
  const int nt = blockIdx.x % n_tiles;
  const int64_t mt = blockIdx.x / n_tiles;
  const QueryEpi epi{rope_cs, q_out, n_cols, n_tokens, mt * gemm::kBM, nt * gemm::kBN};
  gemm::nt_tile<true, kPacked>(wq_b, n_cols, y, n_tokens, kQLora, nt * gemm::kBN, mt * gemm::kBM, 0, kQLora, stage,
                               epi, n_cols);
}

// ---------------------------------------------------------------------------------------------
// Packed weights: wq_b [1536][n_cols] (input x output) -> [n_cols / 32][1536][32], each group of 32
// output columns with its 1536 rows of 64 bytes back to back. A column slice of the products above
// (64, 96, 128 or 256 columns, always whole groups) then streams as a few contiguous runs of 96 KB
// instead of 1536 pieces of 128-512 bytes spread over the 48 KB rows of the stored matrix, while
// the LDS images, and so every product and its rounding, stay the same. One thread moves 16 bytes;
// consecutive threads read consecutive pieces of a stored row.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_wq_b_kernel(const uint16_t* __restrict__ wq_b, int n_cols,
                                                        uint16_t* __restrict__ packed) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int pieces_per_row = n_cols / 8;
  if (t >= static_cast<int64_t>(kQLora) * pieces_per_row) return;
  const int k = static_cast<int>(t / pieces_per_row), c = static_cast<int>(t % pieces_per_row);
  const uint4 v = ldg16(wq_b + static_cast<int64_t>(k) * n_cols + 8 * c);
  *reinterpret_cast<uint4*>(packed + (static_cast<int64_t>(c >> 2) * kQLora + k) * gemm::kPackCols + 8 * (c & 3)) = v;
}

}  // namespace

hipError_t launch_pack_wq_b(int n_heads, const uint16_t* wq_b, uint16_t* packed, hipStream_t stream) {
  const int n_cols = n_heads * kQk;
  const int64_t pieces = static_cast<int64_t>(kQLora) * (n_cols / 8);
  pack_wq_b_kernel<<<static_cast<unsigned>((pieces + 255) / 256), 256, 0, stream>>>(wq_b, n_cols, packed);
  return hipGetLastError();
}

QueryLayout query_layout(int n_heads, int64_t n_tokens) {
  QueryLayout L{};
  if (n_tokens <= kSmallM) return L;
  if (n_tokens >= kNtTokens) {
    L.large = true;
    L.y_off = 0;
    L.inv_off = align_up(static_cast<size_t>(n_tokens) * kQLora * sizeof(uint16_t));
  } else {
    const int64_t n_pad = y_tiles(n_tokens) * kYTile;
    L.y_off = 0;
    L.inv_off = align_up(static_cast<size_t>(n_pad) * kQLora * sizeof(uint16_t));
  }
  L.total = align_up(L.inv_off + static_cast<size_t>(n_tokens) * sizeof(float));
  return L;
}

template <bool kPacked>
static void launch_query_kernels(int n_heads, int64_t n_tokens, const uint16_t* q_latent, const float* gamma,
                                 const uint16_t* wq_b, const float* rope_cs, uint16_t* q_out, float* inv_rms,
                                 void* workspace, const QueryLayout& lay, float eps, hipStream_t stream,
                                 hipEvent_t* ev) {
  const int n_cols = n_heads * kQk;
  mark(ev, 0, stream);
  if (n_tokens <= kSmallM) {
    // one block per CU (at most one per slice); slice counts are multiples of 8, so every XCD has
    // blocks. Slices of 96 columns when they make exactly one per CU (128 heads), else 128 columns
    // when they do not outnumber the CUs and fill at least half of them (one per block), else 64.
    mark(ev, 1, stream);
    if (n_cols == 256 * SmallCfg<6, 8>::kCols) {
      query_gemm_small_kernel<6, 8, kPacked><<<256, 512, 0, stream>>>(q_latent, gamma, wq_b, rope_cs,
                                                                      static_cast<int>(n_tokens), n_cols, eps,
                                                                      inv_rms, q_out);
    } else if (n_cols / SmallCfg<8, 4>::kCols <= 256 && n_cols / SmallCfg<8, 4>::kCols >= 128) {
      query_gemm_small_kernel<8, 4, kPacked><<<n_cols / SmallCfg<8, 4>::kCols, 256, 0, stream>>>(
          q_latent, gamma, wq_b, rope_cs, static_cast<int>(n_tokens), n_cols, eps, inv_rms, q_out);
    } else {
      const int n_slices = n_cols / SmallCfg<4, 4>::kCols;
      const int grid = n_slices < 256 ? n_slices : 256;
      query_gemm_small_kernel<4, 4, kPacked><<<grid, 256, 0, stream>>>(q_latent, gamma, wq_b, rope_cs,
                                                                       static_cast<int>(n_tokens), n_cols, eps,
                                                                       inv_rms, q_out);
    }
  } else {
    char* ws = static_cast<char*>(workspace);
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + lay.y_off);
    float* inv = inv_rms ? inv_rms : reinterpret_cast<float*>(ws + lay.inv_off);
    if (lay.large) {
      normalize_kernel<false><<<static_cast<unsigned>((n_tokens + 3) / 4), 256, 0, stream>>>(q_latent, gamma, n_tokens,
                                                                                            0, eps, inv, y);
      mark(ev, 1, stream);
      const int64_t blocks = static_cast<int64_t>(n_cols / gemm::kBN) * ((n_tokens + gemm::kBM - 1) / gemm::kBM);
      query_gemm_nt_kernel<kPacked><<<static_cast<unsigned>(blocks), 512, 0, stream>>>(wq_b, y, rope_cs, n_tokens,
                                                                                        n_cols, q_out);
    } else {
      const int64_t n_tiles = y_tiles(n_tokens);
      normalize_kernel<true><<<static_cast<unsigned>(n_tiles * kYTile / 4), 256, 0, stream>>>(q_latent, gamma, n_tokens,
                                                                                             n_tiles, eps, inv, y);
      mark(ev, 1, stream);
      // 96-column tiles when they make exactly 256 (128 heads), else 128
      if (n_cols == 256 * 96) {
        const dim3 grid(256, static_cast<unsigned>((n_tokens + 127) / 128));
        query_gemm_big_kernel<96, 128, kPacked><<<grid, 256, 0, stream>>>(y, wq_b, rope_cs, n_tokens, n_cols, q_out);
      } else {
        const dim3 grid(n_cols / 128, static_cast<unsigned>((n_tokens + 127) / 128));
        query_gemm_big_kernel<128, 128, kPacked><<<grid, 256, 0, stream>>>(y, wq_b, rope_cs, n_tokens, n_cols, q_out);
      }
    }
  }
  mark(ev, 2, stream);
}

hipError_t launch_query_path(int n_heads, int64_t n_tokens, const uint16_t* q_latent, const float* gamma,
                             const uint16_t* wq_b, bool packed, const float* rope_cs, uint16_t* q_out,
                             float* inv_rms, void* workspace, const QueryLayout& lay, float eps, hipStream_t stream,
                             hipEvent_t* ev) {
  if (packed)
    launch_query_kernels<true>(n_heads, n_tokens, q_latent, gamma, wq_b, rope_cs, q_out, inv_rms, workspace, lay, eps,
                               stream, ev);
  else
    launch_query_kernels<false>(n_heads, n_tokens, q_latent, gamma, wq_b, rope_cs, q_out, inv_rms, workspace, lay,
                                eps, stream, ev);
  return hipGetLastError();
}

}  // namespace mla
