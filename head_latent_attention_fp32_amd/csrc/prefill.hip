// Non-absorbed causal MLA prefill on gfx950.
//
// Follows "Kimi-K2 · value_states", mla-prefill excerpt: the cached latent is expanded through
// kv_b_proj (wkv_b) into per-head k_nope and value states; each head's key joins its k_nope with
// the rotary key shared by every head; scores are scaled, causally masked, softmaxed in fp32 and
// used to mix the values. The queries are the last q_len of kv_len positions (q_len = kv_len: a
// prefill from position 0; q_len < kv_len: new tokens over a cached prefix, the mask then being
// (q_len, kv_seq_len) as in the excerpt): query i, at position kv_len - q_len + i, sees keys
// 0 .. kv_len - q_len + i.
//
// Two kernels:
//   0. vbound   an upper bound of every value a head can produce: max_t max_c |latent[t,c]| times
//               the largest row L1 norm of the head's W_UV, and from it the power of two 2^e_h that
//               brings the bound into [2^14, 2^15): the head's values are divided by it before they
//               are stored as f16, so that they neither overflow nor fall into f16's subnormals.
//   1. expand   [k_nope | v] = latent . wkv_b^T per head for all kv_len positions (MFMA GEMM, bf16
//               outputs as the bf16 Linear of the excerpt; the values, bf16-rounded and divided by
//               2^e_h -- exact, a power of two -- are stored as f16, which holds every such value
//               exactly and lets P be rounded to f16 rather than bf16 for the P.V product; the
//               attention multiplies its output back by 2^e_h). k_nope is written [b][h][t][128] and v
//               transposed in key tiles of 64, [b][h][t/64][128][64], so that the attention kernel's
//               P.V operand reads runs of keys and each tile's V^T is one contiguous 16 KB run;
//               within every 32 keys the order is permuted (key 16a + 4g + j at 8g + 4a + j) to
//               match the key order in which P^T leaves the score accumulators.
//   2. attend   flash-style causal attention: block = (b, h, 128 queries), wave = 32 queries;
//               S^T = K . Q^T and O^T += V^T . P^T on MFMA with an fp32 online softmax; the
//               score matrix never leaves registers.
#include "gemm_nt.hpp"
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

constexpr int kKBlk = 64;     // key padding granule of the expanded k_nope / V^T

// ---------------------------------------------------------------------------------------------
// 1. Expansion: rows = B*S tokens (S = kv_len), columns = H*256 (k_nope then v per head), K = 512,
//    on the tiled product of gemm_nt.hpp: a 256-column tile is one head. Waves on its k_nope half
//    keep the normal orientation (four consecutive features of one token: an 8-byte store into
//    k_nope[b][h][t][:]); waves on its value half take the transposed product (four consecutive
//    tokens of one feature: an 8-byte store into V^T of (b, h, d), whose key order is permuted
//    within groups of 32 but keeps groups of 4 consecutive keys together).
// ---------------------------------------------------------------------------------------------

// Position of key t in its V^T row: within each group of 32, key 16a + 4g + j sits at 8g + 4a + j.
__device__ __forceinline__ int64_t vt_pos(int64_t t) {
  const int64_t w = t & 31;
  return (t - w) + ((w >> 2) & 3) * 8 + (w >> 4) * 4 + (w & 3);
}

// Element offset of V^T entry (dim d, key t) within one (b, h): the keys are kept in tiles of 64
// ([t / 64][128 dims][64 keys], 16 KB per tile), so that the attention kernel's V^T tile is one
// contiguous run; inside a tile the keys are permuted as vt_pos does.
__device__ __forceinline__ int64_t vt_index(int d, int64_t t) {
  return ((t >> 6) * kVDim + d) * 64 + (vt_pos(t) & 63);
}

struct ExpandEpi {
  uint16_t* knope;
  uint16_t* vt;
  int n_heads, seqlen, h;          // h: this tile's head
  int64_t t_pad, n_rows, m0, b0;   // b0 = m0 / seqlen
  float vdiv;                      // 2^-e_h of this tile's head
  __device__ bool transposed(int wn) const { return wn >= 2; }

  // Through LDS, when the tile's 256 tokens are positions t0 .. t0 + 255 of one sequence with t0 a
  // multiple of 64 (every tile when seqlen is a multiple of 256): k_nope staged as [256 tokens]
  // [128 features] bf16 (16-byte chunk c of token row m at c ^ (m & 15), so that the 16 tokens of a
  // lane group write 16 distinct bank groups), the values as [128 features][4 key tiles][64 keys]
  // f16 in the key order of the attention's V^T tiles, rows of 512 bytes at a pitch of 528 (16
  // features then start at 16 distinct bank groups); then both copied out in 16-byte pieces along
  // their destination rows (256 bytes per token of k_nope, one 16 KB V^T tile after another).
  static constexpr bool kStaged = true;
  static constexpr int kKnStage = 256 * kNope * 2;             // 65536
  static constexpr int kVPitch = 64 * 4 * 2 + 16;              // 528
  static constexpr int kLdsBytes = kKnStage + kVDim * kVPitch; // 133120
  __device__ bool can_stage() const {
    const int64_t t0 = m0 - b0 * seqlen;
    return seqlen % 64 == 0 && m0 + 256 <= n_rows && t0 + 256 <= seqlen;
  }
  __device__ void stage_store(uint8_t* lds, int ml, int nl, f32x4 v, bool tr) const {
    if (!tr) {
      const int c = nl >> 3;
      uint2 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(lds + ml * 256 + ((c ^ (ml & 15)) << 4) + 8 * ((nl >> 2) & 1)) = u;
      return;
    }
    const int d = nl - kNope;
    uint2 u;
    u.x = pack_f16x2(round_bf16(v[0]) * vdiv, round_bf16(v[1]) * vdiv);
    u.y = pack_f16x2(round_bf16(v[2]) * vdiv, round_bf16(v[3]) * vdiv);
    *reinterpret_cast<uint2*>(lds + kKnStage + d * kVPitch + (ml >> 6) * 128 + (vt_pos(ml) & 63) * 2) = u;
  }
  __device__ void copy_out(const uint8_t* lds) const {
    const int tid = threadIdx.x;
    const int64_t t0 = m0 - b0 * seqlen;
    uint16_t* kn = knope + ((b0 * n_heads + h) * t_pad + t0) * kNope;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 512 * i, m = q >> 4, c = q & 15;
      *reinterpret_cast<uint4*>(kn + m * kNope + 8 * c) =
          *reinterpret_cast<const uint4*>(lds + m * 256 + ((c ^ (m & 15)) << 4));
    }
    // V^T tiles t0/64 .. t0/64 + 3 of (b0, h): [128 features][64 keys] each, one after another
    uint16_t* v0 = vt + (b0 * n_heads + h) * kVDim * t_pad + (t0 >> 6) * kVDim * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 512 * i, kt = q >> 10, d = (q >> 3) & 127, c = q & 7;
      *reinterpret_cast<uint4*>(v0 + (kt * kVDim + d) * 64 + 8 * c) =
          *reinterpret_cast<const uint4*>(lds + kKnStage + d * kVPitch + kt * 128 + 16 * c);
    }
  }
  // (b, t) of token row m of this tile
  __device__ void locate(int64_t m, int64_t& b, int64_t& t) const {
    b = b0;
    t = m - b0 * seqlen;
    while (t >= seqlen) {
      t -= seqlen;
      ++b;
    }
  }
  __device__ void store(int64_t m, int n, f32x4 v, bool tr) const {
    const int h = n / kKvRows, j = n % kKvRows;
    int64_t b, t;
    locate(m, b, t);
    if (!tr) {
      uint2 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(knope + ((b * n_heads + h) * t_pad + t) * kNope + j) = u;
      return;
    }
    // values: the bf16 Linear output divided by 2^e_h (exact), stored as f16 -- exact below 65504,
    // which the head's bound keeps them under -- for the f16 P.V product
    const int d = j - kNope;
    if ((t & 3) == 0 && t + 3 < seqlen) {   // four consecutive keys of one sequence, aligned
      uint2 u;
      u.x = pack_f16x2(round_bf16(v[0]) * vdiv, round_bf16(v[1]) * vdiv);
      u.y = pack_f16x2(round_bf16(v[2]) * vdiv, round_bf16(v[3]) * vdiv);
      *reinterpret_cast<uint2*>(vt + (b * n_heads + h) * kVDim * t_pad + vt_index(d, t)) = u;
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (m + e >= n_rows) break;
      int64_t bb, tt;
      locate(m + e, bb, tt);
      vt[(bb * n_heads + h) * kVDim * t_pad + vt_index(d, tt)] =
          static_cast<uint16_t>(pack_f16x2(round_bf16(v[e]) * vdiv, 0.f) & 0xFFFFu);
    }
  }
};

// 2^-e as a float, e in [-100, 100].
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float(static_cast<uint32_t>(127 - e) << 23); }

// Block h < n_heads: the largest row L1 norm of W_UV[h] (rows h*256 + 128 .. h*256 + 255 of
// wkv_b). Block n_heads + s: max |latent| over its slot of the latent, the 8-element groups
// s*256 + i + k*(256*kBoundSlots). Every slot and norm is written exactly once (no accumulation
// across blocks).
constexpr int kBoundSlots = 256;
__global__ __launch_bounds__(256) void vbound_kernel(const uint16_t* __restrict__ lat, int64_t n_elems,
                                                     const uint16_t* __restrict__ wkv_b, int n_heads,
                                                     float* __restrict__ bound) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  float m = 0.f;
  if (static_cast<int>(blockIdx.x) < n_heads) {
    // thread = (row 2 * (tid / 4) + {0, 1}, quarter tid % 4 of its 512 columns); the thread's 32
    // loads go out together (the block's 128 KB in flight at once rather than in rounds)
    const int h = blockIdx.x;
    uint4 u[2][16];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 2 * (tid >> 2) + rr;
      const uint16_t* w = wkv_b + (static_cast<int64_t>(h) * kKvRows + kNope + row) * kKvLora + (tid & 3) * 128;
#pragma unroll
      for (int c = 0; c < 16; ++c) u[rr][c] = ldg16(w + 8 * c);
    }
    __builtin_amdgcn_sched_barrier(0);   // (the scheduler would otherwise pair each load with its sums)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint32_t wd[4] = {u[rr][c].x, u[rr][c].y, u[rr][c].z, u[rr][c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) s += fabsf(bf16_bits_to_f32(wd[k] & 0xFFFFu)) + fabsf(bf16_bits_to_f32(wd[k] >> 16));
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);   // the row's sum over its four quarters
      m = fmaxf(m, s);
    }
  } else {
    const int64_t slot = blockIdx.x - n_heads, n_vec = n_elems / 8;   // rows of 512: whole groups
#pragma unroll 4
    for (int64_t i = slot * 256 + tid; i < n_vec; i += 256 * kBoundSlots) {
      const uint4 u = ldg16(lat + i * 8);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(wd[k] & 0xFFFFu)), fabsf(bf16_bits_to_f32(wd[k] >> 16))));
    }
  }
  red[tid] = m;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
    __syncthreads();
  }
  if (tid == 0) bound[blockIdx.x] = red[0];
}

// e_h = the e with b = (max |latent|) * (row L1 norm of W_UV[h]) * (1 + 2^-7) in [2^(14+e), 2^(15+e)):
// the bf16-rounded values of head h, divided by 2^e_h, stay below 2^15 and thus inside fp16's range,
// and values up to 2^29 times smaller than the bound stay above fp16's subnormals (where a bf16 value
// would lose bits). A zero bound, or NaN or infinite inputs, give e_h = 0 (such values propagate as
// they would without the division).
__global__ __launch_bounds__(256) void vscale_kernel(const float* __restrict__ bound, int n_heads,
                                                     int32_t* __restrict__ vexp) {
  __shared__ float lmax_s;
  const int tid = threadIdx.x;
  float m = bound[n_heads + tid];   // kBoundSlots = 256 = blockDim.x
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wred[4];
  if ((tid & 63) == 0) wred[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) lmax_s = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  __syncthreads();
  for (int h = tid; h < n_heads; h += 256) {
    const float b = lmax_s * bound[h] * (1.f + 0.0078125f);
    int e = 0;
    if (b > 0.f && b <= 3.0e38f) {
      e = static_cast<int>((__float_as_uint(b) >> 23) & 0xff) - 127 - 14;   // 2^(e+14) <= b < 2^(e+15)
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
    }
    vexp[h] = e;
  }
}

__global__ __launch_bounds__(512, 1) void expand_kernel(const uint16_t* __restrict__ lat,
                                                        const uint16_t* __restrict__ wkv_b, int n_heads, int seqlen,
                                                        int64_t t_pad, int64_t n_rows, const int32_t* __restrict__ vexp,
                                                        uint16_t* __restrict__ knope, uint16_t* __restrict__ vt) {
  static_assert(ExpandEpi::kLdsBytes >= 2 * gemm::kStageBytes, "the staged epilogue's LDS holds the stages");
  __shared__ __attribute__((aligned(1024))) uint8_t stage[ExpandEpi::kLdsBytes];
  const int h = blockIdx.x % n_heads;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x / n_heads) * gemm::kBM;
  const ExpandEpi epi{knope, vt, n_heads, seqlen, h, t_pad, n_rows, m0, m0 / seqlen, pow2_neg(vexp[h])};
  gemm::nt_tile(wkv_b, static_cast<int64_t>(n_heads) * kKvRows, lat, n_rows, kKvLora, h * kKvRows, m0, 0, kKvLora,
                stage, epi);
}

// Zero the V^T entries of keys seqlen .. t_pad-1: they sit inside the last key tile, where P is
// exactly 0, and must hold finite values (0 * NaN would poison the product).
__global__ __launch_bounds__(256) void zero_vt_tail_kernel(uint16_t* __restrict__ vt, int64_t rows, int seqlen,
                                                           int64_t t_pad) {
  const int64_t w = t_pad - seqlen;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * w) return;
  const int64_t row = i / w;
  vt[(row / kVDim) * kVDim * t_pad + vt_index(static_cast<int>(row % kVDim), seqlen + (i - row * w))] = 0;
}

// ---------------------------------------------------------------------------------------------
// 2. Causal flash attention for one (b, h, 128-query block); 4 waves x 32 queries.
//
//    Keys stream through two LDS stages of 64 keys, filled by 16-byte direct-to-LDS buffer loads
//    (k_nope rows of 256 B, rotary key rows of 128 B, V^T rows of 64 keys); one barrier per tile.
//    Per tile and wave: S^T (64 keys x 32 queries) = K . Q^T, 48 MFMAs with each K operand read
//    once for both 16-query halves; the online softmax in fp32 (log2 units, scale folded in; the
//    accumulators are rescaled only when a query's maximum grows by more than 8); O^T (128 dims x
//    32 queries) += V^T . P^T, 32 MFMAs, with P^T taken from the score accumulators in registers.
//    Operand reads go out six ahead of their MFMAs, and the first value operands while the softmax
//    runs, so that the LDS latency under eight waves' traffic stays behind the matrix pipe.
//    LDS layouts (16-byte chunks): k_nope chunk c of key row r at c ^ 2(r&7); rotary key and V^T
//    rows (128 B) chunk c of row r at c ^ ((r>>1)&7) -- every 128-bit operand read is free of bank
//    conflicts under the two-pass service of a half-wave (lanes 0-7 with 24-31, lanes 8-23).
//    Blocks of one (b, h) share an XCD (blockIdx mod 8), so its K and V^T stay in that L2; within
//    it the longest query blocks go first.
// ---------------------------------------------------------------------------------------------
constexpr int kPQ = 128;                    // queries per block
constexpr int kPK = 64;                     // keys per tile
constexpr int kKnBytes = kPK * kNope * 2;   // 16384
constexpr int kKpBytes = kPK * kRope * 2;   // 8192
constexpr int kVtBytes = kVDim * kPK * 2;   // 16384
constexpr int kStage = kKnBytes + kKpBytes + kVtBytes;   // 40960

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ int swz_kn(int row) { return 2 * (row & 7); }
__device__ __forceinline__ int swz_128(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ knope, const uint16_t* __restrict__ vt,
    const uint16_t* __restrict__ k_pe, int batch, int n_heads, int q_len, int kv_len, int64_t t_pad,
    const int32_t* __restrict__ vexp, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[2][kStage];

  const int n_qb = (q_len + kPQ - 1) / kPQ;
  const int q_pos0 = kv_len - q_len;                     // position of query 0
  const int n_bh = batch * n_heads;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int bh = xcd + 8 * (i / n_qb);
  if (bh >= n_bh) return;
  const int qb = n_qb - 1 - i % n_qb;                    // longest query blocks first
  const int64_t b = bh / n_heads;
  const int h = bh % n_heads;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int q0 = qb * kPQ + wave * 32;                   // this wave's first query (index)
  const int p0 = q_pos0 + q0;                            // and its position

  // Query fragments (B operand): query q0 + 16 qh + r, k-group grp of each of the 6 k-steps.
  bf16x8 qf[2][6];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int tq = min(q0 + 16 * qh + r, q_len - 1);
    const uint16_t* qp = q + ((b * q_len + tq) * n_heads + h) * kQk + grp * 8;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[qh][ks] = as_bf16x8(ldg16(qp + ks * 32));
  }

  const uint16_t* kn = knope + static_cast<int64_t>(bh) * t_pad * kNope;
  const uint16_t* vh = vt + static_cast<int64_t>(bh) * kVDim * t_pad;
  const uint16_t* pe = k_pe + b * static_cast<int64_t>(kv_len) * kRope;
  const uint32_t st_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)&stage[0][0]));

  // Loads of a tile, 10 per wave: k_nope instructions d = wave + 4e (4 keys x 256 B each), rotary
  // d = wave + 4e (8 keys x 128 B), V^T d = wave + 4e (8 dims x 128 B).
  uint32_t kn_off[4], kp_off[2], vt_off[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int d = wave + 4 * e;
    const int key = 4 * d + (lane >> 4);
    kn_off[e] = static_cast<uint32_t>(key * 256 + (((lane & 15) ^ swz_kn(key)) << 4));
    const int dim = 8 * d + (lane >> 3);
    vt_off[e] = static_cast<uint32_t>(dim * 128 + (((lane & 7) ^ swz_128(dim)) << 4));
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int d = wave + 4 * e;
    const int key = 8 * d + (lane >> 3);
    kp_off[e] = static_cast<uint32_t>(key * 128 + (((lane & 7) ^ swz_128(key)) << 4));
  }
  auto issue = [&](int kt) {
    const int k0 = kt * kPK;
    const uint32_t dst = st_lds + (kt & 1) * kStage;
    // each descriptor covers this tile's rows only (a whole tile of the padded k_nope and V^T; the
    // rotary key up to the last position), so that its 32-bit byte range never wraps
    const auto rk = make_rsrc(kn + static_cast<int64_t>(k0) * kNope, static_cast<uint32_t>(kKnBytes));
    const int rows_pe = min(kv_len - k0, kPK);
    const auto rp = make_rsrc(pe + static_cast<int64_t>(k0) * kRope, static_cast<uint32_t>(rows_pe) * 128u);
    const auto rv = make_rsrc(vh + static_cast<int64_t>(k0) * kVDim, static_cast<uint32_t>(kVtBytes));
#pragma unroll
    for (int e = 0; e < 4; ++e) dma16(rk, dst + (wave + 4 * e) * 1024, kn_off[e]);
#pragma unroll
    for (int e = 0; e < 2; ++e) dma16(rp, dst + kKnBytes + (wave + 4 * e) * 1024, kp_off[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) dma16(rv, dst + kKnBytes + kKpBytes + (wave + 4 * e) * 1024, vt_off[e]);
  };

  // Operand offsets within a stage. Scores: key row 16 kb + r, k-step ks < 4: k_nope chunk
  // 4 ks + grp; ks = 4, 5: rotary chunk 4 (ks - 4) + grp. Values: V^T row 16 db + r, chunk 4 ks + grp
  // (keys 4 grp + j and 16 + 4 grp + j of the 32-key group ks, in the permuted order).
  int kn_rd[4], kp_rd[2], v_rd[2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kn_rd[ks] = r * 256 + (((4 * ks + grp) ^ swz_kn(r)) << 4);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    kp_rd[ks] = kKnBytes + r * 128 + (((4 * ks + grp) ^ swz_128(r)) << 4);
    v_rd[ks] = kKnBytes + kKpBytes + r * 128 + (((4 * ks + grp) ^ swz_128(r)) << 4);
  }

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};   // per query (log2 units)
  f32x4 o[2][8];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[qh][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // keys 0 .. position of the block's last query
  const int k_end = min(kv_len, q_pos0 + (qb + 1) * kPQ);
  const int n_kt = (k_end + kPK - 1) / kPK;
  issue(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));   // vmcnt(0): this wave's loads of tile kt
    lds_barrier();                                               // everyone's; stage kt-1 free
    if (kt + 1 < n_kt) issue(kt + 1);
    const uint8_t* st = &stage[kt & 1][0];
    // Matrix phases run at a raised wave priority and the softmax at the base one, so that of the
    // two blocks on a CU the one in its matrix phase keeps the matrix pipe while the other's
    // softmax fills the vector ALU (about 1% on the 4096-token shape).
    __builtin_amdgcn_s_setprio(1);
    const int k0 = kt * kPK;

    f32x4 s[2][4];   // [query half][key block]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[0][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[1][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // operand reads issued six ahead of their MFMAs (the scheduler otherwise places each read two
    // MFMAs before its use, which leaves the LDS latency exposed)
#pragma unroll
    for (int ks = 0; ks < 6; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = ks < 4 ? lds_b128(st + kb * 16 * 256 + kn_rd[ks]) : lds_b128(st + kb * 16 * 128 + kp_rd[ks - 4]);
        s[0][kb] = mfma16x16x32(a, qf[0][ks], s[0][kb]);
        s[1][kb] = mfma16x16x32(a, qf[1][ks], s[1][kb]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
    __builtin_amdgcn_s_setprio(0);
    // causal and length mask on the tiles that reach past this wave's first query position
    if (k0 + kPK - 1 > p0 || k0 + kPK > kv_len) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const int pq = p0 + 16 * qh + r;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + 16 * kb + 4 * grp + j;
            if (key > pq || key >= kv_len) s[qh][kb][j] = -INFINITY;
          }
      }
    }
    // the first value operands, read while the softmax runs
    constexpr int kVPre = 6;
    f16x8 va[16];
#pragma unroll
    for (int i = 0; i < kVPre; ++i) va[i] = *reinterpret_cast<const f16x8*>(st + (i >> 1) * 16 * 128 + v_rd[i & 1]);
    __builtin_amdgcn_sched_group_barrier(0x100, kVPre, 0);
    f16x8 pb[2][2];   // [query half][key group of 32]
    bool any_up = false;
    float alpha[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float mx = fmaxf(fmaxf(fmaxf(s[qh][0][0], s[qh][0][1]), fmaxf(s[qh][0][2], s[qh][0][3])),
                       fmaxf(fmaxf(s[qh][1][0], s[qh][1][1]), fmaxf(s[qh][1][2], s[qh][1][3])));
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[qh][2][0], s[qh][2][1]), fmaxf(s[qh][2][2], s[qh][2][3])),
                           fmaxf(fmaxf(s[qh][3][0], s[qh][3][1]), fmaxf(s[qh][3][2], s[qh][3][3]))));
      mx = max_over_rows(mx) * scale_log2;
      // the reference moves only when the maximum grows by more than 8 (p <= 2^8 otherwise)
      const bool up = mx > m[qh] + 8.f;
      const float m_new = up ? mx : m[qh];
      alpha[qh] = fast_exp2(m[qh] - m_new);   // 1 when the reference stays; 0 from -inf
      any_up |= up;
      m[qh] = m_new;
      float p[16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[kb * 4 + j] = fast_exp2(s[qh][kb][j] * scale_log2 - m_new);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 4) ps += (p[e] + p[e + 1]) + (p[e + 2] + p[e + 3]);
      lsum[qh] = lsum[qh] * alpha[qh] + ps;
      // k-group order of the 32-key groups: keys 4 grp + j (block 2g) then 16 + 4 grp + j (block 2g+1)
      pb[qh][0] = f16x8_from_f32(p);
      pb[qh][1] = f16x8_from_f32(p + 8);
    }
    if (__any(any_up)) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int db = 0; db < 8; ++db) o[qh][db] *= alpha[qh];
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = kVPre; i < 16; ++i) va[i] = *reinterpret_cast<const f16x8*>(st + (i >> 1) * 16 * 128 + v_rd[i & 1]);
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 a = va[2 * db + ks];
        o[0][db] = mfma16x16x32_f16(a, pb[0][ks], o[0][db]);
        o[1][db] = mfma16x16x32_f16(a, pb[1][ks], o[1][db]);
      }
#pragma unroll
    for (int i = 0; i < 16 - kVPre; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kVPre, 0);
  }

#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float ltot = sum_over_rows(lsum[qh]);
    const int tq = q0 + 16 * qh + r;
    if (tq < q_len) {
      // normalised, and multiplied back by the power of two the stored values were divided by
      const float inv = __uint_as_float(static_cast<uint32_t>(127 + vexp[h]) << 23) / ltot;
      uint16_t* dst = out + ((b * q_len + tq) * n_heads + h) * kVDim + grp * 4;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        uint2 u;
        u.x = pack_bf16x2(o[qh][db][0] * inv, o[qh][db][1] * inv);
        u.y = pack_bf16x2(o[qh][db][2] * inv, o[qh][db][3] * inv);
        *reinterpret_cast<uint2*>(dst + db * 16) = u;
      }
      if (lse && grp == 0) lse[(b * n_heads + h) * q_len + tq] = (m[qh] + __log2f(ltot)) * kLn2;
    }
  }
}

}  // namespace

PrefillLayout prefill_layout(int n_heads, int batch, int seqlen) {
  PrefillLayout L{};
  L.t_pad = (static_cast<int64_t>(seqlen) + kKBlk - 1) / kKBlk * kKBlk;
  const size_t per = static_cast<size_t>(batch) * n_heads * static_cast<size_t>(L.t_pad) * 128 * sizeof(uint16_t);
  L.knope_off = 0;
  L.vt_off = align_up(per);
  L.bound_off = align_up(L.vt_off + per);
  L.vexp_off = align_up(L.bound_off + (static_cast<size_t>(n_heads) + kBoundSlots) * sizeof(float));
  L.total = align_up(L.vexp_off + static_cast<size_t>(n_heads) * sizeof(int32_t));
  return L;
}

hipError_t launch_prefill(int n_heads, int batch, int q_len, int kv_len, const uint16_t* q,
                          const uint16_t* kv_latent, const uint16_t* k_pe, const uint16_t* wkv_b, void* workspace,
                          const PrefillLayout& lay, uint16_t* out, float* lse, float scale,
                          hipStream_t stream, hipEvent_t* ev) {
  char* ws = static_cast<char*>(workspace);
  uint16_t* knope = reinterpret_cast<uint16_t*>(ws + lay.knope_off);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + lay.vt_off);
  const int seqlen = kv_len;   // the expansion covers every key position
  const int64_t n_rows = static_cast<int64_t>(batch) * seqlen;
  mark(ev, 0, stream);
  if (lay.t_pad != seqlen) {
    const int64_t rows = static_cast<int64_t>(batch) * n_heads * kVDim;
    const int64_t n = rows * (lay.t_pad - seqlen);
    zero_vt_tail_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(vt, rows, seqlen, lay.t_pad);
  }
  float* bound = reinterpret_cast<float*>(ws + lay.bound_off);
  int32_t* vexp = reinterpret_cast<int32_t*>(ws + lay.vexp_off);
  vbound_kernel<<<n_heads + kBoundSlots, 256, 0, stream>>>(kv_latent, n_rows * kKvLora, wkv_b, n_heads, bound);
  vscale_kernel<<<1, 256, 0, stream>>>(bound, n_heads, vexp);
  const int64_t m_tiles = (n_rows + gemm::kBM - 1) / gemm::kBM;
  expand_kernel<<<static_cast<unsigned>(m_tiles * n_heads), 512, 0, stream>>>(kv_latent, wkv_b, n_heads, seqlen,
                                                                              lay.t_pad, n_rows, vexp, knope, vt);
  mark(ev, 1, stream);
  {
    // blocks of one (b, h) on one XCD: grid = 8 x ceil(B H / 8) x query blocks
    const int64_t n_qb = (q_len + kPQ - 1) / kPQ;
    const int64_t n_bh8 = (static_cast<int64_t>(batch) * n_heads + 7) / 8;
    attend_kernel<<<static_cast<unsigned>(8 * n_bh8 * n_qb), 256, 0, stream>>>(
        q, knope, vt, k_pe, batch, n_heads, q_len, kv_len, lay.t_pad, vexp, scale * kLog2e, out, lse);
  }
  mark(ev, 2, stream);
  return hipGetLastError();
}

}  // namespace mla
