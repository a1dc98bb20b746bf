// Absorbed MLA decode on gfx950: one new query token per sequence, dense over its cached latent.
//
// Follows "DeepSeek-V3.2-Exp · Attention update", mla-decode (MQA decode) excerpt: the query's
// content part is absorbed through the key half of wkv_b, scores are the 512-wide latent dot plus
// the 64-wide rotary dot times the softmax scale, the softmax-weighted sum of cached latents is
// projected out through the value half of wkv_b ("Kimi-K2 · value_states": [B,1,512] -> [B,H,1,128]).
//
// Three kernels, enqueued back to back on the caller's stream:
//   1. absorb_plan   q_lat = bf16(q_nope . W_UK) per head (MFMA), and (block 0) the run plan:
//                    prefix sums of the clamped lengths and the number of runs.
//   2. attend        split-KV attention: the tokens of all sequences, back to back, are cut into
//                    equal runs; a workgroup streams its run's kv/pe rows through LDS 32 at a
//                    time, computes S^T = [kv|pe] . [q_lat|q_pe]^T and O^T += kv^T . P^T on MFMA
//                    with an fp32 online softmax, and writes one normalised partial per sequence
//                    it touches: o as fp16 with a power-of-two factor per 128 columns, and lse.
//   3. combine_proj  log-sum-exp merge of the partials of each (sequence, head) -> o_lat (bf16, LDS)
//                    and lse, then out = bf16(o_lat . W_UV^T) per head (MFMA).
#include <atomic>
#include <mutex>

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {

constexpr int kTileTok = 32;                     // cached rows per LDS tile

struct Plan {
  int64_t total_tokens;   // N = sum of clamped lengths
  int32_t runs;           // G = number of non-empty runs (<= launched units)
  int32_t pad;
};

__device__ __forceinline__ int64_t run_start(int64_t g, int64_t N, int64_t G) { return g * N / G; }

// Where run g starts: its first sequence b, the position t0 of its first row in b, the boundary
// cum[b + 1] where b ends, and b's first cache row (written by the plan so that an attention block
// reaches its first rows with one load).
struct RunStart {
  int64_t row_base;
  int64_t next;
  int32_t b;
  int32_t t0;
};
// Run containing global token x (0 <= x < N).
__device__ __forceinline__ int64_t run_of(int64_t x, int64_t N, int64_t G) { return ((x + 1) * G - 1) / N; }

// ---------------------------------------------------------------------------------------------
// 1. q_lat[b,h,c] = bf16(sum_d q[b,h,d] W_UK[h,d,c]); block (h, 1 + kCols-column slice of c).
//    W_UK[h] rows are stored with c contiguous; the slice goes to LDS as it is and the transposing
//    LDS read gives the MFMA B operand eight consecutive d per lane. Block (0, 0), dispatched
//    first, builds the plan.
// ---------------------------------------------------------------------------------------------
// W_UK columns per absorb block: 128 from 32 sequences up (each query row is then read by four
// blocks instead of eight, and a block writes 256 contiguous bytes of it), else 64 (more blocks to
// stream W_UK when it dominates). Bytes per W_UK row of a slice in LDS: kCols * 2 + 16.
constexpr int kAbsWideFrom = 32;

template <int kCols>
__global__ __launch_bounds__(256) void absorb_plan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ wkv_b, int batch, int n_heads,
    uint16_t* __restrict__ q_lat, const int32_t* __restrict__ seqlens, int64_t max_seqlen,
    int units, int min_unit_tokens, Plan* __restrict__ plan, int64_t* __restrict__ cum,
    const int64_t* __restrict__ row_offset, int64_t cache_rows_per_seq, RunStart* __restrict__ runs) {
  constexpr int kAbsCols = kCols, kAbsCb = kCols / 16, kWrPitch = kCols * 2 + 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  __shared__ __attribute__((aligned(16))) uint8_t wr[kNope * kWrPitch];
  __shared__ int64_t scan[256];
  __shared__ int64_t rowb_s[256];
  __shared__ int64_t wsum_s[4];
  __shared__ int64_t total_runs[2];

  if (blockIdx.y == 0) {
    // the plan, in a block of its own beside the absorb blocks
    if (blockIdx.x != 0) return;
    const int per = (batch + 255) / 256;
    if (per == 1) {
      // One sequence per thread: its clamped length and first cache row are loaded together, the
      // inclusive prefix sums taken within each wave by shuffles and across the four waves
      // through LDS (cum[b] = sum_{b' < b} clamp(L_b', 0, max_seqlen)).
      int64_t len = 0, rb = 0;
      if (tid < batch) {
        len = min<int64_t>(max<int64_t>(seqlens[tid], 0), max_seqlen);
        rb = row_offset ? row_offset[tid] : static_cast<int64_t>(tid) * cache_rows_per_seq;
      }
      rowb_s[tid] = rb;
      int64_t v = len;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
      }
      if (lane == 63) wsum_s[wave] = v;
      __syncthreads();
      for (int w2 = 0; w2 < wave; ++w2) v += wsum_s[w2];
      scan[tid] = v;
      if (tid < batch) cum[tid] = v - len;
      if (tid == 255) {
        const int64_t N = v;
        cum[batch] = N;
        int64_t G = (N + min_unit_tokens - 1) / min_unit_tokens;
        G = min<int64_t>(G, units);
        plan->total_tokens = N;
        plan->runs = static_cast<int32_t>(N > 0 ? max<int64_t>(G, 1) : 0);
        plan->pad = 0;
        total_runs[0] = N;
        total_runs[1] = N > 0 ? max<int64_t>(G, 1) : 0;
      }
      __syncthreads();   // prefix sums, first rows and the run count are known
      // thread i writes runs i, i + 256, ...: run g starts in the first sequence b whose inclusive
      // prefix sum exceeds run_start(g)
      const int64_t N = total_runs[0], G = total_runs[1];
      for (int64_t g = tid; g < G; g += 256) {
        const int64_t x = run_start(g, N, G);
        int lo_b = 0, hi_b = batch - 1;
        while (lo_b < hi_b) {
          const int mid = (lo_b + hi_b) >> 1;
          if (scan[mid] > x) hi_b = mid;
          else lo_b = mid + 1;
        }
        const int b = lo_b;
        RunStart rs;
        rs.b = b;
        rs.t0 = static_cast<int32_t>(x - (b > 0 ? scan[b - 1] : 0));
        rs.next = scan[b];
        rs.row_base = rowb_s[b];
        runs[g] = rs;
      }
      return;
    }
    // More than 256 sequences: each thread owns a contiguous chunk of them.
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
    const int64_t chunk0 = scan[tid] - s;   // cum[b0]
    int64_t run = chunk0;
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
      total_runs[0] = N;
      total_runs[1] = N > 0 ? max<int64_t>(G, 1) : 0;
    }
    __syncthreads();   // the run count is known
    // Each thread writes the records of the runs that start in its own sequences: run g starts in
    // sequence b iff cum[b] <= g N / G < cum[b+1], i.e. ceil(cum[b] G / N) <= g < ceil(cum[b+1] G / N).
    // run_start(g) = floor(g N / G) is stepped from run to run (quotient and remainder of N / G)
    // rather than divided out per record.
    const int64_t N = total_runs[0], G = total_runs[1];
    if (G > 0) {
      const int64_t qN = N / G, rN = N % G;
      int64_t lo = chunk0;
      for (int b = b0; b < b1; ++b) {
        const int64_t hi = lo + min<int64_t>(max<int64_t>(seqlens[b], 0), max_seqlen);
        const int64_t row_base = row_offset ? row_offset[b] : static_cast<int64_t>(b) * cache_rows_per_seq;
        int64_t g = (lo * G + N - 1) / N;           // first run starting at or after lo
        if (g < G && hi > lo) {
          int64_t x = g * N / G, rem = g * N - x * G;   // x = run_start(g)
          while (g < G && x < hi) {                    // runs starting in [lo, hi)
            RunStart rs;
            rs.b = b;
            rs.t0 = static_cast<int32_t>(x - lo);
            rs.next = hi;
            rs.row_base = row_base;
            runs[g] = rs;
            ++g;
            x += qN;
            rem += rN;
            if (rem >= G) {
              ++x;
              rem -= G;
            }
          }
        }
        lo = hi;
      }
    }
    return;
  }

  // Block (h, 1 + slice): columns kCols slice .. + kCols - 1 for every query. Wave w takes the query groups
  // (16 queries each) w, w + 4, ...; a wave's first kAhead groups are loaded before the weight
  // slice, so that their latency overlaps its load, and every later group kAhead products ahead.
  const int h = blockIdx.x;
  const int c0 = (blockIdx.y - 1) * kAbsCols;
  const int r = lane & 15, grp = lane >> 4;
  const int n_grp = (batch + 15) / 16;
  constexpr int kAhead = 4;
  uint4 qa[kAhead][4];
  auto load_q = [&](int gi, uint4 (&dst)[4]) {
    const uint16_t* qrow = q + (static_cast<int64_t>(min(16 * gi + r, batch - 1)) * n_heads + h) * kQk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dst[ks] = ldg16(qrow + ks * 32 + grp * 8);
  };
#pragma unroll
  for (int i = 0; i < kAhead; ++i)
    if (wave + 4 * i < n_grp) load_q(wave + 4 * i, qa[i]);

  // W_UK[h][0:128][c0:c0+kCols], row-major in LDS (rows kWrPitch bytes apart)
  const uint16_t* wk = wkv_b + static_cast<int64_t>(h) * kKvRows * kKvLora + c0;
#pragma unroll
  for (int i = 0; i < kAbsCols / 16; ++i) {
    const int idx = tid + 256 * i;
    const int d = idx / (kAbsCols / 8), ch = idx % (kAbsCols / 8);
    *reinterpret_cast<uint4*>(wr + d * kWrPitch + ch * 16) = ldg16(wk + static_cast<int64_t>(d) * kKvLora + ch * 8);
  }
  __syncthreads();
  if (wave >= n_grp) return;

  // B operand of column block cb, k-step ks: column c = 16 cb + r, rows d = 32 ks + 8 grp .. +7,
  // by two transposing reads (rows +0..3 and +4..7 of the 16-column block)
  bf16x8 bw[kAbsCb][4];
#pragma unroll
  for (int cb = 0; cb < kAbsCb; ++cb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint8_t* p = wr + (32 * ks + 8 * grp + (r >> 2)) * kWrPitch + (16 * cb + 4 * (r & 3)) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * kWrPitch));
      bw[cb][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }

  // q_lat^T = W_UK^T q^T for the slice's kCols columns x 16 queries: lane (r, grp) ends with
  // columns 16 cb + 4 grp .. +3 of query 16 gi + r (one 8-byte store per column block: 2 kCols
  // contiguous bytes of the query's row per wave)
  auto product = [&](int gi, const uint4 (&a)[4]) {
    const int b = 16 * gi + r;
    uint16_t* dst = q_lat + (static_cast<int64_t>(b) * n_heads + h) * kKvLora + c0 + grp * 4;
#pragma unroll
    for (int cb = 0; cb < kAbsCb; ++cb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(bw[cb][ks], as_bf16x8(a[ks]), acc);
      if (b < batch)
        *reinterpret_cast<uint2*>(dst + 16 * cb) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
  };
  for (int g0 = wave; g0 < n_grp; g0 += 4 * kAhead) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int gi = g0 + 4 * i;
      if (gi < n_grp) {
        product(gi, qa[i]);
        if (gi + 4 * kAhead < n_grp) load_q(gi + 4 * kAhead, qa[i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 0. Top-k mode ("DeepSeek-V3.2-Exp · Attention update", mla-decode excerpt: the indexer's top-k
//    positions of each sequence become a mask of 0 at those positions and -inf elsewhere, added to
//    the scores). The mask is a scatter, so a position the list names twice is still attended
//    once. Block b keeps, in list order, the first entry for each position of the sequence
//    (0 <= index < L_b) and counts them; the attention then runs over that many rows of sequence b,
//    read through the compacted list. Entries outside [0, L_b) name nothing.
//    Caches of up to kBitmapPositions positions (max_seqlen): a bitmap of the sequence's positions
//    in LDS, one bit set per named position (a repeat sets it again), then a scan over its words
//    writes the named positions in ascending order -- the attention then reads the cache rows
//    front to back. Longer caches: an open-addressing table of `slots` (a power of two >= 2 k) per
//    sequence, in LDS or the workspace, key = position, value = the lowest list index naming it
//    (atomicMin), and the first entries in list order, so that neither the survivors nor their
//    order depend on the order of the atomics.
// ---------------------------------------------------------------------------------------------
constexpr int32_t kEmptySlot = -1;

__device__ __forceinline__ uint32_t topk_hash(int32_t idx, int slots) {
  return (static_cast<uint32_t>(idx) * 0x9E3779B1u) & static_cast<uint32_t>(slots - 1);
}

constexpr int kBitmapWords = 15360;                       // 60 KB of LDS
constexpr int64_t kBitmapPositions = 32LL * kBitmapWords;   // 491,520 positions

__global__ __launch_bounds__(256) void topk_bitmap_kernel(const int32_t* __restrict__ topk, int k,
                                                          const int32_t* __restrict__ seqlens, int64_t max_seqlen,
                                                          int32_t* __restrict__ list, int32_t* __restrict__ counts) {
  extern __shared__ uint32_t bits[];
  __shared__ int wave_total[4];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = static_cast<int>(min<int64_t>(max<int64_t>(seqlens[b], 0), max_seqlen));
  const int32_t* src = topk + static_cast<int64_t>(b) * k;
  int32_t* dst = list + static_cast<int64_t>(b) * k;
  const int nw = (L + 31) >> 5;
  for (int i = tid; i < nw; i += 256) bits[i] = 0u;
  __syncthreads();
  for (int j = tid; j < k; j += 256) {
    const int32_t idx = src[j];
    if (idx >= 0 && idx < L) atomicOr(&bits[idx >> 5], 1u << (idx & 31));
  }
  __syncthreads();
  // thread t owns words [t per, t per + per): its count, the block's exclusive prefix of the counts
  // (shuffles within a wave, then across the four waves through LDS), then its positions in order
  const int per = (nw + 255) >> 8;
  const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_total[w];
  int pos = base + incl - cnt;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      dst[pos++] = 32 * w + __ffs(m) - 1;
      m &= m - 1;
    }
  }
  if (tid == 255) counts[b] = base + incl;
}

// Lists of up to kTopkLdsEntries entries keep their table in LDS (slots * 8 bytes, dynamic);
// longer ones in the workspace, where the atomics go to L2.
constexpr int kTopkLdsEntries = 2048;

template <bool kLds>
__global__ __launch_bounds__(256) void topk_compact_kernel(const int32_t* __restrict__ topk, int k,
                                                           const int32_t* __restrict__ seqlens, int64_t max_seqlen,
                                                           int slots, int2* __restrict__ table,
                                                           int32_t* __restrict__ list, int32_t* __restrict__ counts) {
  extern __shared__ int2 tab_lds[];
  __shared__ int wave_count[4];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = min<int64_t>(max<int64_t>(seqlens[b], 0), max_seqlen);
  const int32_t* src = topk + static_cast<int64_t>(b) * k;
  int32_t* dst = list + static_cast<int64_t>(b) * k;
  int2* tab = kLds ? tab_lds : table + static_cast<int64_t>(b) * slots;
  const uint32_t mask = static_cast<uint32_t>(slots - 1);
  // the table starts empty
  for (int i = threadIdx.x; i < slots; i += 256) tab[i] = make_int2(kEmptySlot, 0x7fffffff);
  if (!kLds) __threadfence();
  __syncthreads();
  // every valid entry claims its position's slot (or finds it claimed) and lowers its value
  for (int j = threadIdx.x; j < k; j += 256) {
    const int32_t idx = src[j];
    if (idx < 0 || idx >= L) continue;
    uint32_t h = topk_hash(idx, slots);
    while (true) {
      const int32_t prev = atomicCAS(&tab[h].x, kEmptySlot, idx);
      if (prev == kEmptySlot || prev == idx) {
        atomicMin(&tab[h].y, j);
        break;
      }
      h = (h + 1) & mask;
    }
  }
  if (!kLds) __threadfence();
  __syncthreads();
  // the entry survives iff it is the first naming its position (workspace table: read at device
  // scope, since atomics wrote it in L2)
  auto slot_key = [&](uint32_t h) {
    return kLds ? tab[h].x : __hip_atomic_load(&tab[h].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto slot_val = [&](uint32_t h) {
    return kLds ? tab[h].y : __hip_atomic_load(&tab[h].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int base = 0;
  for (int j0 = 0; j0 < k; j0 += 256) {
    const int j = j0 + static_cast<int>(threadIdx.x);
    const int32_t idx = j < k ? src[j] : -1;
    bool keep = idx >= 0 && idx < L;
    if (keep) {
      uint32_t h = topk_hash(idx, slots);
      while (slot_key(h) != idx) h = (h + 1) & mask;
      keep = slot_val(h) == j;
    }
    const uint64_t m = __ballot(keep);
    if (lane == 0) wave_count[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_count[w];
    if (keep) dst[off + __popcll(m & ((uint64_t(1) << lane) - 1))] = idx;
    base += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[b] = base;
}

// ---------------------------------------------------------------------------------------------
// 2. Split-KV attention over runs.
//
//    Block = 8 waves and 64 heads: head group hg covers heads [64 hg, 64 hg + 64); slots past
//    n_heads (16 or 32 heads) run on a zero query and are never stored. Cached rows stream through
//    a 4-deep ring of 32-row LDS tiles filled by 16-byte direct-to-LDS buffer loads. Each tile's
//    buffer descriptor ends at the segment's last row, so rows past it read as zeros, and every
//    row is read from HBM once per head group.
//    Waves w and w + 4 share a SIMD. The waves split by role:
//      score waves 0, 1   wave s holds the query of heads 32s .. 32s+31 (absorbed latent and rotary
//                         part, 576 features, as two blocks of 16 heads) in VGPRs and computes
//                         S^T[t][h] = sum_k tile[t][k] q[h][k] on MFMA (A operand: ds_read_b128 of
//                         tile rows, each read feeding both head blocks), then the softmax: per
//                         head a reference m (log2 units, scale folded in) that moves only when a
//                         lane's sum of a tile's weights exceeds 2^16 (then to the head's maximum,
//                         if that lies more than 8 above it), p = 2^(s - m) written to LDS as bf16
//                         (a common part keeps the reference; a full part on a branch of its own
//                         moves it);
//      value waves 2, 3, 6, 7   value wave v (0..3 in that order) owns latent columns
//                         [128 v, 128 v + 128) of all 64 heads and adds O^T[c][h] += sum_t
//                         tile[t][c] P^T[t][h] (A operand: ds_read_b64_tr_b16, the transposing LDS
//                         read, of tile columns; B operand: ds_read_b128 of P); the two value waves
//                         of SIMDs 2 and 3 keep those matrix pipes busy while the score waves keep
//                         those of SIMDs 0 and 1;
//      loader waves 4, 5  issue every tile load (18 each per tile) and wait for them.
//    One barrier per tile. Iteration j: the score waves run the MFMAs of S(j+1) with the softmax
//    of tile j (its scores held in registers since the previous iteration) interleaved between
//    them, so that the matrix pipe works on the scores while the vector ALU works on the
//    exponentials; the value waves run the MFMAs of tile j-1 against P(j-1) and read tile j's V^T
//    into registers; the loaders issue the loads of tile j+3 into the stage tile j-1 held (so three
//    tiles are in flight). P and the rescale factors are double-buffered by tile parity. A head
//    block with a rescale factor other than 1 (its reference moved) has its accumulators rescaled
//    before the value MFMAs of that tile, outside the MFMA chain.
//    P^T comes out of the S^T accumulators with lane l holding tokens 4(l/16)+{0..3} and
//    16+4(l/16)+{0..3} of head l%16 of a head block -- its k-group of the P.V product -- and V^T is
//    read in the same token order.
//    LDS layouts: latent part of a tile [32 rows][1024 B] with 16-byte chunk c of row r at
//    c ^ fk(r), fk(r) = 2(r&7); rotary part [32 rows][128 B] with chunk c at c ^ ((r>>1)&7); P as
//    [4 token chunks][64 heads][16 B]. A 128-bit LDS read serves each half-wave in two passes, one
//    for lanes 0-7 and 24-31 and one for lanes 8-23 (as measured with the LDS bank-conflict
//    counter), over 64 banks that hold one 256-byte line: each pass of the score reads (rows r,
//    chunks 4k + l/16), of the P reads (heads r, chunk l/16) and of the rotary reads then touches
//    16 distinct 16-byte bank groups, and the transposing reads of a half-wave (8 rows at two
//    adjacent chunks each) touch all 32 8-byte bank pairs once.
// ---------------------------------------------------------------------------------------------
constexpr int kKvBytes = kTileTok * kKvLora * 2;           // 32768
constexpr int kPeBytes = kTileTok * kRope * 2;             // 4096
constexpr int kTileBytes = kKvBytes + kPeBytes;            // 36864
constexpr int kStages = 4;                                 // tiles in the LDS ring
constexpr int kBlockHeads = 64;                            // heads of one workgroup
constexpr int kPBytes = kTileTok / 8 * kBlockHeads * 16;   // one P buffer
constexpr int kLoadsPerLoader = kTileBytes / 1024 / 2;     // 18: 16 latent rows and 16 rotary rows

__device__ __forceinline__ int fk(int row) { return 2 * (row & 7); }
__device__ __forceinline__ int fp(int row) { return (row >> 1) & 7; }

// Wait until at most `tiles_after` tiles of this wave's loads (L per tile) are still in flight
// (one tile is the steady state of the loops).
template <int L>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  if (tiles_after == 1) wait_vm<L>();
  else if (tiles_after >= 3) wait_vm<3 * L>();
  else if (tiles_after == 2) wait_vm<2 * L>();
  else wait_vm<0>();
}

__device__ __forceinline__ bf16x8 lds_b128(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Two transposing 8-byte reads (rows +0 and +16 of the tile) -> one A operand of 8 tokens.
__device__ __forceinline__ bf16x8 lds_vt(const uint8_t* p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 16 * 1024));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// State shared by the three roles of an attention workgroup. All walk the same segments (the
// pieces of the run that lie in one sequence) and pass the same n_tiles + 3 barriers per segment.
// Barrier k: tile k has landed (loaders wait for it before); for k >= 1 the stage of tile k-2 is
// free (its scores were taken after barrier k-2, its V^T read after barrier k-1), and the score
// waves have published P(k-2); after the last tile, barrier n_tiles + 1 publishes P(n_tiles - 1)
// and barrier n_tiles + 2 the per-head sums. Score waves: barrier 0, then scores(0); barrier j + 1,
// then scores(j+1) and softmax(j). Value waves: barriers 0 and 1, then V^T(0); barrier j + 1
// (j >= 1), then P(j-1), the MFMAs of tile j-1 and V^T(j). Loaders: tiles 0, 1, barrier 0,
// tiles 2, 3, barrier 1; barrier j + 1 (j >= 1), then tile j + 3.
struct AttendCtx {
  const uint16_t* q_lat;
  const uint16_t* q;
  const uint16_t* kv;
  const uint16_t* pe;
  const int64_t* row_offset;
  int64_t max_seqlen;
  const int32_t* list;       // top-k mode: attended positions of each sequence, compacted; else null
  int list_pitch;
  const int64_t* cum;
  const RunStart* runs;
  int batch, n_heads, head0;
  int64_t g, start, end;
  float scale_log2;
  uint16_t* part_o;
  float* part_s;
  float* part_l;
  uint8_t* ring;
  uint8_t* pbuf;
  float (*alpha_s)[kBlockHeads];
  float* l_s;
  int wave, lane;
};

struct Segment {
  int b, n_rows, n_tiles;
  const uint16_t* kv_seg;   // first row of the segment (top-k mode: of the sequence)
  const uint16_t* pe_seg;
  const int32_t* list_seg;  // top-k mode: the segment's positions
};

// First sequence of the run; then advance() steps through the sequences the run covers.
struct SegmentWalk {
  int64_t start;
  int b;
  bool first;
  RunStart rs;
  __device__ SegmentWalk(const AttendCtx& c) : start(c.start), first(true) {
    rs = c.runs[c.g];
    b = rs.b;
  }
  __device__ bool next(const AttendCtx& c, Segment& sg) {
    if (start >= c.end) return false;
    // the run's first segment comes from its record; later ones from the prefix sums
    const int64_t seq0 = first ? start - rs.t0 : c.cum[b];
    const int64_t seg_end = min(c.end, first ? rs.next : c.cum[b + 1]);
    const int t0 = static_cast<int>(start - seq0);
    sg.b = b;
    sg.n_rows = static_cast<int>(seg_end - start);
    sg.n_tiles = (sg.n_rows + kTileTok - 1) / kTileTok;
    const int64_t base = first ? rs.row_base
                               : (c.row_offset ? c.row_offset[b] : static_cast<int64_t>(b) * c.max_seqlen);
    first = false;
    const int64_t row0 = c.list ? base : base + t0;
    sg.kv_seg = c.kv + row0 * kKvLora;
    sg.pe_seg = c.pe + row0 * kRope;
    sg.list_seg = c.list ? c.list + static_cast<int64_t>(b) * c.list_pitch + t0 : nullptr;
    start = seg_end;
    ++b;
    while (b < c.batch && c.cum[b + 1] <= start) ++b;
    return true;
  }
};

// Loads of tile t of segment sg into ring stage t % 4 by loader ld (0, 1): latent rows ld + 2k
// (k < 16) -- physical chunk `lane` holds logical chunk lane ^ fk(row) -- and rotary rows
// 16 ld + 8e + lane/8 (e < 2; physical chunk lane%8 holds logical chunk (lane%8) ^ fp(row)). The
// descriptors start at the tile's first row and cover its rows up to the segment's last (none for
// a tile past the segment: it loads zeros and reads no memory); kv_voff[k] / pe_voff[e] are the
// byte offsets of the lane's chunks from the tile's first row.
__device__ __forceinline__ void issue_tile(const AttendCtx& c, const Segment& sg, int t, int ld,
                                           const uint32_t* kv_voff, const uint32_t* pe_voff) {
  const int left = sg.n_rows - t * kTileTok;
  const uint32_t rows = static_cast<uint32_t>(left <= 0 ? 0 : (left < kTileTok ? left : kTileTok));
  const int64_t row0 = left <= 0 ? 0 : static_cast<int64_t>(t) * kTileTok;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(sg.kv_seg + row0 * kKvLora, rows * 1024u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(sg.pe_seg + row0 * kRope, rows * 128u);
  const uint32_t dst = lds_addr(c.ring) + (t % kStages) * kTileBytes;
#pragma unroll
  for (int k = 0; k < 16; ++k) dma16(rk, dst + (ld + 2 * k) * 1024, kv_voff[k]);
#pragma unroll
  for (int e = 0; e < 2; ++e) dma16(rp, dst + kKvBytes + (2 * ld + e) * 1024, pe_voff[e]);
}

// Top-k mode: the tile's rows are the cache rows of the positions list_seg[32 t .. 32 t + 31] of
// the sequence (read with scalar loads: the list is uniform across the wave and never changes
// during the kernel), fetched one issue ahead (TilePos) so that their latency is not paid at the
// issue. Rows past the segment get a position one past the descriptors' range (max_seqlen rows
// from the sequence's first), so they read as zeros. kv_chunk[k] and pe_chunk[e] are the lane's
// byte offsets within its row.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
struct TilePos {
  uint32_t kv[16];   // rows ld + 2k of the tile
  uint32_t pe[16];   // rows 16 ld + j
};
__device__ __forceinline__ void load_tile_pos(const AttendCtx& c, const Segment& sg, int t, int ld, TilePos& p) {
  const int left = sg.n_rows - t * kTileTok;
  const uint32_t past = static_cast<uint32_t>(c.max_seqlen);
  const const_i32_ptr ti = (const_i32_ptr)(sg.list_seg + t * kTileTok);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int row = ld + 2 * k;
    p.kv[k] = row < left ? static_cast<uint32_t>(ti[row]) : past;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 16 * ld + j;
    p.pe[j] = row < left ? static_cast<uint32_t>(ti[row]) : past;
  }
}
__device__ __forceinline__ void issue_tile_gather(const AttendCtx& c, const Segment& sg, int t, int ld,
                                                  const uint32_t* kv_chunk, const uint32_t* pe_chunk,
                                                  const TilePos& p) {
  const uint32_t past = static_cast<uint32_t>(c.max_seqlen);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(sg.kv_seg, past * 1024u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(sg.pe_seg, past * 128u);
  const uint32_t dst = lds_addr(c.ring) + (t % kStages) * kTileBytes;
#pragma unroll
  for (int k = 0; k < 16; ++k) dma16(rk, dst + (ld + 2 * k) * 1024, p.kv[k] * 1024u + kv_chunk[k]);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t ppos = past;
#pragma unroll
    for (int j = 0; j < 8; ++j) ppos = (c.lane >> 3) == j ? p.pe[8 * e + j] : ppos;
    dma16(rp, dst + kKvBytes + (2 * ld + e) * 1024, ppos * 128u + pe_chunk[e]);
  }
}

// Loader waves 4, 5: every tile load of the block, and the waits for them before the barrier that
// publishes a tile. The first two tiles of a segment go out alone and the next two once the first
// has landed, so that at a launch the first tile of every block is not queued behind 147 KB per CU;
// then iteration j issues tile j+3 into the stage tile j-1 held.
template <bool kGather>
__device__ __forceinline__ void load_role(const AttendCtx& c) {
  constexpr int L = kLoadsPerLoader;
  const int ld = c.wave - 4, lane = c.lane;
  uint32_t kv_voff[16], pe_voff[2];   // dense mode: from the tile's first row; top-k: within the row
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int row = ld + 2 * k;
    kv_voff[k] = static_cast<uint32_t>((kGather ? 0 : row * 1024) + ((lane ^ fk(row)) << 4));
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = 16 * ld + 8 * e + (lane >> 3);
    pe_voff[e] = static_cast<uint32_t>((kGather ? 0 : row * 128) + (((lane & 7) ^ fp(row)) << 4));
  }
  TilePos pos;   // top-k mode: positions of the next tile to issue
  SegmentWalk walk(c);
  Segment sg;
  while (walk.next(c, sg)) {
    const int n_tiles = sg.n_tiles;
    int issued = 0;
    auto issue = [&]() {
      if (kGather) {
        issue_tile_gather(c, sg, issued, ld, kv_voff, pe_voff, pos);
        if (issued + 1 < n_tiles) load_tile_pos(c, sg, issued + 1, ld, pos);
      } else {
        issue_tile(c, sg, issued, ld, kv_voff, pe_voff);
      }
      ++issued;
    };
    if (kGather) load_tile_pos(c, sg, 0, ld, pos);
    while (issued < 2 && issued < n_tiles) issue();
    wait_tiles<L>(issued - 1);
    lds_barrier();   // tile 0 landed
    while (issued < kStages && issued < n_tiles) issue();
    if (n_tiles > 1) wait_tiles<L>(issued - 2);
    lds_barrier();   // tile 1 landed
    for (int j = 1; j <= n_tiles; ++j) {
      if (j + 1 < n_tiles) wait_tiles<L>(issued - 2 - j);
      lds_barrier();   // tile j+1 landed; the stage of tile j-1 is free
      if (issued < n_tiles) issue();
    }
    lds_barrier();   // l published
  }
}

// Score waves 0, 1. Wave s holds the query of heads 32s + 16hb + r (hb = 0, 1: absorbed latent part,
// 16 k-steps, and rotary part, 2 k-steps; B operands, k-group grp of the head per lane) and
// computes S^T[t][h] for all 32 tokens of a tile over the full 576 features (A operand:
// ds_read_b128 of tile rows, each read feeding the MFMAs of both head blocks). Iteration j (one
// barrier each) runs the MFMAs of tile j+1 and, interleaved with them, the softmax of tile j, whose
// scores the previous iteration left in registers: per head a reference m (log2 units, scale folded
// in) that moves only when a lane's sum of a tile's weights p = 2^(s - m) exceeds 2^16; P goes to
// LDS as bf16 with the head's rescale factor. They issue no loads: a tile is complete
// once the loader waves, which wait for their own loads of it, reach the next barrier.
__device__ __forceinline__ void score_role(const AttendCtx& c) {
  const int s = c.wave, lane = c.lane, r = lane & 15, grp = lane >> 4;
  // LDS byte offsets. Latent k-step ks = 4a + k: row 16 tb + r, logical chunk 4 ks + grp at
  // physical 16 a + 4 (k ^ (fk>>2)) + (grp ^ (fk&3)); a and tb go into immediates. Rotary k-step
  // 16 + e: row 16 tb + r, chunk 4 e + grp at (4 e + grp) ^ fp(r).
  const int sf = fk(r);
  int s_off[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s_off[k] = r * 1024 + 64 * (k ^ (sf >> 2)) + 16 * (grp ^ (sf & 3));
  int e_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) e_off[e] = kKvBytes + r * 128 + 16 * ((4 * e + grp) ^ fp(r));
  const int hl0 = 32 * s + r;                       // block-local head of head block 0 (+16 for block 1)
  const int p_wr = (grp * kBlockHeads + hl0) * 16;  // + 256 for head block 1
  const int head0 = c.head0 + hl0;
  const bool real0 = head0 < c.n_heads, real1 = head0 + 16 < c.n_heads;

  SegmentWalk walk(c);
  Segment sg;
  while (walk.next(c, sg)) {
    const int n_tiles = sg.n_tiles;
    bf16x8 qf[2][18];
    {
      const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bool real = hb ? real1 : real0;
        const int hq = real ? head0 + 16 * hb : 0;
        const uint16_t* ql = c.q_lat + (static_cast<int64_t>(sg.b) * c.n_heads + hq) * kKvLora + grp * 8;
        const uint16_t* qp = c.q + (static_cast<int64_t>(sg.b) * c.n_heads + hq) * kQk + kNope + grp * 8;
#pragma unroll
        for (int j = 0; j < 16; ++j) qf[hb][j] = as_bf16x8(real ? ldg16(ql + j * 32) : z);
#pragma unroll
        for (int e = 0; e < 2; ++e) qf[hb][16 + e] = as_bf16x8(real ? ldg16(qp + e * 32) : z);
      }
    }
    // S^T of tile t: acc[tb][hb] holds tokens 16 tb + 4 grp + {0..3} of head 32 s + 16 hb + r.
    auto scores = [&](int t, f32x4 (&acc)[2][2]) {
      const uint8_t* tile = c.ring + (t % kStages) * kTileBytes;
      auto rd = [&](int tb, int ks) {
        return ks < 16 ? lds_b128(tile + tb * 16384 + (ks >> 2) * 256 + s_off[ks & 3])
                       : lds_b128(tile + tb * 2048 + e_off[ks - 16]);
      };
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const bf16x8 a = rd(tb, ks);
          acc[tb][0] = mfma16x16x32(a, qf[0][ks], acc[tb][0]);
          acc[tb][1] = mfma16x16x32(a, qf[1][ks], acc[tb][1]);
        }
    };
    // per head block: reference (log2 units) and this lane's running sum of its tokens' weights. The
    // reference starts finite, far below any score, so that a masked score (-inf) gives the weight
    // 0 rather than NaN before the first tile moves it (this file is built without NaN semantics).
    constexpr float kNoRef = -1e30f;
    float m_ref[2] = {kNoRef, kNoRef}, lsum[2] = {0.f, 0.f}, lsum_prev[2] = {0.f, 0.f};
    // Softmax of tile t from its scores, in two parts. The common part assumes the references stay
    // (rescale factor exactly 1): P = 2^(s - m) and the sums, with no cross-lane step and no
    // maximum, and reports whether the lane's sum of its 8 weights of a head exceeds 2^16 (each
    // weight is below that sum, so the bf16 weights and the fp32 sums stay far inside their range
    // otherwise). If one does anywhere in the wave (rare after the first tile of a segment, whose
    // reference kNoRef makes every weight +inf), the full part, on a branch of its own, takes each
    // head's maximum, moves the references that lie more than 8 below it and redoes P, the sums and
    // the factors. kMask: rows at or past the segment end count as -inf (only the last tile of a
    // segment can have such rows).
    bool above = false;
    auto scaled = [&](int t, const f32x4 (&sc)[2][2], int hb, bool mask, float (&y)[8]) {
      const int valid = sg.n_rows - t * kTileTok - 4 * grp;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = sc[tb][hb][j] * c.scale_log2;
          y[tb * 4 + j] = (!mask || tb * 16 + j < valid) ? v : -INFINITY;
        }
    };
    // The common part works on the raw scores: p = 2^(s c - m) as one fma and one exp per score
    // (c = scale log2 e > 0), and tests the sum of the lane's weights, which it forms anyway.
    auto softmax_common = [&](int t, const f32x4 (&sc)[2][2], bool mask) {
      const int valid = sg.n_rows - t * kTileTok - 4 * grp;
      bool up = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float x[8], p[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            x[tb * 4 + j] = (!mask || tb * 16 + j < valid) ? sc[tb][hb][j] : -INFINITY;
        const float nm = -m_ref[hb];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(x[i], c.scale_log2, nm));
        lsum_prev[hb] = lsum[hb];
        const float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        lsum[hb] += ps;
        *reinterpret_cast<bf16x8*>(c.pbuf + (t & 1) * kPBytes + p_wr + hb * 256) = bf16x8_from_f32(p);
        c.alpha_s[t & 1][hl0 + 16 * hb] = 1.f;
        up |= ps > 65536.f;
      }
      above = up;
    };
    auto softmax_full = [&](int t, const f32x4 (&sc)[2][2], bool mask) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float y[8], p[8];
        scaled(t, sc, hb, mask, y);
        const float m =
            fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
        const float mx = max_over_rows(m);
        const bool up = mx > m_ref[hb] + 8.f;
        const float m_new = up ? mx : m_ref[hb];
        const float alpha = fast_exp2(m_ref[hb] - m_new);
        m_ref[hb] = m_new;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(y[i] - m_new);
        lsum[hb] = lsum_prev[hb] * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        *reinterpret_cast<bf16x8*>(c.pbuf + (t & 1) * kPBytes + p_wr + hb * 256) = bf16x8_from_f32(p);
        c.alpha_s[t & 1][hl0 + 16 * hb] = alpha;
      }
    };
    // Iteration j < n_tiles - 1: the scores of tile j+1 and the common softmax part of tile j in
    // one basic block, so that the softmax's vector
    // instructions can fill the gaps between MFMAs: four operand reads go out first, then each
    // pair of MFMAs (one per head block) is followed by the next read.
    auto step = [&](int j, const f32x4 (&cur)[2][2], f32x4 (&next)[2][2], bool mask) {
      lds_barrier();   // tile j+1 landed; P(j-1) consumed by the value waves
      scores(j + 1, next);
      softmax_common(j, cur, mask);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      if (__any(above)) softmax_full(j, cur, mask);
    };
    // The segment's last tile: its masked softmax alone (there is no next tile to score).
    auto last_step = [&](int j, const f32x4 (&cur)[2][2]) {
      lds_barrier();   // P(j-1) consumed by the value waves
      softmax_common(j, cur, true);
      if (__any(above)) softmax_full(j, cur, true);
    };

    f32x4 sa[2][2], sb[2][2];
    lds_barrier();   // tile 0 landed
    scores(0, sa);
    // Unrolled by two so that the scores of consecutive tiles alternate between sa and sb; the
    // last tile of the segment takes the masked softmax.
    int j = 0;
    for (; j + 2 < n_tiles; j += 2) {
      step(j, sa, sb, false);
      step(j + 1, sb, sa, false);
    }
    if (n_tiles - j == 2) {
      step(j, sa, sb, false);
      last_step(j + 1, sb);
    } else {
      last_step(j, sa);
    }
    lds_barrier();   // P of the last tile published
    // the log-sum-exp from the fp32 weights (the value waves normalise by their rounded sum)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float ltot = sum_over_rows(lsum[hb]);
      if (grp == 0 && (hb ? real1 : real0))
        c.part_l[(c.g + sg.b) * c.n_heads + head0 + 16 * hb] = (m_ref[hb] + __log2f(ltot)) * kLn2;
    }
    lds_barrier();   // l published
  }
}

// Value waves 2, 3, 6, 7 (v = 0..3): O^T += V^T P^T for latent columns [128 v, 128 v + 128) of
// all 64 heads, one tile behind the score waves. Iteration j: P^T and the rescale factors of tile
// j-1 from LDS (a head block whose reference moved has its accumulators scaled first, outside the
// MFMA chain), then, in one basic block, the MFMAs of tile j-1 (V^T from registers, read in the
// previous iteration) with the transposing reads of tile j's V^T placed between them.
__device__ __forceinline__ void value_role(const AttendCtx& c) {
  const int w = (c.wave & 1) + ((c.wave >> 2) << 1), lane = c.lane, r = lane & 15, grp = lane >> 4;
  // V^T: source row 4 grp + (r>>2) (+16), columns 16 (8 w + cb) + 4 (r&3) .. +3 at physical chunk
  // pair (8 w + cb) ^ (row & 7). P^T: head 16 hb + r, chunk grp.
  const int vrow = 4 * grp + (r >> 2);
  int v_off[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) v_off[cb] = vrow * 1024 + 256 * w + 32 * (cb ^ (vrow & 7)) + 8 * (r & 3);
  const int p_rd = (grp * kBlockHeads + r) * 16;

  SegmentWalk walk(c);
  Segment sg;
  while (walk.next(c, sg)) {
    const int n_tiles = sg.n_tiles;
    f32x4 o[8][4];   // O^T[16 (8 w + cb) + 4 grp + j][16 hb + r]
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) o[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Running sum of the bf16 weights of heads 16 w + r (this wave's head block w) over this lane's
    // k-group: exactly the weights the value MFMAs multiply, so that normalising by their total
    // leaves the rounding of P no effect on the weights' sum (the log-sum-exp the score waves keep
    // comes from the fp32 weights).
    float lr = 0.f;
    auto sum_mine = [&](int t) {
      const bf16x8 pm = lds_b128(c.pbuf + (t & 1) * kPBytes + p_rd + w * 256);
      const float am = c.alpha_s[t & 1][w * 16 + r];
      lr = lr * am + sum_bf16x8(pm);
    };
    auto read_v = [&](int t, bf16x8 (&vf)[8]) {
      const uint8_t* tile = c.ring + (t % kStages) * kTileBytes;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) vf[cb] = lds_vt(tile + v_off[cb]);
    };
    // P^T of tile t and its rescale factors; then the accumulators of heads whose reference moved
    // scaled (those of tile 0 are still zero)
    auto read_p = [&](int t, bf16x8 (&pf)[4], float (&a)[4]) {
      const uint8_t* pb = c.pbuf + (t & 1) * kPBytes + p_rd;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        pf[hb] = lds_b128(pb + hb * 256);
        a[hb] = c.alpha_s[t & 1][hb * 16 + r];
      }
    };
    auto rescale = [&](int t, const float (&a)[4]) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        if (t > 0 && __any(a[hb] != 1.f)) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) o[cb][hb] *= a[hb];
        }
      }
    };
    auto mfmas = [&](const bf16x8 (&vf)[8], const bf16x8 (&pf)[4]) {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) o[cb][hb] = mfma16x16x32(vf[cb], pf[hb], o[cb][hb]);
    };
    // Iteration 1 <= j <= n_tiles: barrier (tile j+1 landed; for j = n_tiles: P of the last tile
    // published), values of tile j-1, then the V^T of tile j (for j = n_tiles a stale stage, never
    // used), two MFMAs per transposing read.
    auto step = [&](int j, const bf16x8 (&prev)[8], bf16x8 (&cur)[8]) {
      lds_barrier();
      bf16x8 pf[4];
      float a[4];
      read_p(j - 1, pf, a);
      rescale(j - 1, a);
      mfmas(prev, pf);
      sum_mine(j - 1);
      read_v(j, cur);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
      for (int i = 0; i < 14; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    };

    bf16x8 va[8], vb[8];
    lds_barrier();   // tile 0 landed
    lds_barrier();   // tile 1 landed
    read_v(0, va);
    // unrolled by two so that the V^T of consecutive tiles alternates between va and vb
    for (int j = 1; j <= n_tiles; j += 2) {
      step(j, va, vb);
      if (j + 1 <= n_tiles) step(j + 1, vb, va);
    }
    {
      const float lt = sum_over_rows(lr);   // over the head's four k-groups
      if (grp == 0) c.l_s[w * 16 + r] = lt;
    }
    lds_barrier();   // l published
    // The normalised partial of each head, as fp16 times a power of two that brings the largest
    // magnitude among this wave's 128 columns into [2^14, 2^15); the inverse factor goes to part_s.
    const int64_t slot = c.g + sg.b;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float inv = 1.f / c.l_s[hb * 16 + r];
      float m = 0.f;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        o[cb][hb] *= inv;
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(o[cb][hb][j]));
      }
      m = max_over_rows(m);   // over the head's four lane groups
      int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xff) - 127;
      e = e < -110 ? -110 : (e > 127 ? 127 : e);
      const float sc = __uint_as_float(static_cast<uint32_t>(127 + 14 - e) << 23);
      if (c.head0 + hb * 16 < c.n_heads) {
        const int64_t row = slot * c.n_heads + c.head0 + hb * 16 + r;
        uint16_t* po = c.part_o + row * kKvLora + w * 128 + grp * 4;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const f32x4 v = o[cb][hb] * sc;
          *reinterpret_cast<uint2*>(po + cb * 16) = make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
        }
        if (grp == 0) c.part_s[row * 4 + w] = __uint_as_float(static_cast<uint32_t>(127 - 14 + e) << 23);
      }
    }
  }
}

template <bool kGather>
__global__ __launch_bounds__(512, 1) void attend_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ pe, const int64_t* __restrict__ row_offset, int64_t max_seqlen,
    const int32_t* __restrict__ list, int list_pitch,
    const Plan* __restrict__ plan, const int64_t* __restrict__ cum, const RunStart* __restrict__ runs, int batch,
    int n_heads, float scale_log2, uint16_t* __restrict__ part_o, float* __restrict__ part_s,
    float* __restrict__ part_l) {
  // The blocks of the head groups of one run share blockIdx mod 8 -- the same XCD and its L2 --
  // and are dispatched next to each other, so the tiles one of them pulls from HBM are L2 hits for
  // the others.
  const int64_t N = plan->total_tokens;
  const int64_t G = plan->runs;
  const int n_groups = (n_heads + kBlockHeads - 1) / kBlockHeads;
  const int hg = (blockIdx.x >> 3) % n_groups;
  const int64_t g = (blockIdx.x & 7) + 8 * (blockIdx.x / (8 * n_groups));
  if (g >= G) return;

  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * kPBytes];
  __shared__ float alpha_s[2][kBlockHeads];
  __shared__ float l_s[kBlockHeads];

  AttendCtx c;
  c.q_lat = q_lat; c.q = q; c.kv = kv; c.pe = pe; c.row_offset = row_offset; c.max_seqlen = max_seqlen;
  c.list = kGather ? list : nullptr; c.list_pitch = list_pitch;
  c.cum = cum; c.runs = runs; c.batch = batch; c.n_heads = n_heads; c.head0 = hg * kBlockHeads;
  c.g = g; c.start = run_start(g, N, G); c.end = run_start(g + 1, N, G);
  c.scale_log2 = scale_log2; c.part_o = part_o; c.part_s = part_s; c.part_l = part_l;
  c.ring = ring; c.pbuf = pbuf; c.alpha_s = alpha_s; c.l_s = l_s;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: wave-derived values live in SGPRs
  c.lane = threadIdx.x & 63;
  if (c.wave < 2) score_role(c);
  else if (c.wave == 4 || c.wave == 5) load_role<kGather>(c);
  else value_role(c);
}

// ---------------------------------------------------------------------------------------------
// 3. Merge and project out, per (head h, group of 16 sequences); a block takes every gridDim.y-th
//    group of its head, keeping the head's W_UV in registers across them. The partials of each
//    (sequence, h) over its runs are merged by their log-sum-exp weights (o_lat = sum_s
//    e^(lse_s - M) o_s / sum_s e^(lse_s - M), lse = M + ln sum_s e^(lse_s - M)) into an o_lat
//    tile in LDS (thread = sequence x 16 latent columns), kept as two bf16 tiles, the rounded
//    value and its residual, then out[b,h,d] = bf16(sum_c o_lat[b,c] W_UV[h,d,c]) on MFMA, one
//    product per tile into the same accumulator (A: o_lat rows from LDS; B: W_UV rows 16 w ..
//    16 w + 15 for wave w, from VGPRs). A sequence with no rows gets out = 0, lse = -inf.
// ---------------------------------------------------------------------------------------------
constexpr int kMergeAhead = 2;   // runs whose partial loads go out together

__global__ __launch_bounds__(512, 4) void combine_proj_kernel(
    const Plan* __restrict__ plan, const int64_t* __restrict__ cum, int batch, int n_heads,
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_s, const float* __restrict__ part_l,
    const uint16_t* __restrict__ wkv_b, int dsplit,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  // one buffer for the parts' partial merges (fp32 [16][512]) and, after them, the o_lat tile as
  // two bf16 tiles, the rounded value and its rounding residual ([2][16][512 + 8])
  __shared__ __attribute__((aligned(16))) float4 mbuf[2 * 16 * (kKvLora + 8) * 2 / 16];
  __shared__ float pm_s[16][2];
  float (*pa_s)[kKvLora] = reinterpret_cast<float (*)[kKvLora]>(mbuf);
  uint16_t (*ol)[kKvLora + 8] = reinterpret_cast<uint16_t (*)[kKvLora + 8]>(mbuf);
  uint16_t (*ol_lo)[kKvLora + 8] = ol + 16;
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int64_t N = plan->total_tokens, G = plan->runs;
  // blockIdx.y = group slot gy x output part dp: the block produces outputs d0 .. d0 + 128 / dsplit
  // of its head, from the first 8 / dsplit waves
  const int gy = blockIdx.y / dsplit, dp = blockIdx.y % dsplit, ngy = gridDim.y / dsplit;
  const int d0 = dp * (kVDim / dsplit);
  const bool proj = wave < 8 / dsplit;

  const uint16_t* wrow = wkv_b + (static_cast<int64_t>(h) * kKvRows + kNope + d0 + wave * 16 + r) * kKvLora + grp * 8;
  bf16x8 bw[16];
  if (proj) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) bw[ks] = as_bf16x8(ldg16(wrow + ks * 32));
  }

  const int j = tid >> 5, c0 = (tid & 31) * 16;   // thread group j (32 threads), columns c0 .. c0 + 15
  // A wave holds thread groups ja and ja + 1: the prefix sums they need are wave-uniform and come
  // through scalar loads, which do not queue behind W_UV's vector loads (those complete in issue
  // order, so a vector load of them would wait for all of W_UV)
  const int ja = 2 * __builtin_amdgcn_readfirstlane(wave);
  typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
  // groups of 16 sequences b0, b0 + 16 gridDim.y, ...: W_UV stays in registers across them
  for (int b0 = gy * 16; b0 < batch; b0 += ngy * 16) {
    // With fewer than 9 sequences in the group, each sequence's runs are shared by `parts` thread
    // groups (runs part, part + parts, ...), whose partial merges are then merged through LDS.
    const int nseq = min(16, batch - b0);
    const int parts = nseq <= 1 ? 16 : nseq <= 2 ? 8 : nseq <= 4 ? 4 : nseq <= 8 ? 2 : 1;
    const int js = j / parts, part = j % parts;   // sequence b0 + js
    const int b = b0 + js;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    float M = -INFINITY, wsum = 0.f;
    if (js < nseq) {
      const const_i64_ptr cs = (const_i64_ptr)(cum + b0);
      const int ka = min(ja / parts, nseq - 1), kb = min((ja + 1) / parts, nseq - 1);
      const int64_t xa0 = cs[ka], xa1 = cs[ka + 1], xb0 = cs[kb], xb1 = cs[kb + 1];
      const int64_t x0 = j == ja ? xa0 : xb0, x1 = j == ja ? xa1 : xb1;
      if (x1 > x0) {
        // One pass over the runs, kMergeAhead at a time: their loads go out together, then the running
        // maximum M moves to cover them (the sums so far scaled by e^(M_old - M_new)).
        const int64_t g0 = run_of(x0, N, G) + part, g1 = run_of(x1 - 1, N, G);
        for (int64_t g = g0; g <= g1; g += kMergeAhead * parts) {
          float l[kMergeAhead], s[kMergeAhead];
          uint4 v[kMergeAhead][2];
#pragma unroll
          for (int u = 0; u < kMergeAhead; ++u) {
            const int64_t gg = g + u * parts;
            const int64_t slot = (gg <= g1 ? gg : g) + b;
            l[u] = part_l[slot * n_heads + h];
            // factor of the 128-column slice c0 / 128 (one attention wave's columns)
            s[u] = part_s[(slot * n_heads + h) * 4 + (c0 >> 7)];
            const uint4* src = reinterpret_cast<const uint4*>(part_o + (slot * n_heads + h) * kKvLora + c0);
            v[u][0] = src[0];
            v[u][1] = src[1];
          }
          float mt = M;
#pragma unroll
          for (int u = 0; u < kMergeAhead; ++u)
            if (g + u * parts <= g1) mt = fmaxf(mt, l[u]);
          const float a = M == -INFINITY ? 0.f : __expf(M - mt);
          wsum *= a;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] *= a;
          M = mt;
#pragma unroll
          for (int u = 0; u < kMergeAhead; ++u) {
            if (g + u * parts > g1) continue;
            const float w = __expf(l[u] - M);
            wsum += w;
            // fp16 partial times the inverse of its power-of-two factor
            const float ws = w * s[u];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t uu[4] = {v[u][i].x, v[u][i].y, v[u][i].z, v[u][i].w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const f32x2 f = unpack_f16x2(uu[k]);
                acc[8 * i + 2 * k] += ws * f[0];
                acc[8 * i + 2 * k + 1] += ws * f[1];
              }
            }
          }
        }
      }
    }
    if (parts > 1) {
      // merge of the parts: thread group (js, 0) takes the others' (M, wsum, acc) from LDS
      if (b0 != gy * 16) __syncthreads();   // previous group's o_lat read
      pm_s[j][0] = M;
      pm_s[j][1] = wsum;
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<float4*>(&pa_s[j][c0 + i]) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
      __syncthreads();
      if (part == 0) {
        float Mt = M;
        for (int q = 1; q < parts; ++q) Mt = fmaxf(Mt, pm_s[j + q][0]);
        const float a0 = M == -INFINITY ? 0.f : __expf(M - Mt);
        wsum *= a0;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] *= a0;
        for (int q = 1; q < parts; ++q) {
          const float Mq = pm_s[j + q][0];
          const float aq = Mq == -INFINITY ? 0.f : __expf(Mq - Mt);
          wsum += aq * pm_s[j + q][1];
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(&pa_s[j + q][c0 + i]);
            acc[i] += aq * v.x;
            acc[i + 1] += aq * v.y;
            acc[i + 2] += aq * v.z;
            acc[i + 3] += aq * v.w;
          }
        }
        M = Mt;
      }
    }
    if (js < nseq && part == 0 && lse && dp == 0 && (tid & 31) == 0)
      lse[static_cast<int64_t>(b) * n_heads + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    // the parts' partials, or the previous group's o_lat, are read before o_lat is written
    if (parts > 1 || b0 != gy * 16) __syncthreads();
    if (part == 0) {
      // o_lat = hi + lo, both bf16: the product through W_UV sees o_lat to about 16 bits
#pragma unroll
      for (int i = 0; i < 16; i += 8) {
        float v[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = acc[i + e] * inv;
          lo[e] = v[e] - round_bf16(v[e]);
        }
        *reinterpret_cast<bf16x8*>(&ol[js][c0 + i]) = bf16x8_from_f32(v);
        *reinterpret_cast<bf16x8*>(&ol_lo[js][c0 + i]) = bf16x8_from_f32(lo);
      }
    }
    __syncthreads();
    if (proj) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        o = mfma16x16x32(*reinterpret_cast<const bf16x8*>(&ol[r][ks * 32 + grp * 8]), bw[ks], o);
        o = mfma16x16x32(*reinterpret_cast<const bf16x8*>(&ol_lo[r][ks * 32 + grp * 8]), bw[ks], o);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bb = b0 + grp * 4 + e;
        if (bb < batch) out[(static_cast<int64_t>(bb) * n_heads + h) * kVDim + d0 + wave * 16 + r] = f32_to_bf16_bits(o[e]);
      }
    }
  }
}

}  // namespace

constexpr int kMergeBlocks = 512;
constexpr int64_t kMinRunTokens = 32;

DecodeLayout decode_layout(int n_heads, int batch, int64_t max_seqlen, int topk) {
  DecodeLayout L{};
  // attended rows: at most max_seqlen per sequence, or topk in top-k mode (topk >= 0)
  const int64_t upper = static_cast<int64_t>(batch) * (topk >= 0 ? topk : max_seqlen);
  // one block per compute unit: 256 CUs, shared by the head groups of a run
  const int64_t max_units = 256 / ((n_heads + 63) / 64);
  // Runs of 256 tokens or more; shorter (whole tiles, down to kMinRunTokens) when the runs would
  // not fill the chip, so that a short cache is not read by a few blocks one tile after another.
  // Shorter runs mean more partials (H x 1 KB each) for the merge to read: a block's time grows
  // with its run (about 0.9 us per tile of 32 tokens) and the merge's with the number of runs
  // (H x 1 KB each at about 5 TB/s), which balance near 0.085 sqrt(tokens x H) tokens per run.
  int64_t run_tokens = (upper + max_units - 1) / max_units;
  const int64_t balance = static_cast<int64_t>(0.085 * std::sqrt(static_cast<double>(upper) * n_heads));
  run_tokens = run_tokens > balance ? run_tokens : balance;
  run_tokens = (run_tokens + 31) / 32 * 32;
  run_tokens = run_tokens < kMinRunTokens ? kMinRunTokens : (run_tokens > 256 ? 256 : run_tokens);
  L.min_unit_tokens = static_cast<int>(run_tokens);
  int64_t units = (upper + L.min_unit_tokens - 1) / L.min_unit_tokens;
  units = units < 1 ? 1 : (units > max_units ? max_units : units);
  L.units = static_cast<int>(units);
  const size_t B = static_cast<size_t>(batch), H = static_cast<size_t>(n_heads);
  const size_t slots = static_cast<size_t>(L.units) + B;
  size_t off = 0;
  L.plan_off = off;   off = align_up(off + sizeof(Plan));
  L.cum_off = off;    off = align_up(off + (B + 1) * sizeof(int64_t));
  L.runs_off = off;   off = align_up(off + static_cast<size_t>(L.units) * sizeof(RunStart));
  L.qlat_off = off;   off = align_up(off + B * H * kKvLora * sizeof(uint16_t));
  L.part_o_off = off; off = align_up(off + slots * H * kKvLora * sizeof(uint16_t));
  L.part_s_off = off; off = align_up(off + slots * H * 4 * sizeof(float));
  L.part_l_off = off; off = align_up(off + slots * H * sizeof(float));
  L.list_off = L.count_off = L.table_off = 0;
  L.topk_slots = 0;
  if (topk >= 0) {
    // 64 entries of slack: the attention's scalar loads of a last partial tile may read past a
    // sequence's count (those values are never used)
    L.list_off = off;  off = align_up(off + (B * static_cast<size_t>(topk) + 64) * sizeof(int32_t));
    L.count_off = off; off = align_up(off + B * sizeof(int32_t));
    // first-entry table: a power of two >= 2 topk slots (at least 256) of 8 bytes per sequence
    int64_t slots = 256;
    while (slots < 2 * static_cast<int64_t>(topk)) slots *= 2;
    L.topk_slots = static_cast<int>(slots);
    // (needed only beyond the bitmap's positions, and in LDS for lists of up to kTopkLdsEntries)
    L.table_off = off;
    if (max_seqlen > kBitmapPositions && topk > kTopkLdsEntries) off = align_up(off + B * static_cast<size_t>(slots) * 8);
  }
  L.total = off;
  return L;
}

hipError_t launch_decode(int n_heads, int batch, const uint16_t* q, const uint16_t* wkv_b,
                         const uint16_t* kv_cache, const uint16_t* pe_cache, const int64_t* row_offset,
                         const int32_t* seqlens, int64_t max_seqlen, const int32_t* topk_indices, int topk,
                         void* workspace, const DecodeLayout& lay, uint16_t* out, float* lse, float scale,
                         hipStream_t stream, hipEvent_t* ev) {
  char* ws = static_cast<char*>(workspace);
  Plan* plan = reinterpret_cast<Plan*>(ws + lay.plan_off);
  int64_t* cum = reinterpret_cast<int64_t*>(ws + lay.cum_off);
  RunStart* runs = reinterpret_cast<RunStart*>(ws + lay.runs_off);
  uint16_t* q_lat = reinterpret_cast<uint16_t*>(ws + lay.qlat_off);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(ws + lay.part_o_off);
  float* part_s = reinterpret_cast<float*>(ws + lay.part_s_off);
  float* part_l = reinterpret_cast<float*>(ws + lay.part_l_off);
  const float scale_log2 = scale * kLog2e;

  const bool sparse = topk >= 0;
  int32_t* list = sparse ? reinterpret_cast<int32_t*>(ws + lay.list_off) : nullptr;
  int32_t* counts = sparse ? reinterpret_cast<int32_t*>(ws + lay.count_off) : nullptr;

  mark(ev, 0, stream);
  if (sparse) {
    int2* table = reinterpret_cast<int2*>(ws + lay.table_off);
    if (max_seqlen <= kBitmapPositions)
      topk_bitmap_kernel<<<batch, 256, static_cast<size_t>((max_seqlen + 31) / 32) * sizeof(uint32_t), stream>>>(
          topk_indices, topk, seqlens, max_seqlen, list, counts);
    else if (topk <= kTopkLdsEntries)
      topk_compact_kernel<true><<<batch, 256, static_cast<size_t>(lay.topk_slots) * sizeof(int2), stream>>>(
          topk_indices, topk, seqlens, max_seqlen, lay.topk_slots, table, list, counts);
    else
      topk_compact_kernel<false><<<batch, 256, 0, stream>>>(topk_indices, topk, seqlens, max_seqlen, lay.topk_slots,
                                                            table, list, counts);
  }
  // the run plan covers the attended rows: L_b per sequence, or the count of its top-k positions
  if (batch >= kAbsWideFrom)
    absorb_plan_kernel<128><<<dim3(n_heads, 1 + kKvLora / 128), 256, 0, stream>>>(
        q, wkv_b, batch, n_heads, q_lat, sparse ? counts : seqlens, sparse ? topk : max_seqlen, lay.units,
        lay.min_unit_tokens, plan, cum, row_offset, max_seqlen, runs);
  else
    absorb_plan_kernel<64><<<dim3(n_heads, 1 + kKvLora / 64), 256, 0, stream>>>(
        q, wkv_b, batch, n_heads, q_lat, sparse ? counts : seqlens, sparse ? topk : max_seqlen, lay.units,
        lay.min_unit_tokens, plan, cum, row_offset, max_seqlen, runs);
  mark(ev, 1, stream);
  {
    const int n_groups = (n_heads + 63) / 64;
    const int blocks = (lay.units + 7) / 8 * 8 * n_groups;
    if (sparse)
      attend_kernel<true><<<blocks, 512, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen, list, topk,
                                                      plan, cum, runs, batch, n_heads, scale_log2, part_o, part_s, part_l);
    else
      attend_kernel<false><<<blocks, 512, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen, nullptr,
                                                       0, plan, cum, runs, batch, n_heads, scale_log2, part_o, part_s, part_l);
  }
  mark(ev, 2, stream);
  {
    // At most kMergeBlocks blocks, each with its head's W_UV in registers for as many sequence
    // groups as that leaves to it. A single group (16 sequences or fewer) is merged by two blocks
    // per head, each projecting half of the outputs with half of W_UV, so that W_UV is read by more
    // compute units; by four when it holds at most four sequences, whose partials are few (every
    // block of the group merges all of them).
    const int groups = (batch + 15) / 16, per_head = kMergeBlocks / n_heads;
    const int dsplit = groups > 1 ? 1 : (batch <= 4 && per_head >= 4) ? 4 : (per_head >= 2 ? 2 : 1);
    combine_proj_kernel<<<dim3(n_heads, (groups < per_head ? groups : per_head) * dsplit), 512, 0, stream>>>(
        plan, cum, batch, n_heads, part_o, part_s, part_l, wkv_b, dsplit, out, lse);
  }
  mark(ev, 3, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Fixed scratch for decode without a caller workspace. Every GPU the library runs on holds its own
// copy of this array for the life of the process. In host code `scratch` names a host-side stand-in,
// not device memory: the array's device address is looked up per device with hipGetSymbolAddress
// (with that device current) and only that address is handed to kernels.
// ---------------------------------------------------------------------------------------------
namespace {
__device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace mla
