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
// 2. Split-KV attention over runs.
//
//    Block = NW waves, H = 16 NW heads. Cached rows stream through an NSTAGE-deep ring of 32-row
//    LDS tiles filled by 16-byte direct-to-LDS buffer loads (the descriptor's range check
//    zero-fills rows past the end of the sequence), so every row is read from HBM once.
//    Per tile:
//      scores:  wave w holds the query of heads 16w .. 16w+15 (absorbed latent and rotary part,
//               576 features) in VGPRs and computes S^T[t][h] = sum_k tile[t][k] q[h][k] on MFMA
//               (A operand: ds_read_b128 of tile rows), the per-head maximum and P = 2^(s - m),
//               which it writes to a small LDS buffer;
//      values:  wave w owns latent columns [512 w / NW, 512 (w+1) / NW) of every head and adds
//               O^T[c][h] += sum_t tile[t][c] P^T[t][h] (A operand: ds_read_b64_tr_b16, the
//               transposing LDS read, of tile columns; B operand: ds_read_b128 of P).
//    So a wave holds 72 registers of query and 128 of accumulators whatever H is.
//    P^T comes out of the S^T accumulators with lane l holding tokens 4(l/16)+{0..3} and
//    16+4(l/16)+{0..3} of head l%16 -- its k-group of the P.V product -- and is stored per head
//    in that order; V^T is read in the same token order.
//    LDS tile: latent part [32 rows][1024 B] whose 16-byte chunk c of row r sits at c ^ fk(r),
//    fk(r) = 2(r&7) + ((r>>3)&1); rotary part [32 rows][128 B] with chunk c at c ^ ((r>>1)&7);
//    P rows of 80 B. Then 16 rows read at one chunk, and 8 consecutive rows read at two adjacent
//    chunks, touch 16 distinct 16-byte bank groups.
//    Softmax: per head a reference m (log2 units, scale folded in) that moves only when a tile's
//    maximum exceeds it by more than 8 -- then every wave rescales its accumulators and l by the
//    factor each head publishes in LDS -- so p = 2^(s - m) <= 2^8.
// ---------------------------------------------------------------------------------------------
constexpr int kKvBytes = kTileTok * kKvLora * 2;           // 32768
constexpr int kPeBytes = kTileTok * kRope * 2;             // 4096
constexpr int kTileBytes = kKvBytes + kPeBytes;            // 36864
constexpr int kTileLoads = kTileBytes / 1024;              // 36 loads of 64 lanes x 16 B
constexpr int kPStride = kTileTok * 2 + 16;                // bytes per head row of P
constexpr uint32_t kRsrcWord3 = 0x00020000u;               // raw buffer, 32-bit data format

__device__ __forceinline__ int fk(int row) { return 2 * (row & 7) + ((row >> 3) & 1); }
__device__ __forceinline__ int fp(int row) { return (row >> 1) & 7; }

// Workgroup barrier that orders LDS accesses only. __syncthreads() also orders global memory,
// which waits for every vector-memory load in flight -- here, the next tiles' loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `tiles_after` tiles of loads (of `L` loads each) are still in flight.
template <int L>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  if (tiles_after >= 3) wait_vm<3 * L>();
  else if (tiles_after == 2) wait_vm<2 * L>();
  else if (tiles_after == 1) wait_vm<L>();
  else wait_vm<0>();
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;

// Raw buffer descriptor over [base, base + bytes) built from wave-uniform values (so that it
// lives in SGPRs); loads beyond the range return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// 16-byte direct-to-LDS buffer load: lane l's 16 bytes at rsrc + voff land at LDS byte offset
// dst + 16 l. Issued from an asm block: the compiler cannot tell which ring stage such a load
// writes and would otherwise wait for every load in flight before any LDS read. Completion is
// tracked with explicit vmcnt waits and barriers. The block writes no registers.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, const uint8_t* dst, uint32_t voff) {
  const uint32_t d = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)dst));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(d)
               : "memory");
}
template <int NW, int NSTAGE>
__global__ __launch_bounds__(NW * 64, 1) void attend_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ pe, const int64_t* __restrict__ row_offset, int64_t max_seqlen,
    const Plan* __restrict__ plan, const int64_t* __restrict__ cum, int batch, int n_heads, float scale_log2,
    float* __restrict__ part_o, float* __restrict__ part_l) {
  // A block attends H = 16 NW heads: head group hg covers heads [H hg, H hg + H); slots past
  // n_heads (fewer heads than H) run on a zero query and are never stored. The blocks of the
  // head groups of one run share blockIdx mod 8 -- the same XCD and its L2 -- and are dispatched
  // next to each other, so the tiles one of them pulls from HBM are L2 hits for the others.
  constexpr int H = 16 * NW;
  constexpr int CB = 32 / NW;                              // 16-column blocks of the latent per wave
  constexpr int LMAX = (kTileLoads + NW - 1) / NW;         // loads per wave per tile (first waves)
  constexpr int LMIN = kTileLoads / NW;
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "pipeline depth");

  const int64_t N = plan->total_tokens;
  const int64_t G = plan->runs;
  const int n_groups = (n_heads + H - 1) / H;
  const int hg = (blockIdx.x >> 3) % n_groups;
  const int64_t g = (blockIdx.x & 7) + 8 * (blockIdx.x / (8 * n_groups));
  if (g >= G) return;
  const int head0 = hg * H;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[H * kPStride];
  __shared__ float alpha_s[H];
  __shared__ int flag_s[NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets wave-derived values live in SGPRs
  const int r = lane & 15, grp = lane >> 4;
  const int my_loads = (kTileLoads - wave + NW - 1) / NW;  // loads j = wave + NW k of each tile
  const int c_wave = wave * CB;                            // first 16-column block of this wave

  int64_t start = run_start(g, N, G);
  const int64_t end = run_start(g + 1, N, G);
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid + 1] > start) hi = mid; else lo = mid + 1;
  }
  int b = lo;

  while (start < end) {
    const int64_t seq0 = cum[b];
    const int64_t seg_end = min(end, cum[b + 1]);
    const int t0 = static_cast<int>(start - seq0), t1 = static_cast<int>(seg_end - seq0);
    const int64_t base_row = row_offset ? row_offset[b] : static_cast<int64_t>(b) * max_seqlen;
    const int n_tiles = (t1 - t0 + kTileTok - 1) / kTileTok;
    // Descriptors over rows [0, t1) of this sequence: loads of later rows return zeros.
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv + base_row * kKvLora, t1 * (kKvLora * 2));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(pe + base_row * kRope, t1 * (kRope * 2));

    bf16x8 qf[18];
    {
      const int head = head0 + wave * 16 + r;
      const bool real = head < n_heads;
      const int hq = real ? head : 0;
      const uint16_t* ql = q_lat + (static_cast<int64_t>(b) * n_heads + hq) * kKvLora + grp * 8;
      const uint16_t* qp = q + (static_cast<int64_t>(b) * n_heads + hq) * kQk + kNope + grp * 8;
      const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = as_bf16x8(real ? ldg16(ql + ks * 32) : z);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) qf[16 + ks] = as_bf16x8(real ? ldg16(qp + ks * 32) : z);
    }

    // Load j of a tile fills latent row j (j < 32; lane = physical chunk) or rotary rows
    // 8 (j - 32) .. +7 (lane = 8 rows x 8 physical chunks); this wave issues j = wave + NW k.
    auto issue = [&](int tile) {
      const int tt0 = t0 + tile * kTileTok;
      uint8_t* dst = lds + (tile % NSTAGE) * kTileBytes;
#pragma unroll
      for (int k = 0; k < LMAX; ++k) {
        const int j = wave + NW * k;
        if (j < kTileLoads) {
          if (j < kTileTok) {
            const uint32_t voff = static_cast<uint32_t>(tt0 + j) * (kKvLora * 2) + ((lane ^ fk(j)) << 4);
            dma16(rk, dst + j * 1024, voff);
          } else {
            const int row = 8 * (j - kTileTok) + (lane >> 3);
            const uint32_t voff =
                static_cast<uint32_t>(tt0 + row) * (kRope * 2) + (((lane & 7) ^ fp(row)) << 4);
            dma16(rp, dst + kKvBytes + (j - kTileTok) * 1024, voff);
          }
        }
      }
    };

    float m_ref = -INFINITY, lsum = 0.f;       // of head 16 wave + r
    f32x4 o[CB][NW];                           // O^T[16 (c_wave + cb) + 4 grp + j][16 hb + r]
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) o[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};

    int issued = 0;
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
      if (issued < n_tiles) issue(issued++);

    f32x4 s[2];
    float mx = 0.f;
    // Wait for tile it, make it visible, start the next loads, S^T and its masked maximum.
    auto scores = [&](int it) {
      const int after = issued - 1 - it;
      if (my_loads == LMAX) wait_tiles<LMAX>(after); else wait_tiles<LMIN>(after);
      lds_barrier();
      if (issued < n_tiles) issue(issued++);
      const uint8_t* tile = lds + (it % NSTAGE) * kTileBytes;
      // Per-lane operand offsets, recomputed per tile from an opaque copy of the lane id (cheaper
      // than keeping them live through the loop). S^T latent k-steps: row tb*16 + r, logical chunk
      // 4 ks + grp; rotary k-steps 16, 17: row tb*16 + r, logical chunk 4 (ks-16) + grp.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int lr = ln & 15, lg = ln >> 4;
      const int sf = fk(lr);
      const int s_lane = lr * 1024 + ((lg ^ sf) & 3) * 16;
      const int s_flip = sf >> 2;
      const int p_off0 = kKvBytes + lr * 128 + ((lg ^ fp(lr)) * 16);
      const int p_off1 = kKvBytes + lr * 128 + (((4 + lg) ^ fp(lr)) * 16);
      s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto rd = [&](int tb, int ks) {
        const uint8_t* p = ks < 16 ? tile + tb * 16 * 1024 + s_lane + 64 * ((ks & ~3) + ((ks & 3) ^ s_flip))
                                   : tile + tb * 16 * 128 + (ks == 16 ? p_off0 : p_off1);
        return *reinterpret_cast<const bf16x8*>(p);
      };
      // Operand reads run kAhead k-steps ahead of the MFMAs (both 16-token halves per step).
      constexpr int kAhead = 4;
      bf16x8 fa[kAhead][2];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) {
        fa[ks][0] = rd(0, ks);
        fa[ks][1] = rd(1, ks);
      }
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const bf16x8 a0 = fa[ks % kAhead][0], a1 = fa[ks % kAhead][1];
        if (ks + kAhead < 18) {
          fa[ks % kAhead][0] = rd(0, ks + kAhead);
          fa[ks % kAhead][1] = rd(1, ks + kAhead);
        }
        s[0] = mfma16x16x32(a0, qf[ks], s[0]);
        s[1] = mfma16x16x32(a1, qf[ks], s[1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int valid = t1 - (t0 + it * kTileTok);
      float m = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (tb * 16 + grp * 4 + j >= valid) s[tb][j] = -INFINITY;
          m = fmaxf(m, s[tb][j]);
        }
      mx = max_over_rows(m) * scale_log2;
    };

    // P = 2^(s - m) into l and the LDS buffer (tokens in k-group order), then the barrier that
    // publishes P, the rescale factors and the flags.
    auto publish = [&]() {
      float p[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[tb * 4 + j] = exp2f(s[tb][j] * scale_log2 - m_ref);
          lsum += p[tb * 4 + j];
        }
      *reinterpret_cast<bf16x8*>(pbuf + (wave * 16 + r) * kPStride + grp * 16) = bf16x8_from_f32(p);
      lds_barrier();
    };

    // O^T += V^T P^T for this wave's latent columns and all heads.
    auto values = [&](int it) {
      const uint8_t* tile = lds + (it % NSTAGE) * kTileBytes;
      // V^T: source row 4 grp + (r>>2) (+16), logical chunk 2 cb + ((r&3)>>1), byte (r&1)*8.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int lr = ln & 15, lg = ln >> 4;
      const int vrow = 4 * lg + (lr >> 2);
      const int vf = fk(vrow);
      const int v_lane = vrow * 1024 + ((((lr & 3) >> 1) ^ (vf & 1)) * 16) + (lr & 1) * 8;
      const int v_flip = vf >> 1;
      auto rdv = [&](int cb) {
        const int c = c_wave + cb;
        const uint8_t* v0 = tile + v_lane + 32 * ((c & ~7) + ((c & 7) ^ v_flip));
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(v0));
        const i16x4 hi4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(v0 + 16 * 1024));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      auto rdp = [&](int hb) { return *reinterpret_cast<const bf16x8*>(pbuf + (hb * 16 + r) * kPStride + grp * 16); };
      if constexpr (CB <= 8) {
        // the wave's V^T fragments and all P fragments are read up front, each once
        bf16x8 vf[CB], pf[NW];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) vf[cb] = rdv(cb);
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) pf[hb] = rdp(hb);
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) o[cb][hb] = mfma16x16x32(vf[cb], pf[hb], o[cb][hb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8 a = rdv(cb);
#pragma unroll
          for (int hb = 0; hb < NW; ++hb) o[cb][hb] = mfma16x16x32(a, rdp(hb), o[cb][hb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // The first tile sets the reference (O and l are still zero).
    scores(0);
    m_ref = mx;
    publish();
    values(0);
    int it = 1;
    while (it < n_tiles) {
      // Tiles whose maximum stays within 2^8 of the reference of every head: the accumulators are
      // only ever updated by MFMAs in this loop.
      bool rescale = false;
      for (; it < n_tiles; ++it) {
        scores(it);
        const bool up = __any(mx > m_ref + 8.f) != 0;
        if (up) {
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = exp2f(m_ref - m_new);
          m_ref = m_new;
          lsum *= alpha;
          if (grp == 0) alpha_s[wave * 16 + r] = alpha;
        }
        if (lane == 0) flag_s[wave] = up ? 1 : 0;
        publish();
#pragma unroll
        for (int w = 0; w < NW; ++w) rescale |= flag_s[w] != 0;
        if (rescale) break;
        values(it);
      }
      if (!rescale) break;
      // Some head moved its reference: scale every accumulator by its head's factor.
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) {
        const bool moved = flag_s[hb] != 0;
        const float a = moved ? alpha_s[hb * 16 + r] : 1.f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][hb] *= a;
      }
      values(it);
      ++it;
    }

    // Final normalisation: every wave needs l of all heads; publish them through alpha_s.
    const float ltot = sum_over_rows(lsum);
    lds_barrier();
    if (grp == 0) alpha_s[wave * 16 + r] = ltot;
    lds_barrier();
    const int64_t slot = g + b;
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      if (head0 + hb * 16 < n_heads) {
        const float inv = 1.f / alpha_s[hb * 16 + r];
        float* po = part_o + (slot * n_heads + head0 + hb * 16 + r) * kKvLora + c_wave * 16 + grp * 4;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const f32x4 v = o[cb][hb] * inv;
          *reinterpret_cast<float4*>(po + cb * 16) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    if (grp == 0 && head0 + wave * 16 < n_heads)
      part_l[slot * n_heads + head0 + wave * 16 + r] = (m_ref + __log2f(ltot)) * kLn2;
    lds_barrier();   // alpha_s / pbuf / ring are reused by the next segment

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
  // one block per compute unit: 256 CUs, shared by the head groups of a run
  const int64_t max_units = 256 / ((n_heads + 63) / 64);
  units = units < 1 ? 1 : (units > max_units ? max_units : units);
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
  {
    const int n_groups = (n_heads + 63) / 64;
    const int blocks = (lay.units + 7) / 8 * 8 * n_groups;
    attend_kernel<4, 4><<<blocks, 256, 0, stream>>>(q_lat, q, kv_cache, pe_cache, row_offset, max_seqlen, plan, cum,
                                                    batch, n_heads, scale_log2, part_o, part_l);
  }
  mark(ev, 2, stream);
  combine_kernel<<<dim3(batch, n_heads / 16), 256, 0, stream>>>(plan, cum, n_heads, part_o, part_l, o_lat, lse);
  mark(ev, 3, stream);
  value_proj_kernel<<<dim3(n_heads, kVDim / 64), 256, 0, stream>>>(o_lat, wkv_b, batch, n_heads, out);
  mark(ev, 4, stream);
  return hipGetLastError();
}

}  // namespace mla
