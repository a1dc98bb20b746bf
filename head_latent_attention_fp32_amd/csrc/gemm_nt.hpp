// Tiled bf16 product on gfx950 for the projections of the path whose two operands are both stored
// with k contiguous ("NT"): C[m][n] = sum_k X[m][k] W[n][k], X = token rows, W = weight rows
// (output features), fp32 accumulation on MFMA.
//
// Block tile 256 tokens x 256 features, 8 waves as 2 (tokens) x 4 (features), 128 x 64 each; k in
// steps of 64 through two LDS stages (64 KB each: 256 weight rows, then 256 token rows of 128 B)
// filled by 16-byte direct-to-LDS buffer loads, the next step's loads in flight during this step's
// MFMAs; one barrier per step. Rows past either operand's end read as zeros (descriptor range).
// Only waves 0-3 (one per SIMD) issue the loads, so that on every SIMD one wave's MFMAs run while
// the other waits for the address unit to take its loads.
// Stage rows: 16-byte chunk c of row r at c ^ ((r >> 1) & 7), so every 128-bit operand read
// (16 rows, 4 chunks) is free of LDS bank conflicts.
// Per wave and k-step: 4 weight and 8 token operands (ds_read_b128), 32 MFMA 16x16x32.
// Orientation: normally the weight row is the MFMA A operand, so a lane ends with four consecutive
// features of one token; an epilogue may ask a wave for the transposed product instead (token as A:
// four consecutive tokens of one feature), chosen per wave.
// Weights stored input x output instead (kWkn: W[k][n], n contiguous, row pitch w_pitch elements):
// the weight part of a stage is [64 k][256 n], 512-byte rows whose 32-byte column group g sits at
// g ^ wswz(k), wswz(k) = (k & 3) | ((k >> 1) & 4) (the 8 rows of a half-wave's transposing read, two
// groups of 4 consecutive rows, then hit 8 distinct 32-byte bank groups), and the A operand (16
// features x 8 consecutive k) comes from two ds_read_b64_tr_b16. Normal orientation only; the
// tile's 256 features must all exist.
// Weights stored input x output in 32-column groups instead (kWkn and kPacked: group g = columns
// 32 g .. 32 g + 31, its K rows of 64 bytes back to back, groups one after another; see
// packed_lane_off): the same LDS image, filled from the group runs.
#pragma once

#include <type_traits>

#include "mla_common.hpp"

namespace mla {
namespace gemm {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;              // 64 KB
constexpr int kIssuers = 4;                                     // waves 0-3 issue the loads
constexpr int kLoadsPerWave = kStageBytes / 1024 / kIssuers;    // 16 loads of 1 KB per issuing wave and step
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int wswz(int k) { return (k & 3) | ((k >> 1) & 4); }

// Packed input x output weights: [n / 32][K][32]. Byte offset, from the start of the group that
// holds column n0 (n0 a multiple of 32), of the 16 bytes at row k, columns n0 + 8 c .. n0 + 8 c + 7.
constexpr int kPackCols = 32;
__device__ __forceinline__ uint32_t packed_lane_off(int K, int k, int c) {
  return static_cast<uint32_t>((c >> 2) * K * (kPackCols * 2) + k * (kPackCols * 2) + (c & 3) * 16);
}

template <class E, class = void>
struct staged_epi : std::false_type {};
template <class E>
struct staged_epi<E, std::void_t<decltype(E::kStaged)>> : std::bool_constant<E::kStaged> {};

// One block tile: features [n0, n0 + 256) of W (w_rows rows in all), tokens [m0, m0 + 256) of X
// (x_rows rows), k in [k_begin, k_begin + k_len) (k_len a multiple of 64; rows are K elements).
// At the end calls, per wave and 16 x 16 sub-tile,
//   epi.store(m, n, v, false)  v = C[m][n .. n+3]      (normal orientation), or
//   epi.store(m, n, v, true)   v = C[m .. m+3][n]      (when epi.transposed(wn) for the wave)
// for tokens m < x_rows and features n < w_rows only. An epilogue with kStaged = true may instead
// take the whole tile through LDS when epi.can_stage() holds (the same for the whole block): after
// the last step's reads, epi.stage_store(lds, ml, nl, v, tr) with tile-local ml, nl, a barrier, then
// epi.copy_out(lds) by all threads; `stage` must then hold what the epilogue stages.
template <bool kWkn = false, bool kPacked = false, class Epi>
__device__ __forceinline__ void nt_tile(const uint16_t* __restrict__ w, int64_t w_rows, const uint16_t* __restrict__ x,
                                        int64_t x_rows, int K, int n0, int64_t m0, int k_begin, int k_len,
                                        uint8_t* stage, const Epi& epi, int w_pitch = 0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, grp = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;

  // Loads: instruction d (0..63) of a step covers 8 rows x 128 B: d < 32 weight rows 8d.., else
  // token rows 8(d-32)..; wave w < 4 issues d = w + 4e, waves 4-7 none. Waves w and w + 4 share a
  // SIMD, so while one stalls issuing loads (the address unit takes a step's 64 KB at 64 B per
  // clock) the other's MFMAs keep the matrix pipe busy. Lane l: row 8d' + l/8, physical chunk l%8
  // holding logical chunk (l%8) ^ swz(row).
  const bool issuer = wave < kIssuers;
  // (kWkn: weight instruction d < 32 covers k rows 2d, 2d + 1 of 512 B; lane l: row 2d + l/32,
  // physical 16-byte chunk l%32, i.e. 32-byte group (l%32)/2 holding logical group that ^ wswz(row))
  uint32_t voff[kLoadsPerWave];
#pragma unroll
  for (int e = 0; e < kLoadsPerWave; ++e) {
    const int d = (wave & (kIssuers - 1)) + kIssuers * e;
    if (kWkn && d < 32) {
      const int row = 2 * d + (lane >> 5), pc = lane & 31;
      const int lc = (((pc >> 1) ^ wswz(row)) << 1) | (pc & 1);
      voff[e] = kPacked ? packed_lane_off(K, row, lc) : static_cast<uint32_t>(row * w_pitch * 2 + lc * 16);
    } else {
      const int row = 8 * (d & 31) + (lane >> 3);
      voff[e] = static_cast<uint32_t>(row * K * 2 + (((lane & 7) ^ swz(row)) << 4));
    }
  }
  const uint32_t st_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)stage));
  // Descriptor ranges: the rows this tile reads (at most 256 of each operand; rows past an operand's
  // end read as zeros), so that the 32-bit byte ranges stay below 4 GiB for any operand size
  // (256 rows x K x 2 B; K <= 16384 here).
  // (kWkn: the K rows of the tile's 256 columns, K x w_pitch x 2 bytes from column n0; packed:
  // the tile's eight column groups)
  const int64_t w_left = w_rows - n0, x_left = x_rows - m0;
  const uint32_t w_bytes =
      kWkn ? (kPacked ? static_cast<uint32_t>(K) * (kBN * 2)
                      : static_cast<uint32_t>(static_cast<int64_t>(K) * w_pitch * 2 - static_cast<int64_t>(n0) * 2))
           : static_cast<uint32_t>((w_left < kBN ? w_left : kBN) * K * 2);
  const uint16_t* w_tile = kWkn ? (kPacked ? w + static_cast<int64_t>(n0) * K : w + n0) : w + static_cast<int64_t>(n0) * K;
  const uint32_t x_bytes = static_cast<uint32_t>((x_left < kBM ? x_left : kBM) * K * 2);
  auto issue = [&](int kt) {
    if (!issuer) return;
    // descriptors rebuilt per step (scalar work): short-lived, they stay in SGPRs
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_tile, w_bytes);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + m0 * K, x_bytes);
    const uint32_t koff = static_cast<uint32_t>(k_begin + kt * kBK) * 2u;
    const uint32_t wkoff = !kWkn ? koff
                           : kPacked ? static_cast<uint32_t>(k_begin + kt * kBK) * (kPackCols * 2u)
                                     : static_cast<uint32_t>(k_begin + kt * kBK) * static_cast<uint32_t>(w_pitch) * 2u;
    const uint32_t dst = st_lds + (kt & 1) * kStageBytes;
#pragma unroll
    for (int e = 0; e < kLoadsPerWave; ++e) {
      const int d = wave + kIssuers * e;
      if (d < 32) dma16(rw, dst + d * 1024, voff[e] + wkoff);
      else dma16(rx, dst + d * 1024, voff[e] + koff);
    }
  };

  // operand offsets in a stage: weight row 64 wn + 16 nb + r, token row 128 wm + 16 mb + r;
  // chunk 4 ks + grp (+ 16 nb / 16 mb rows keep swz)
  int a_off[2], b_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ra = 64 * wn + r, rb = 128 * wm + r;
    a_off[ks] = ra * 128 + (((4 * ks + grp) ^ swz(ra)) << 4);
    b_off[ks] = kBN * 128 + rb * 128 + (((4 * ks + grp) ^ swz(rb)) << 4);
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool tr = epi.transposed(wn);
  auto run = [&](auto transposed) {
    constexpr bool T = decltype(transposed)::value;
    const int n_kt = k_len / kBK;
    issue(0);
    for (int kt = 0; kt < n_kt; ++kt) {
      __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));   // vmcnt(0): this wave's loads of kt
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();                                // all loads of kt; stage kt-1 free
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (kt + 1 < n_kt) issue(kt + 1);
      const uint8_t* st = stage + (kt & 1) * kStageBytes;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[4], bf[8];
        if constexpr (kWkn) {
          // k rows 32 ks + 8 grp + 4 h + r/4, features 16 (4 wn + nb) + 4 (r%4) .. +3
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            i16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int row = 32 * ks + 8 * grp + 4 * h + (r >> 2);
              const int byte = row * 512 + (((4 * wn + nb) ^ wswz(row)) << 5) + 8 * (r & 3);
              half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(st + byte));
            }
            af[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) af[nb] = *reinterpret_cast<const bf16x8*>(st + a_off[ks] + nb * 16 * 128);
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) bf[mb] = *reinterpret_cast<const bf16x8*>(st + b_off[ks] + mb * 16 * 128);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int mb = 0; mb < 8; ++mb)
            acc[nb][mb] = T ? mfma16x16x32(bf[mb], af[nb], acc[nb][mb]) : mfma16x16x32(af[nb], bf[mb], acc[nb][mb]);
      }
    }
  };
  if (tr) run(std::true_type{});
  else run(std::false_type{});

  if constexpr (staged_epi<Epi>::value) {
    if (epi.can_stage()) {
      __syncthreads();   // every wave's operand reads of the last stage are done
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          if (!tr) epi.stage_store(stage, 128 * wm + 16 * mb + r, 64 * wn + 16 * nb + 4 * grp, acc[nb][mb], false);
          else epi.stage_store(stage, 128 * wm + 16 * mb + 4 * grp, 64 * wn + 16 * nb + r, acc[nb][mb], true);
        }
      __syncthreads();
      epi.copy_out(stage);
      return;
    }
  }

#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      if (!tr) {
        // C[m][n .. n+3]: m = m0 + 128 wm + 16 mb + r, n = n0 + 64 wn + 16 nb + 4 grp
        const int64_t m = m0 + 128 * wm + 16 * mb + r;
        const int n = n0 + 64 * wn + 16 * nb + 4 * grp;
        if (m < x_rows && n < w_rows) epi.store(m, n, acc[nb][mb], false);
      } else {
        // C[m .. m+3][n]: m = m0 + 128 wm + 16 mb + 4 grp, n = n0 + 64 wn + 16 nb + r
        const int64_t m = m0 + 128 * wm + 16 * mb + 4 * grp;
        const int n = n0 + 64 * wn + 16 * nb + r;
        if (m < x_rows && n < w_rows) epi.store(m, n, acc[nb][mb], true);
      }
    }
}

}  // namespace gemm
}  // namespace mla
