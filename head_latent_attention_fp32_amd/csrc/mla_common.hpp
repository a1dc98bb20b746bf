// Device-side helpers shared by the MLA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Model widths the kernels are built for (DeepSeek-V3.2-Exp / Kimi-K2 attention).
constexpr int kQLora = 1536;   // query latent width
constexpr int kKvLora = 512;   // cached latent width
constexpr int kNope = 128;     // per-head content features of q and k
constexpr int kRope = 64;      // rotary features (32 pairs), shared rotary key
constexpr int kVDim = 128;     // per-head value features
constexpr int kQk = kNope + kRope;          // 192 features per query head
constexpr int kKvRows = kNope + kVDim;      // 256 rows of wkv_b per head
constexpr int kLat = kKvLora + kRope;       // 576 features of one cached row (latent | rotary key)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16). Lane l holds A row l%16 and B column l%16,
// eight consecutive k of group l/16 each; D column l%16, rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float round_bf16(float f) {
  return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// Two fp32 -> one packed bf16 pair, round-to-nearest-even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 as_uint4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint16_t u4_elem(const uint4& v, int e) {
  const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__device__ __forceinline__ bf16x8 bf16x8_from_f32(const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(u);
}

// Sum, in fp32, of the eight bf16 values of v (v_dot2 against ones, two chains): softmax weights
// that enter an MFMA rounded to bf16 can be normalised by the sum of exactly those rounded values,
// so that their rounding perturbs the weights' shape but not their total.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, 0.f, false);
  float s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, 0.f, false);
  s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, s0, false);
  s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, s1, false);
  return s0 + s1;
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// D(16x16, fp32) += A(16x32, f16) * B(32x16, f16), same lane layout as the bf16 form.
__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two fp32 -> one packed f16 pair, round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
// One packed f16 pair -> two fp32 (exact).
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t u) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
}

__device__ __forceinline__ f16x8 f16x8_from_f32(const float* v) {
  uint4 u;
  u.x = pack_f16x2(v[0], v[1]);
  u.y = pack_f16x2(v[2], v[3]);
  u.z = pack_f16x2(v[4], v[5]);
  u.w = pack_f16x2(v[6], v[7]);
  return __builtin_bit_cast(f16x8, u);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48): the k-groups
// of an MFMA operand / the row groups of its 16x16 result. v_permlane16_swap / v_permlane32_swap
// exchange rows between two registers; called with the same value twice, the two results hold
// each lane's own value and that of lane l^16 (l^32) in some order.
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (v_exp_f32): no range reduction around it, so results below
// 2^-126 flush to zero -- for softmax weights, which are at most 2^16 here (2^8 in the prefill),
// that is far below bf16's resolution of any sum they enter. 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------------
// Buffer loads straight into LDS, and the barriers around them.
// ---------------------------------------------------------------------------------------------
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;

// LDS byte address of a __shared__ object (the M0 operand of a direct-to-LDS load).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// Raw buffer descriptor over [base, base + bytes) built from wave-uniform values (so that it
// lives in SGPRs); loads beyond the range return zeros. Callers size `bytes` to what the loads
// that use the descriptor may reach, so that it never wraps.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           kRsrcWord3);
}

// 16-byte direct-to-LDS buffer load: lane l's 16 bytes at rsrc + voff land at LDS byte address
// lds_addr + 16 l. Issued from an asm block: the compiler cannot tell which LDS stage such a load
// writes and would otherwise wait for every load in flight before any LDS read. Completion is
// tracked with explicit vmcnt waits and barriers. The block writes no registers.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also orders global memory,
// which waits for every vector-memory load in flight -- the next stages' loads among them. The
// explicit lgkmcnt(0) (an asm block, which the compiler's wait insertion cannot relax) makes every
// LDS access this wave issued complete before it reaches the barrier: the release fence alone, and
// the same wait as a builtin, were seen compiled to a wait after the barrier on a path whose last
// LDS stores came from a branch, so that another wave could read before they landed.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace mla
