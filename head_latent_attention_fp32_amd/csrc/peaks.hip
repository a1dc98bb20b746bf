// Microbenchmarks of the two rates the path is measured against, run in the benchmark's own
// process on the same GPU: a plain streaming read of device memory (the achievable HBM read rate)
// and a loop of independent bf16 MFMAs (the achievable matrix rate at the clock the chip holds
// under that load). Not part of libmla's ABI: built into libmla_peaks.so, which only the
// benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Every thread reads 16-byte chunks at a grid stride and folds them into one word; the word is
// stored only if it equals a value the data never produces, so the loads cannot be removed.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Eight independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave, `iters` rounds. The
// round is one asm block so that the accumulators stay in place (the compiler otherwise shuffles
// them through other registers every round); a chain's next product comes eight products later,
// past the result latency. The values only feed a comparison that keeps the loop alive.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.001f * ((lane + e) & 7));
    b[e] = static_cast<__bf16>(0.5f - 0.001f * ((lane * 3 + e) & 7));
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 c0 = z, c1 = z, c2 = z, c3 = z, c4 = z, c5 = z, c6 = z, c7 = z;
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7\n\t"
        "s_nop 7"
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
        : "v"(a), "v"(b));
  }
  const f32x4 t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  const float s = (t[0] + t[1]) + (t[2] + t[3]);
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) starting at the 16-byte aligned device pointer `buf` once.
int mla_peak_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15)) return 1;
  stream_read_kernel<<<256 * 8, 256, 0, stream>>>(static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// blocks x 4 waves, each issuing 8 * iters MFMAs of 16 x 16 x 32 (16384 flops each).
int mla_peak_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
  if (!sink || blocks <= 0 || iters <= 0) return 1;
  mfma_loop_kernel<<<blocks, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
