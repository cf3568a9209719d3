// Measured-peak probe for the benchmark's roofline context (not part of the MHLA path): a loop of
// dense bf16 MFMAs (v_mfma_f32_16x16x32_bf16, 16384 flops per wave and instruction) on register
// operands, eight independent accumulator chains per wave, no memory traffic in the loop.
#include "mhla_device.hpp"

namespace mhla {

__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(float* out, int iters) {
  const uint32_t t = threadIdx.x;
  const u32x4_t a = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};          // 1.0
  // a different B operand per chain (~2^-10, low mantissa bits from the chain and the lane), so
  // that no two chains compute the same values; eight named accumulators
  auto bop = [&](uint32_t j) {
    const uint32_t w = 0x3a803a80u | j | ((t & 7u) << 3);
    return u32x4_t{w, w, w, w};
  };
  const u32x4_t b0 = bop(0), b1 = bop(1), b2 = bop(2), b3 = bop(3), b4 = bop(4), b5 = bop(5), b6 = bop(6), b7 = bop(7);
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  // each accumulator stays in its own registers (the compiler's allocation of eight loop-carried
  // MFMA accumulators copies them through a shared tuple every iteration)
#define MHLA_PEAK_MFMA(C, B) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(C) : "v"(a), "v"(B))
  for (int i = 0; i < iters; ++i) {
    MHLA_PEAK_MFMA(c0, b0);
    MHLA_PEAK_MFMA(c1, b1);
    MHLA_PEAK_MFMA(c2, b2);
    MHLA_PEAK_MFMA(c3, b3);
    MHLA_PEAK_MFMA(c4, b4);
    MHLA_PEAK_MFMA(c5, b5);
    MHLA_PEAK_MFMA(c6, b6);
    MHLA_PEAK_MFMA(c7, b7);
  }
#undef MHLA_PEAK_MFMA
  // the compiler sees no MFMA in the asm, so it inserts no wait states before the VALU reads of
  // the accumulators below: give them explicitly (more than any MFMA-to-VALU hazard needs)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4_t c[8] = {c0, c1, c2, c3, c4, c5, c6, c7};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
  // the sums are positive, so the store never happens; it keeps the chains from being removed
  if (s < -1.0f) out[(int64_t)blockIdx.x * kThreads + t] = s;
}

}  // namespace mhla

// `blocks` workgroups of 256 threads, each wave issuing 8 * iters MFMAs; `out` holds
// blocks * 256 floats (never written in practice).  Returns a hipError_t.
extern "C" int mhla_peak_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mhla::mfma_peak_kernel, dim3((unsigned)blocks), dim3(mhla::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}
