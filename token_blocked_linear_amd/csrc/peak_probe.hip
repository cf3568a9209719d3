// Measured-peak probes for the benchmark's roofline context (not part of the MHLA path):
//   - a loop of dense bf16 MFMAs (v_mfma_f32_16x16x32_bf16, 16384 flops per wave and
//     instruction) on register operands, eight independent accumulator chains per wave, no
//     memory traffic in the loop;
//   - streaming HBM probes: a read (non-temporal 16-byte buffer loads, the policy the kernels
//     use for data they stream once), a write (default-policy 16-byte stores) and a copy, each
//     workgroup covering 64 KiB with four 16-byte accesses per thread in flight.
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

// kind 0: read `bytes` of src; 1: write `bytes` of dst; 2: copy src -> dst.  Workgroup w covers
// bytes [w * 64 KiB, (w + 1) * 64 KiB) through buffer resources (accesses past the end are
// dropped by the resource's range).  The read keeps an xor of what it loaded and stores it only
// when it equals a value that the all-ones probe data never produces.
__global__ __launch_bounds__(kThreads) void stream_kernel(const char* src, char* dst, uint64_t bytes, int kind,
                                                          uint32_t* sink) {
  constexpr uint32_t kChunk = 64u << 10;
  const uint64_t base = (uint64_t)blockIdx.x * kChunk;
  const uint32_t n = (uint32_t)(bytes - base < kChunk ? bytes - base : kChunk);
  const Rsrc rs = make_rsrc(src ? src + base : nullptr, src ? n : 0u);
  const Rsrc rd = make_rsrc(dst ? dst + base : nullptr, dst ? n : 0u);
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const u32x4_t val = {0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
  for (uint32_t off = threadIdx.x * 16u; off < kChunk; off += 4u * kThreads * 16u) {
    if (kind == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) buf_st16(rd, off + j * kThreads * 16u, val);
    } else {
      u32x4_t x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = buf_ld16<2>(rs, off + j * kThreads * 16u);
      if (kind == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) buf_st16(rd, off + j * kThreads * 16u, x[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= x[j];
      }
    }
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (kind == 0 && x == 0x12345678u) sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

}  // namespace mhla

// Streaming probe over `bytes` (a multiple of 64 KiB, at most 2^40): kind 0 reads src, 1 writes
// dst, 2 copies src to dst; `sink` holds bytes / 64 KiB * 256 words (never written in practice
// for the all-ones data the benchmark passes).  Returns a hipError_t.
extern "C" int mhla_peak_stream(int kind, const void* src, void* dst, uint64_t bytes, uint32_t* sink, void* stream) {
  if (kind < 0 || kind > 2 || bytes == 0 || bytes % (64u << 10) != 0 || bytes > ((uint64_t)1 << 40))
    return (int)hipErrorInvalidValue;
  if ((kind != 1 && !src) || (kind != 0 && !dst) || !sink) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mhla::stream_kernel, dim3((unsigned)(bytes / (64u << 10))), dim3(mhla::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const char*>(src), static_cast<char*>(dst),
                     bytes, kind, sink);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads, each wave issuing 8 * iters MFMAs; `out` holds
// blocks * 256 floats (never written in practice).  Returns a hipError_t.
extern "C" int mhla_peak_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mhla::mfma_peak_kernel, dim3((unsigned)blocks), dim3(mhla::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}
