// Mixing kernel: reduce the summary kernel's token-slice partials and mix the per-block
// summaries with the coefficient matrix, S~_i = sum_b m_ib S_b and z~_i = sum_b m_ib z_b
// ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method ->
// Key design 2, multi-head mixing; row i of M_c belongs to query block i).
//
// This VALU kernel serves the fp32-partials path (split accuracy, fp32 inputs) when there are
// too many blocks for the readout to mix in its prologue, and the backward's transposed mixing
// dS_b = sum_i m_ib dS~_i (chain rule of the same step).
//
// Every output element is a fixed-order fp32 sum (deterministic).  The result is written
// in the fragment layout as bf16 (hi) and, for split accuracy, the bf16 residual (lo).
#include "mhla_device.hpp"

namespace mhla {

constexpr int kMixRows = 16;   // query blocks produced per thread

template <bool SPLIT>
__device__ inline void store_hi_lo(uint16_t* hi, uint16_t* lo, int64_t idx, float x) {
  if (SPLIT) {
    uint32_t h, l;
    split_bf16(x, h, l);
    hi[idx] = (uint16_t)h;
    lo[idx] = (uint16_t)l;
  } else {
    hi[idx] = (uint16_t)f32_to_bf16_bits(x);
  }
}

// grid: (ceil((FRAG + D) / 256), ceil(M / kMixRows), BH).  Positions [0, FRAG) are summary
// elements, [FRAG, FRAG + D) the normaliser.
template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void mix_kernel(MixParams p, int frag, int d) {
  const int pos = blockIdx.x * kThreads + threadIdx.x;
  if (pos >= frag + d) return;
  const int i0 = blockIdx.y * kMixRows;
  const int bh = blockIdx.z;
  const int M = p.M;
  const int nrows = min(kMixRows, M - i0);
  const float* mc = p.mc ? p.mc + (int64_t)(bh % p.H) * p.mc_head_stride : nullptr;  // NULL: M == 1
  const bool is_z = pos >= frag;
  const int zpos = pos - frag;

  float acc[kMixRows];
#pragma unroll
  for (int r = 0; r < kMixRows; ++r) acc[r] = 0.f;

  // weight of summary b in output row i: M_c[i][b], or M_c[b][i] for the transposed mixing
  const int64_t si = p.mc_transposed ? 1 : M, sb = p.mc_transposed ? M : 1;
  for (int b = 0; b < M; ++b) {
    float s = 0.f;
    if (is_z) {
      const int64_t slot0 = ((int64_t)bh * M + b) * p.zsplits;
      for (int sp = 0; sp < p.zsplits; ++sp) s += p.pz[(slot0 + sp) * d + zpos];
    } else {
      const int64_t slot0 = ((int64_t)bh * M + b) * p.splits;
      for (int sp = 0; sp < p.splits; ++sp) s += p.ps[(slot0 + sp) * frag + pos];
    }
#pragma unroll
    for (int r = 0; r < kMixRows; ++r)
      if (r < nrows && !(p.causal && b >= i0 + r))
        acc[r] = fmaf(mc ? mc[(int64_t)(i0 + r) * si + b * sb] : 1.0f, s, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kMixRows; ++r) {
    if (r >= nrows) break;
    const int64_t row = (int64_t)bh * M + i0 + r;
    if (is_z)
      p.zt[row * d + zpos] = acc[r];
    else
      store_hi_lo<SPLIT>(p.st_hi, p.st_lo, row * frag + pos, acc[r]);
  }
}

hipError_t launch_mix(const MixParams& p, int d, int frag, int bh, bool split, hipStream_t stream) {
  const dim3 block(kThreads);
  const int nx = (frag + d + kThreads - 1) / kThreads;
  const dim3 grid(nx, (p.M + kMixRows - 1) / kMixRows, bh);
  if (split)
    hipLaunchKernelGGL(mix_kernel<true>, grid, block, 0, stream, p, frag, d);
  else
    hipLaunchKernelGGL(mix_kernel<false>, grid, block, 0, stream, p, frag, d);
  return hipGetLastError();
}

}  // namespace mhla
