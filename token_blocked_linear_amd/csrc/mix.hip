// Mixing kernel: reduce the summary kernel's token-slice partials and mix the per-block
// summaries with the coefficient matrix, S~_i = sum_b m_ib S_b and z~_i = sum_b m_ib z_b
// ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method ->
// Key design 2, multi-head mixing; row i of M_c belongs to query block i).
//
// MALA mode (one block; "Rectifying Magnitude Neglect in Linear Attention", Method -> Key
// design, linear form Y_i = beta_i phi(Q_i) S - gamma_i u with S = sum_j phi(K_j)^T V_j,
// u = sum_j V_j, beta_i = 1 + 1/s_i, gamma_i = s_i/N, s_i = phi(Q_i) z):  substituting
// S = C + z u^T / N gives Y_i = u/N + beta_i phi(Q_i) C exactly, with C = S - z u^T / N.
// C is formed here in fp32, so the readout never subtracts two large, nearly equal terms.
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

  for (int b = 0; b < M; ++b) {
    const int64_t slot0 = ((int64_t)bh * M + b) * p.splits;
    float s = 0.f;
    for (int sp = 0; sp < p.splits; ++sp)
      s += is_z ? p.pz[(slot0 + sp) * d + zpos] : p.ps[(slot0 + sp) * frag + pos];
#pragma unroll
    for (int r = 0; r < kMixRows; ++r)
      if (r < nrows) acc[r] = fmaf(mc ? mc[(int64_t)(i0 + r) * M + b] : 1.0f, s, acc[r]);
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

// MALA (M == 1): grid (ceil((FRAG + D) / 256), 1, BH).
template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void mala_center_kernel(MixParams p, int frag, int d) {
  const int pos = blockIdx.x * kThreads + threadIdx.x;
  if (pos >= frag + d) return;
  const int bh = blockIdx.z;
  const int64_t slot0 = (int64_t)bh * p.splits;
  const float inv_n = 1.0f / (float)p.N;
  if (pos >= frag) {
    const int c = pos - frag;
    float z = 0.f, u = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      z += p.pz[(slot0 + sp) * d + c];
      u += p.pu[(slot0 + sp) * d + c];
    }
    p.zt[(int64_t)bh * d + c] = z;
    p.ubar[(int64_t)bh * d + c] = u * inv_n;
    return;
  }
  // fragment position -> (k, c)
  const int e = pos & 7;
  const int lane = (pos >> 3) & 63;
  const int fr = pos >> 9;
  const int nct = d / 16;
  const int kc = fr / nct, ct = fr % nct;
  const int k = 32 * kc + 8 * (lane >> 4) + e;
  const int c = 16 * ct + (lane & 15);
  float s = 0.f, z = 0.f, u = 0.f;
  for (int sp = 0; sp < p.splits; ++sp) {
    s += p.ps[(slot0 + sp) * frag + pos];
    if (k < d) z += p.pz[(slot0 + sp) * d + k];
    u += p.pu[(slot0 + sp) * d + c];
  }
  const float cval = s - z * u * inv_n;
  store_hi_lo<SPLIT>(p.st_hi, p.st_lo, (int64_t)bh * frag + pos, cval);
}

hipError_t launch_mix(const MixParams& p, int d, int frag, int bh, bool mala, bool split,
                      hipStream_t stream) {
  const dim3 block(kThreads);
  const int nx = (frag + d + kThreads - 1) / kThreads;
  if (mala) {
    const dim3 grid(nx, 1, bh);
    if (split)
      hipLaunchKernelGGL(mala_center_kernel<true>, grid, block, 0, stream, p, frag, d);
    else
      hipLaunchKernelGGL(mala_center_kernel<false>, grid, block, 0, stream, p, frag, d);
  } else {
    const dim3 grid(nx, (p.M + kMixRows - 1) / kMixRows, bh);
    if (split)
      hipLaunchKernelGGL(mix_kernel<true>, grid, block, 0, stream, p, frag, d);
    else
      hipLaunchKernelGGL(mix_kernel<false>, grid, block, 0, stream, p, frag, d);
  }
  return hipGetLastError();
}

}  // namespace mhla
