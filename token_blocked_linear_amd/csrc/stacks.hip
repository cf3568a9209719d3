// The forward's intermediate stacks in plain fp32 layouts, for inspection: the block summaries
// S_b, z_b of step 3 and the mixed summaries S~_i, z~_i of step 4 ("MHLA: Restoring Expressivity
// of Linear Attention via Token-Level Multi-Head", Overall framework and Key design 2).  The
// kernels keep a d x d summary T (rows: key features k, columns: value channels c) in MFMA
// fragment layout: element (kc, ct, lane, e) is T[32kc + 8(lane/16) + e][16ct + lane%16] at
// position ((kc * NCT + ct) * 64 + lane) * 8 + e, NCT = d / 16, rows k >= d zero padding (d = 16),
// as bf16 (a high part, optionally a low part) or as fp32 partials over token slices.
#include "mhla_device.hpp"

namespace mhla {

namespace {

// out[row][k][c] from the fragment-layout stack of `row`: hi (+ lo) bf16, or the sum over
// `splits` fp32 partials [row][splits][frag].
__global__ __launch_bounds__(kThreads) void frag_to_rowmajor_kernel(const uint16_t* hi, const uint16_t* lo,
                                                                    const float* part, int splits, int64_t rows,
                                                                    int d, int frag, float* out) {
  const int nct = d / 16;
  const int64_t total = rows * frag;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / frag;
    const int pos = (int)(i - row * frag);
    const int e = pos & 7, lane = (pos >> 3) & 63, fr = pos >> 9;
    const int kc = fr / nct, ct = fr - kc * nct;
    const int k = 32 * kc + 8 * (lane >> 4) + e, c = 16 * ct + (lane & 15);
    if (k >= d) continue;   // padding rows of d = 16
    float x;
    if (part) {
      x = 0.f;
      for (int s = 0; s < splits; ++s) x += part[(row * splits + s) * frag + pos];
    } else {
      x = __uint_as_float((uint32_t)hi[i] << 16);
      if (lo) x += __uint_as_float((uint32_t)lo[i] << 16);
    }
    out[(row * d + k) * d + c] = x;
  }
}

// out[row][j] = sum over `splits` of part[row][s][j] (j < d)
__global__ __launch_bounds__(kThreads) void sum_splits_kernel(const float* part, int splits, int64_t rows, int d,
                                                              float* out) {
  const int64_t total = rows * d;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / d;
    const int j = (int)(i - row * d);
    float x = 0.f;
    for (int s = 0; s < splits; ++s) x += part[(row * splits + s) * d + j];
    out[i] = x;
  }
}

unsigned grid_for(int64_t total) {
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_frag_to_rowmajor(const uint16_t* hi, const uint16_t* lo, const float* part, int splits,
                                   int64_t rows, int d, int frag, float* out, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(frag_to_rowmajor_kernel, dim3(grid_for(rows * frag)), dim3(kThreads), 0, stream, hi, lo, part,
                     splits, rows, d, frag, out);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int splits, int64_t rows, int d, float* out, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_splits_kernel, dim3(grid_for(rows * d)), dim3(kThreads), 0, stream, part, splits, rows, d,
                     out);
  return hipGetLastError();
}

}  // namespace mhla
