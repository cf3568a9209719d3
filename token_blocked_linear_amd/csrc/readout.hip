// Readout kernel: for every query token t of block i,
//   normalised    o_t = phi(q_t)^T S~_i / phi(q_t)^T z~_i
//   unnormalised  o_t = phi(q_t)^T S~_i
//   MALA          o_t = u/N + (1 + 1/s_t) phi(q_t)^T C,   s_t = phi(q_t)^T z
// Sources: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Method -> Overall framework (flowchart readout) and Key design 2 (the normaliser may be
// dropped); "Rectifying Magnitude Neglect in Linear Attention", Method -> Key design (beta,
// gamma and the linear form; the centred summary C is formed by the mixing kernel).
//
// One workgroup (4 wave64s) owns one token slice of one query block of one (batch, head).
// The block's mixed summary is staged once in LDS (fragment layout, so each MFMA A operand is
// one 16-byte LDS read).  Each wave walks 16-token tiles: the lane owning token t = lane%16
// and key features 32*kc + 8*(lane/16) + 0..7 loads them with one 16-byte global read, applies
// phi in fp32, and the MFMAs compute O^T = S~^T phi(Q)^T, so lane (t, g) ends up holding
// channels 16*ct + 4g + 0..3 of token t.  The denominator is each lane's fp32 partial dot
// product reduced across the four lanes of a token with two xor shuffles.
#include "mhla_device.hpp"

namespace mhla {

enum { kModeNormalized = 0, kModeUnnormalized = 1, kModeMala = 2 };

template <typename TIn, typename TOut, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void readout_kernel(ReadoutParams p, int mode) {
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_hi = smem;                  // [FRAG]
  uint16_t* s_lo = smem + FRAG;           // [FRAG] (SPLIT)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int blk = blockIdx.y;
  const int bh = blockIdx.z;
  const Geom& g = p.g;
  const int pr = lane & 15, lg = lane >> 4;

  const int64_t row = (int64_t)bh * g.M + blk;
  {
    const uint16_t* src_hi = p.st_hi + row * FRAG;
    const uint16_t* src_lo = SPLIT ? p.st_lo + row * FRAG : nullptr;
    for (int i = tid * 8; i < FRAG; i += kThreads * 8) {
      st16(s_hi + i, ld16(src_hi + i));
      if (SPLIT) st16(s_lo + i, ld16(src_lo + i));
    }
  }
  // normaliser entries for this lane's key features
  float zt[NKC][8];
  const float* zsrc = p.zt + row * D;
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 32 * kc + 8 * lg + e;
      zt[kc][e] = k < D ? zsrc[k] : 0.f;
    }
  float ub[NCT][4];
  if (mode == kModeMala) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) ub[ct][r] = p.ubar[(int64_t)bh * D + 16 * ct + 4 * lg + r];
  }
  __syncthreads();

  const int32_t j_begin = split * p.tok_per_split;
  const int32_t j_end = min(j_begin + p.tok_per_split, g.n_b);
  const int32_t base_tok = block_base_token(g, blk);
  const int64_t head_off = (int64_t)bh * g.N * D;
  const int n_tiles = (j_end - j_begin + 15) >> 4;

  for (int tile = wave; tile < n_tiles; tile += kThreads / 64) {
    const int32_t j = j_begin + tile * 16 + pr;
    const bool valid = j < j_end;
    int64_t tok_off = 0;
    if (valid) tok_off = head_off + (int64_t)(base_tok + block_token_offset(g, (uint32_t)j)) * D;

    u32x4_t b_hi[NKC], b_lo[NKC];
    float den = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int k0 = 32 * kc + 8 * lg;
      In8<TIn> raw;
      if (valid && k0 < D)
        raw.load(p.q, tok_off + k0);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (valid && k0 < D) ? phi_elu1(raw.get(e)) : 0.f;
        den = fmaf(x[e], zt[kc][e], den);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (SPLIT) {
          uint32_t h0, l0, h1, l1;
          split_bf16(x[2 * i], h0, l0);
          split_bf16(x[2 * i + 1], h1, l1);
          b_hi[kc][i] = h0 | (h1 << 16);
          b_lo[kc][i] = l0 | (l1 << 16);
        } else {
          b_hi[kc][i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        }
      }
    }
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);

    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int off = ((kc * NCT + ct) * 64 + lane) * 8;
        const u32x4_t a_hi = *reinterpret_cast<const u32x4_t*>(s_hi + off);
        acc[ct] = mfma_bf16(a_hi, b_hi[kc], acc[ct]);
        if (SPLIT) {
          const u32x4_t a_lo = *reinterpret_cast<const u32x4_t*>(s_lo + off);
          acc[ct] = mfma_bf16(a_lo, b_hi[kc], acc[ct]);
          acc[ct] = mfma_bf16(a_hi, b_lo[kc], acc[ct]);
        }
      }
    }

    if (!valid) continue;
    float scale = 1.f;
    if (mode == kModeNormalized) scale = 1.0f / den;
    else if (mode == kModeMala) scale = 1.0f + 1.0f / den;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = acc[ct][r] * scale;
        if (mode == kModeMala) o[r] += ub[ct][r];
      }
      const int64_t dst = tok_off + 16 * ct + 4 * lg;
      if constexpr (sizeof(TOut) == 4) {
        float* out = reinterpret_cast<float*>(p.o) + dst;
        st16(out, u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                          __float_as_uint(o[3])});
      } else {
        uint32_t* out = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.o) + dst);
        out[0] = pack_bf16x2(o[0], o[1]);
        out[1] = pack_bf16x2(o[2], o[3]);
      }
    }
  }
}

template <typename TIn, typename TOut, int D>
static hipError_t launch_t(const ReadoutParams& p, int mode, bool split, dim3 grid, hipStream_t s) {
  const size_t lds = (size_t)Dims<D>::FRAG * 2 * (split ? 2 : 1);
  if (split)
    hipLaunchKernelGGL((readout_kernel<TIn, TOut, D, true>), grid, dim3(kThreads), lds, s, p, mode);
  else
    hipLaunchKernelGGL((readout_kernel<TIn, TOut, D, false>), grid, dim3(kThreads), lds, s, p, mode);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
static hipError_t dispatch_d(const ReadoutParams& p, int d, int mode, bool split, dim3 grid,
                             hipStream_t s) {
  switch (d) {
    case 16: return launch_t<TIn, TOut, 16>(p, mode, split, grid, s);
    case 32: return launch_t<TIn, TOut, 32>(p, mode, split, grid, s);
    case 64: return launch_t<TIn, TOut, 64>(p, mode, split, grid, s);
    case 128: return launch_t<TIn, TOut, 128>(p, mode, split, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_readout(const ReadoutParams& p, int d, bool in_fp32, bool out_fp32, int mode,
                          bool split, dim3 grid, hipStream_t stream) {
  if (in_fp32)
    return out_fp32 ? dispatch_d<float, float>(p, d, mode, split, grid, stream)
                    : dispatch_d<float, uint16_t>(p, d, mode, split, grid, stream);
  return out_fp32 ? dispatch_d<uint16_t, float>(p, d, mode, split, grid, stream)
                  : dispatch_d<uint16_t, uint16_t>(p, d, mode, split, grid, stream);
}

}  // namespace mhla
