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
// Prologue: the block's mixed summary is staged in LDS in fragment layout (each MFMA A operand
// is one 16-byte LDS read), together with one extra "normaliser" fragment per 32-feature
// chunk whose rows 4g+0 hold hi(z~[k]) and rows 4g+1 hold lo(z~[k]) for every lane group g.
// Main loop: each wave walks 16-token tiles; the lane owning token t = lane%16 and key
// features 32*kc + 8*(lane/16) + 0..7 loads them with one 16-byte global read (the next
// tile's loads are issued before the current tile is computed), applies phi in fp32, and
// MFMAs compute O^T = S~^T phi(Q)^T: lane (t, g) holds channels 16*ct + 4g + 0..3 of token t,
// and the normaliser fragment leaves phi(q_t)^T z~ = D[4g] + D[4g+1] in every lane of token t
// with no cross-lane reduction.
#include "mhla_device.hpp"

namespace mhla {

enum { kModeNormalized = 0, kModeUnnormalized = 1, kModeMala = 2 };

template <typename TIn, typename TOut, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void readout_kernel(ReadoutParams p, int mode) {
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int ZF = NKC * 512;            // normaliser fragments (elements)

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_hi = smem;                   // [FRAG]
  uint16_t* s_lo = s_hi + FRAG;            // [FRAG]       (SPLIT)
  uint16_t* s_z = s_lo + (SPLIT ? FRAG : 0);   // [ZF]
  float* s_ub = reinterpret_cast<float*>(s_z + ZF);   // [D]   (MALA)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int blk = blockIdx.y;
  const int bh = blockIdx.z;
  const Geom& g = p.g;
  const int pr = lane & 15, lg = lane >> 4;

  const int32_t j_begin = split * p.tok_per_split;
  const int32_t j_end = min(j_begin + p.tok_per_split, g.n_b);
  const int32_t base_tok = block_base_token(g, blk);
  const int64_t head_off = (int64_t)bh * g.N * D;
  const int n_tiles = (j_end - j_begin + 15) >> 4;

  // first tile's query loads go out before the prologue
  auto tok_offset = [&](int tile, bool& valid) -> int64_t {
    const int32_t j = j_begin + tile * 16 + pr;
    valid = j < j_end;
    return valid ? head_off + (int64_t)(base_tok + block_token_offset(g, (uint32_t)j)) * D : 0;
  };
  // query loads through a buffer resource over this head: invalid tokens and key features
  // beyond D (d = 16) read as zero without a branch
  constexpr uint32_t ES = sizeof(TIn);
  const Rsrc rsq = make_rsrc(reinterpret_cast<const TIn*>(p.q) + head_off, (uint32_t)g.N * D * ES);
  In8<TIn> raw[NKC];
  bool valid = false;
  int64_t toff = 0;
  auto issue = [&](int tile) {
    toff = tok_offset(tile, valid);
    const uint32_t rel = (uint32_t)(toff - head_off);       // element offset within the head
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int k0 = 32 * kc + 8 * lg;
      raw[kc].load_buf(rsq, (valid && k0 < D) ? (rel + k0) * ES : kOutOfRange);
    }
  };
  int tile = wave;
  if (tile < n_tiles) issue(tile);

  // ---- prologue: mixed summary, normaliser fragments, mean of V ---------------------------
  const int64_t row = (int64_t)bh * g.M + blk;
  {
    const uint16_t* src_hi = p.st_hi + row * FRAG;
    for (int i = tid * 8; i < FRAG; i += kThreads * 8) {
      st16(s_hi + i, ld16(src_hi + i));
      if (SPLIT) st16(s_lo + i, ld16(p.st_lo + row * FRAG + i));
    }
    if (tid < NKC * 64) {                       // one lane-fragment of 8 elements per thread
      const int kc = tid >> 6, l = tid & 63;
      const int rowp = l & 15, grp = l >> 4;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if ((rowp & 3) < 2) {
        const float* zsrc = p.zt + row * D;
        uint32_t bits[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 32 * kc + 8 * grp + e;
          const float zv = k < D ? zsrc[k] : 0.f;
          uint32_t h, lo;
          split_bf16(zv, h, lo);
          bits[e] = (rowp & 3) == 0 ? h : lo;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = bits[2 * i] | (bits[2 * i + 1] << 16);
      }
      st16(s_z + (kc * 64 + l) * 8, u32x4_t{w[0], w[1], w[2], w[3]});
    }
    if (mode == kModeMala && tid < D) s_ub[tid] = p.ubar[(int64_t)bh * D + tid];
  }
  __syncthreads();

  for (; tile < n_tiles; tile += kThreads / 64) {
    // take this tile's inputs and issue the next tile's loads
    In8<TIn> cur[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) cur[kc] = raw[kc];
    const bool cvalid = valid;
    const int64_t coff = toff;
    if (tile + kThreads / 64 < n_tiles) issue(tile + kThreads / 64);

    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t accz = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int k0 = 32 * kc + 8 * lg;
      u32x4_t b_hi, b_lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = 0.f, x1 = 0.f;
        if (cvalid && k0 < D) {
          x0 = phi_elu1(cur[kc].get(2 * i));
          x1 = phi_elu1(cur[kc].get(2 * i + 1));
        }
        if (SPLIT) {
          uint32_t h0, l0, h1, l1;
          split_bf16(x0, h0, l0);
          split_bf16(x1, h1, l1);
          b_hi[i] = h0 | (h1 << 16);
          b_lo[i] = l0 | (l1 << 16);
        } else {
          b_hi[i] = pack_bf16x2(x0, x1);
        }
      }
      const u32x4_t az = *reinterpret_cast<const u32x4_t*>(s_z + (kc * 64 + lane) * 8);
      accz = mfma_bf16(az, b_hi, accz);
      if (SPLIT) accz = mfma_bf16(az, b_lo, accz);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int off = ((kc * NCT + ct) * 64 + lane) * 8;
        const u32x4_t a_hi = *reinterpret_cast<const u32x4_t*>(s_hi + off);
        acc[ct] = mfma_bf16(a_hi, b_hi, acc[ct]);
        if (SPLIT) {
          const u32x4_t a_lo = *reinterpret_cast<const u32x4_t*>(s_lo + off);
          acc[ct] = mfma_bf16(a_lo, b_hi, acc[ct]);
          acc[ct] = mfma_bf16(a_hi, b_lo, acc[ct]);
        }
      }
      // keep each chunk's LDS operand reads next to their MFMAs: hoisting all of them would
      // cost NKC*NCT*4 registers and halve the waves per SIMD at d = 128
      __builtin_amdgcn_sched_barrier(0);
    }

    if (!cvalid) continue;
    const float den = accz[0] + accz[1];      // phi(q_t)^T z~  (hi row + lo row)
    float scale = 1.f;
    if (mode == kModeNormalized) scale = 1.0f / den;
    else if (mode == kModeMala) scale = 1.0f + 1.0f / den;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = acc[ct][r] * scale;
      if (mode == kModeMala) {
        const u32x4_t ub = *reinterpret_cast<const u32x4_t*>(s_ub + 16 * ct + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] += __uint_as_float(ub[r]);
      }
      const int64_t dst = coff + 16 * ct + 4 * lg;
      if constexpr (sizeof(TOut) == 4) {
        st16_stream(reinterpret_cast<float*>(p.o) + dst,
             u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
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
  using Dm = Dims<D>;
  const size_t lds = (size_t)Dm::FRAG * 2 * (split ? 2 : 1) + (size_t)Dm::NKC * 512 * 2 + D * 4;
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
