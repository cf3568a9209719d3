// Readout kernel: for every query token t of block i,
//   normalised    o_t = phi(q_t)^T S~_i / phi(q_t)^T z~_i
//   unnormalised  o_t = phi(q_t)^T S~_i
//   MALA          o_t = u/N + (1 + 1/s_t) phi(q_t)^T C,   s_t = phi(q_t)^T z
// Sources: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Method -> Overall framework (flowchart readout) and Key design 2 (mixing S~_i = sum_b m_ib S_b;
// the normaliser may be dropped); "Rectifying Magnitude Neglect in Linear Attention", Method ->
// Key design (beta, gamma and the linear form, with C = S - z u^T / N so that
// Y = u/N + beta q~^T C exactly).
//
// One workgroup (4 wave64s) owns one token slice of one query block of one (batch, head).
// Prologue: the block's mixed summary is staged in LDS in fragment layout (each MFMA A operand
// is one 16-byte LDS read), together with one extra "normaliser" fragment per 32-feature chunk
// whose rows 4g+0 hold hi(z~[k]) and rows 4g+1 hold lo(z~[k]) for every lane group g.  The mixed
// summary either comes from the mixing kernel, or -- for few blocks -- is formed right here:
//   FUSE_BF16      S~_i = sum_b m_ib S_b from the bf16 stack, z~_i likewise, in fp32;
//   FUSE_PARTIALS  from the fp32 token-slice partials: S_b = sum of slices, then the mixing
//                  (MHLA) or the centring C = S - z u^T / N (MALA), split into bf16 hi + lo.
// With all workgroups of a head on one XCD, the stack is read from HBM once per head and from
// that XCD's L2 afterwards.
// Main loop: each wave walks 16-token tiles; the lane owning token t = lane%16 and key
// features 32*kc + 8*(lane/16) + 0..7 loads them with one 16-byte read (the next tile's loads
// are issued before the current tile is computed), applies phi in fp32, and MFMAs compute
// O^T = S~^T phi(Q)^T, with the normaliser fragment leaving phi(q_t)^T z~ = D[4g] + D[4g+1] in
// every lane of token t with no cross-lane reduction.  Output channels are taken 32 at a time as
// two MFMA tiles h = 0, 1 whose A row m is channel 8*(m/4) + 4h + m%4 of the group, so lane
// (t, g) ends with the 8 consecutive channels 8g .. 8g+7 of token t: 16-byte stores, and the four
// lane groups of a token write 64 (bf16) or 128 (fp32) contiguous bytes.  In LDS, bit 2 of a
// fragment's lane index is flipped when bit 3 is set, so that every 8 lanes of these operand
// reads cover all banks once.
#include "mhla_device.hpp"

namespace mhla {

enum { kModeNormalized = 0, kModeUnnormalized = 1, kModeMala = 2 };
enum { kFuseNone = 0, kFuseBf16 = 1, kFusePartials = 2 };

template <bool SPLIT>
__device__ inline void store_frag8(uint16_t* s_hi, uint16_t* s_lo, int pos, const float (&a)[8]) {
  if (SPLIT) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16(a[e], h[e], l[e]);
    st16(s_hi + pos, u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                             h[6] | (h[7] << 16)});
    st16(s_lo + pos, u32x4_t{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                             l[6] | (l[7] << 16)});
  } else {
    st16(s_hi + pos, u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                             pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])});
  }
}

// LDS element offset of fragment element `pos` (a multiple of 8): see the bank note above
template <int NCT>
__device__ inline int lds_pos(int pos) {
  if constexpr (NCT >= 2) {
    const int u = pos >> 3;
    return (u ^ (((u >> 3) & 1) << 2)) << 3;
  } else {
    return pos;
  }
}

template <typename TIn, typename TOut, int D, bool SPLIT, int FUSE>
__global__ __launch_bounds__(kThreads) void readout_kernel(ReadoutParams p, int mode) {
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int ZF = NKC * 512;            // normaliser fragments (elements)

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_hi = smem;                   // [FRAG]
  uint16_t* s_lo = s_hi + FRAG;            // [FRAG]       (SPLIT)
  uint16_t* s_z = s_lo + (SPLIT ? FRAG : 0);   // [ZF]
  float* s_ub = reinterpret_cast<float*>(s_z + ZF);   // [D]   mean of V (MALA)
  float* s_zt = s_ub + D;                             // [D]   z~ (fp32) before fragmenting

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const Geom& g = p.g;
  const int pr = lane & 15, lg = lane >> 4;

  // ---- workgroup -> (token slice, block, head); heads pinned to XCDs when requested --------
  int split, blk, bh;
  {
    const int per_head = p.splits * g.M;
    const int L = blockIdx.x;
    int r;
    if (p.xcd_map) {   // dispatch is round-robin over the 8 XCDs by workgroup index
      const int xcd = L & 7, s = L >> 3;
      bh = (s / per_head) * 8 + xcd;
      r = s % per_head;
    } else {
      bh = L / per_head;
      r = L % per_head;
    }
    blk = r / p.splits;
    split = r % p.splits;
  }

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
      raw[kc].template load_buf<MHLA_READOUT_LOAD_CPOL>(rsq, (valid && k0 < D) ? (rel + k0) * ES : kOutOfRange);
    }
  };
  int tile = wave;
  if (tile < n_tiles) issue(tile);

  // ---- prologue: mixed summary (loaded or formed here), z~, mean of V ------------------
  const int M = g.M;
  const int64_t row = (int64_t)bh * M + blk;
  if constexpr (FUSE == kFuseNone) {
    const uint16_t* src_hi = p.st_hi + row * FRAG;
    for (int i = tid * 8; i < FRAG; i += kThreads * 8) {
      st16(s_hi + lds_pos<NCT>(i), ld16(src_hi + i));
      if (SPLIT) st16(s_lo + lds_pos<NCT>(i), ld16(p.st_lo + row * FRAG + i));
    }
    if (tid < D) s_zt[tid] = p.zt[row * D + tid];
  } else if constexpr (FUSE == kFuseBf16) {
    // S~_i = sum_b m_ib S_b and z~_i = sum_b m_ib z_b in fp32 (NULL M_c: M == 1, weight 1)
    const float* mrow =
        p.mc ? p.mc + (int64_t)(bh % p.H) * p.mc_head_stride + (int64_t)blk * M : nullptr;
    // blocks are taken 8 at a time with all 8 loads in flight; blocks >= M read as zero
    // through the buffer resource and carry the weight 0
    const Rsrc rss = make_rsrc(p.sb + (int64_t)bh * M * FRAG, (uint32_t)M * FRAG * 2u);
    auto weight = [&](int b) { return b < M ? (mrow ? mrow[b] : 1.0f) : 0.0f; };
    for (int pos = tid * 8; pos < FRAG; pos += kThreads * 8) {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int b0 = 0; b0 < M; b0 += 8) {
        u32x4_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = buf_ld16(rss, b0 + j < M ? (uint32_t)((b0 + j) * FRAG + pos) * 2u : kOutOfRange);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float m = weight(b0 + j);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t x = w[j][e >> 1];
            a[e] = fmaf(m, (e & 1) ? bf16hi_to_f32(x) : bf16lo_to_f32(x), a[e]);
          }
        }
      }
      store_frag8<false>(s_hi, s_lo, lds_pos<NCT>(pos), a);
    }
    if (tid < D) {
      // one token slice per block on this path: z_b = pz[bh][b][:]
      const float* zsrc = p.pz + (int64_t)bh * M * D + tid;
      float a = 0.f;
      for (int b0 = 0; b0 < M; b0 += 8) {
        float zb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) zb[j] = zsrc[(int64_t)min(b0 + j, M - 1) * D];
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaf(weight(b0 + j), zb[j], a);
      }
      s_zt[tid] = a;
    }
  } else {  // kFusePartials
    const int ss = p.ssplits;
    if (mode == kModeMala) {
      // one block: S, z, u are sums over the token slices; C = S - z u^T / N
      const float inv_n = 1.0f / (float)g.N;
      const Rsrc rsp = make_rsrc(p.ps + (int64_t)bh * ss * FRAG, (uint32_t)ss * FRAG * 4u);
      if (tid < D) {
        float z = 0.f, u = 0.f;
        for (int s = 0; s < ss; ++s) {
          z += p.pz[((int64_t)bh * ss + s) * D + tid];
          u += p.pu[((int64_t)bh * ss + s) * D + tid];
        }
        s_zt[tid] = z;
        s_ub[tid] = u;          // u for now; scaled to u / N below
      }
      __syncthreads();
      for (int pos = tid * 8; pos < FRAG; pos += kThreads * 8) {
        const int l = (pos >> 3) & 63, fr = pos >> 9;
        const int kc = fr / NCT, ct = fr % NCT;
        const int k0 = 32 * kc + 8 * (l >> 4);
        const float uc = s_ub[16 * ct + (l & 15)] * inv_n;
        // slices 4 at a time with all loads in flight; slices >= ss read as zero
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < ss; s0 += 4) {
          u32x4_t w[4][2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t off = s0 + j < ss ? (uint32_t)((s0 + j) * FRAG + pos) * 4u : kOutOfRange;
            w[j][0] = buf_ld16(rsp, off);
            w[j][1] = buf_ld16(rsp, off == kOutOfRange ? kOutOfRange : off + 16u);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] += __uint_as_float(w[j][0][e]);
              a[4 + e] += __uint_as_float(w[j][1][e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = k0 + e;
          a[e] -= (k < D ? s_zt[k] : 0.f) * uc;
        }
        store_frag8<SPLIT>(s_hi, s_lo, lds_pos<NCT>(pos), a);
      }
      __syncthreads();
      if (tid < D) s_ub[tid] *= inv_n;
    } else {
      // MHLA from fp32 partials: S~_i = sum_b m_ib sum_s S_{b,s}
      const float* mrow =
          p.mc ? p.mc + (int64_t)(bh % p.H) * p.mc_head_stride + (int64_t)blk * M : nullptr;
      for (int pos = tid * 8; pos < FRAG; pos += kThreads * 8) {
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int b = 0; b < M; ++b) {
          const float m = mrow ? mrow[b] : 1.0f;
          float sb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int s = 0; s < ss; ++s) {
            const float* src = p.ps + (((int64_t)bh * M + b) * ss + s) * FRAG + pos;
            const u32x4_t w0 = ld16(src), w1 = ld16(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sb[e] += __uint_as_float(w0[e]);
              sb[4 + e] += __uint_as_float(w1[e]);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = fmaf(m, sb[e], a[e]);
        }
        store_frag8<SPLIT>(s_hi, s_lo, lds_pos<NCT>(pos), a);
      }
      if (tid < D) {
        float a = 0.f;
        for (int b = 0; b < M; ++b) {
          float zb = 0.f;
          for (int s = 0; s < ss; ++s) zb += p.pz[(((int64_t)bh * M + b) * ss + s) * D + tid];
          a = fmaf(mrow ? mrow[b] : 1.0f, zb, a);
        }
        s_zt[tid] = a;
      }
    }
  }
  __syncthreads();
  // normaliser fragments from z~ (fp32 in LDS)
  if (tid < NKC * 64) {                       // one lane-fragment of 8 elements per thread
    const int kc = tid >> 6, l = tid & 63;
    const int rowp = l & 15, grp = l >> 4;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if ((rowp & 3) < 2) {
      uint32_t bits[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * kc + 8 * grp + e;
        const float zv = k < D ? s_zt[k] : 0.f;
        uint32_t h, lo;
        split_bf16(zv, h, lo);
        bits[e] = (rowp & 3) == 0 ? h : lo;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = bits[2 * i] | (bits[2 * i + 1] << 16);
    }
    st16(s_z + (kc * 64 + l) * 8, u32x4_t{w[0], w[1], w[2], w[3]});
  }
  __syncthreads();

  // A row pr of tile ct is channel 32*(ct/2) + 8*(pr/4) + 4*(ct%2) + pr%4 (d >= 32): it sits in
  // fragment ct & ~1 (or the next one for pr >= 8) at lane 16*lg + 8*b + 4*(ct%2) + pr%4,
  // b = (pr/4)%2, which the LDS swizzle moves to 16*lg + 8*b + 4*((ct%2) ^ b) + pr%4
  const int b3 = (pr >> 2) & 1;
  const int a_even = ((pr >> 3) * 64 + 16 * lg + 8 * b3 + 4 * (0 ^ b3) + (pr & 3)) * 8;
  const int a_odd = ((pr >> 3) * 64 + 16 * lg + 8 * b3 + 4 * (1 ^ b3) + (pr & 3)) * 8;

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
        const int off = NCT >= 2 ? (kc * NCT + (ct & ~1)) * 512 + ((ct & 1) ? a_odd : a_even)
                                 : (kc * 64 + lane) * 8;
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
    // lane (t, g) holds channels cg0 + 0..7 of each 32-channel group (d = 16: channels 4g..4g+3)
    constexpr int NG = NCT >= 2 ? NCT / 2 : 1;      // channel groups
    constexpr int W = NCT >= 2 ? 8 : 4;             // channels per lane and group
#pragma unroll
    for (int cgp = 0; cgp < NG; ++cgp) {
      const int c0 = NCT >= 2 ? 32 * cgp + 8 * lg : 4 * lg;
      float o[W];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = acc[NCT >= 2 ? 2 * cgp : 0][r] * scale;
        if constexpr (W == 8) o[4 + r] = acc[2 * cgp + 1][r] * scale;
      }
      if (mode == kModeMala) {
#pragma unroll
        for (int j = 0; j < W; j += 4) {
          const u32x4_t ub = *reinterpret_cast<const u32x4_t*>(s_ub + c0 + j);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[j + r] += __uint_as_float(ub[r]);
        }
      }
      const int64_t dst = coff + c0;
      if constexpr (sizeof(TOut) == 4) {
#pragma unroll
        for (int j = 0; j < W; j += 4)
          st16_pol<MHLA_READOUT_STORE_NT>(
              reinterpret_cast<float*>(p.o) + dst + j,
              u32x4_t{__float_as_uint(o[j]), __float_as_uint(o[j + 1]), __float_as_uint(o[j + 2]),
                      __float_as_uint(o[j + 3])});
      } else if constexpr (W == 8) {
        st16_pol<MHLA_READOUT_STORE_NT>(
            reinterpret_cast<uint16_t*>(p.o) + dst,
            u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7])});
      } else {
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(p.o) + dst) =
            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
  }
}

template <typename TIn, typename TOut, int D, bool SPLIT, int FUSE>
static hipError_t launch_t(const ReadoutParams& p, int mode, int n_wg, hipStream_t s) {
  using Dm = Dims<D>;
  const size_t lds = (size_t)Dm::FRAG * 2 * (SPLIT ? 2 : 1) + (size_t)Dm::NKC * 512 * 2 + 2 * D * 4;
  hipLaunchKernelGGL((readout_kernel<TIn, TOut, D, SPLIT, FUSE>), dim3(n_wg), dim3(kThreads), lds,
                     s, p, mode);
  return hipGetLastError();
}

// Valid (split, fuse) pairs: the bf16-stack fusion exists for bf16 operands only; the others
// for both operand precisions.
template <typename TIn, typename TOut, int D>
static hipError_t dispatch_fuse(const ReadoutParams& p, int mode, bool split, int fuse, int n_wg,
                                hipStream_t s) {
  if (split) {
    if (fuse == kFuseNone) return launch_t<TIn, TOut, D, true, kFuseNone>(p, mode, n_wg, s);
    if (fuse == kFusePartials) return launch_t<TIn, TOut, D, true, kFusePartials>(p, mode, n_wg, s);
    return hipErrorInvalidValue;
  }
  if (fuse == kFuseNone) return launch_t<TIn, TOut, D, false, kFuseNone>(p, mode, n_wg, s);
  if (fuse == kFusePartials) return launch_t<TIn, TOut, D, false, kFusePartials>(p, mode, n_wg, s);
  if constexpr (sizeof(TIn) == 2) {
    if (fuse == kFuseBf16) return launch_t<TIn, TOut, D, false, kFuseBf16>(p, mode, n_wg, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, typename TOut>
static hipError_t dispatch_d(const ReadoutParams& p, int d, int mode, bool split, int fuse,
                             int n_wg, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_fuse<TIn, TOut, 16>(p, mode, split, fuse, n_wg, s);
    case 32: return dispatch_fuse<TIn, TOut, 32>(p, mode, split, fuse, n_wg, s);
    case 64: return dispatch_fuse<TIn, TOut, 64>(p, mode, split, fuse, n_wg, s);
    case 128: return dispatch_fuse<TIn, TOut, 128>(p, mode, split, fuse, n_wg, s);
    default: return hipErrorInvalidValue;
  }
}

// n_wg = splits * M * BH workgroups (one-dimensional grid).
hipError_t launch_readout(const ReadoutParams& p, int d, bool in_fp32, bool out_fp32, int mode,
                          bool split, int fuse, int n_wg, hipStream_t stream) {
  if (in_fp32)
    return out_fp32 ? dispatch_d<float, float>(p, d, mode, split, fuse, n_wg, stream)
                    : dispatch_d<float, uint16_t>(p, d, mode, split, fuse, n_wg, stream);
  return out_fp32 ? dispatch_d<uint16_t, float>(p, d, mode, split, fuse, n_wg, stream)
                  : dispatch_d<uint16_t, uint16_t>(p, d, mode, split, fuse, n_wg, stream);
}

}  // namespace mhla
