// Summary kernel: phi(K) in registers, per-block S_b = sum_j phi(K_j) V_j^T on bf16 MFMA with
// fp32 accumulation, z_b = sum_j phi(K_j) (and, for the MALA readout, u = sum_j V_j) in fp32.
//
// Source: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Method -> Overall framework (local KV summary S_b and normaliser z_b of every block); the
// MALA linear form in "Rectifying Magnitude Neglect in Linear Attention", Method -> Key design,
// also needs sum_j V_j.
//
// One workgroup (4 wave64s) owns one token slice of one block of one (batch, head).  Tokens
// are streamed in rounds.  Each thread owns 8 consecutive block-local tokens x 8 consecutive
// features: it issues one 16-byte load per token row (D/8 lanes cover a row, so every load
// instruction reads whole rows), applies phi in fp32, and transposes its 8x8 piece in
// registers so that LDS holds phi(K)^T and V^T with tokens contiguous (one 16-byte LDS write
// per feature).  The MFMA phase then reads every operand with one 16-byte LDS read.
// The next round's global loads are issued before the MFMA phase of the current one.
#include "mhla_device.hpp"

namespace mhla {

template <typename TIn, int D, bool SPLIT_K, bool SPLIT_V, bool WANT_U, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void summary_kernel(SummaryParams p) {
  using Dm = Dims<D>;
  constexpr int DK = Dm::DK, NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int LPR = D / 8;               // threads per token row
  constexpr int TG_ALL = kThreads / LPR;   // token groups the workgroup could cover
  constexpr int TG = TG_ALL < 32 ? TG_ALL : 32;   // token groups of 8 per round (<= 256 tokens)
  constexpr int ROUND = TG * 8;            // tokens per round
  constexpr int PITCH = ROUND + 8;         // LDS row pitch in bf16 elements (16-byte pad)
  // MFMA work split: waves form WR x WC over (32-feature chunks, 16-channel tiles).
  constexpr int WR = NKC >= 2 ? 2 : 1;
  constexpr int WC = NCT >= 2 ? 2 : 1;
  constexpr int KCW = NKC / WR;
  constexpr int CTW = NCT / WC;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* kt_hi = smem;                                   // [DK][PITCH]
  uint16_t* kt_lo = kt_hi + DK * PITCH;                     // [DK][PITCH]   (SPLIT_K)
  uint16_t* vt_hi = kt_lo + (SPLIT_K ? DK * PITCH : 0);     // [D][PITCH]
  uint16_t* vt_lo = vt_hi + D * PITCH;                      // [D][PITCH]    (SPLIT_V)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int blk = blockIdx.y;
  const int bh = blockIdx.z;
  const Geom& g = p.g;

  const int fgrp = tid % LPR;              // features [8*fgrp, 8*fgrp+8)
  const int tgrp = tid / LPR;              // tokens [8*tgrp, 8*tgrp+8) of each round
  const bool loader = tgrp < TG;           // small D: some threads only help with MFMA

  const int32_t j_begin = split * p.tok_per_split;
  const int32_t j_end = min(j_begin + p.tok_per_split, g.n_b);
  const int32_t base_tok = block_base_token(g, blk);
  const int64_t head_off = (int64_t)bh * g.N * D;

  if (DK > D) {  // key rows beyond D stay zero for the whole kernel
    for (int i = tid; i < (DK - D) * PITCH; i += kThreads) {
      kt_hi[D * PITCH + i] = 0;
      if (SPLIT_K) kt_lo[D * PITCH + i] = 0;
    }
  }

  In8<TIn> rk[8], rv[8];
  auto issue_loads = [&](int32_t round_base) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t j = round_base + 8 * tgrp + i;
      if (loader && j < j_end) {
        const int64_t t = base_tok + block_token_offset(g, (uint32_t)j);
        const int64_t idx = head_off + t * D + 8 * fgrp;
        rk[i].load(p.k, idx);
        rv[i].load(p.v, idx);
      } else {
        rk[i].zero();
        rv[i].zero();
      }
    }
  };

  float zacc[8], uacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { zacc[e] = 0.f; uacc[e] = 0.f; }

  f32x4_t acc[KCW][2][CTW];
#pragma unroll
  for (int a = 0; a < KCW; ++a)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < CTW; ++c) acc[a][r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bool mfma_wave = wave < WR * WC;
  const int wr = wave / WC, wc = wave % WC;

  issue_loads(j_begin);
  for (int32_t rb = j_begin; rb < j_end; rb += ROUND) {
    // ---- phi, split, transpose into LDS --------------------------------------------------
    if (loader) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int f = 8 * fgrp + e;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool valid = rb + 8 * tgrp + i < j_end;
        x[i] = valid ? phi_elu1(rk[i].get(e)) : 0.f;   // padding is zero AFTER phi
        zacc[e] += x[i];
      }
      u32x4_t hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (SPLIT_K) {
          uint32_t h0, l0, h1, l1;
          split_bf16(x[2 * i], h0, l0);
          split_bf16(x[2 * i + 1], h1, l1);
          hi[i] = h0 | (h1 << 16);
          lo[i] = l0 | (l1 << 16);
        } else {
          hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        }
      }
      *reinterpret_cast<u32x4_t*>(kt_hi + f * PITCH + 8 * tgrp) = hi;
      if (SPLIT_K) *reinterpret_cast<u32x4_t*>(kt_lo + f * PITCH + 8 * tgrp) = lo;

      u32x4_t vh, vl;
      if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vh[i] = rv[2 * i].bits(e) | (rv[2 * i + 1].bits(e) << 16);   // exact: no rounding
        if (WANT_U) {
#pragma unroll
          for (int i = 0; i < 8; ++i) uacc[e] += rv[i].get(e);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = rv[2 * i].get(e), v1 = rv[2 * i + 1].get(e);
          if (WANT_U) uacc[e] += v0 + v1;
          if (SPLIT_V) {
            uint32_t h0, l0, h1, l1;
            split_bf16(v0, h0, l0);
            split_bf16(v1, h1, l1);
            vh[i] = h0 | (h1 << 16);
            vl[i] = l0 | (l1 << 16);
          } else {
            vh[i] = pack_bf16x2(v0, v1);
          }
        }
      }
      *reinterpret_cast<u32x4_t*>(vt_hi + f * PITCH + 8 * tgrp) = vh;
      if (SPLIT_V) *reinterpret_cast<u32x4_t*>(vt_lo + f * PITCH + 8 * tgrp) = vl;
    }
    }
    __syncthreads();

    const int32_t valid_round = min(ROUND, j_end - rb);
    if (rb + ROUND < j_end) issue_loads(rb + ROUND);

    // ---- MFMA: S_quadrant += phi(K)^T V over this round --------------------------------
    if (mfma_wave) {
      const int nsteps = (valid_round + 31) >> 5;
      const int pr = lane & 15, lg = lane >> 4;
      for (int ks = 0; ks < nsteps; ++ks) {
        const int tok = 32 * ks + 8 * lg;
        u32x4_t a_hi[KCW][2], a_lo[KCW][2], b_hi[CTW], b_lo[CTW];
#pragma unroll
        for (int a = 0; a < KCW; ++a) {
          const int kc = wr * KCW + a;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int f = 32 * kc + 8 * (pr >> 2) + 4 * r + (pr & 3);
            a_hi[a][r] = *reinterpret_cast<const u32x4_t*>(kt_hi + f * PITCH + tok);
            if (SPLIT_K) a_lo[a][r] = *reinterpret_cast<const u32x4_t*>(kt_lo + f * PITCH + tok);
          }
        }
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
          const int ch = 16 * (wc * CTW + c) + pr;
          b_hi[c] = *reinterpret_cast<const u32x4_t*>(vt_hi + ch * PITCH + tok);
          if (SPLIT_V) b_lo[c] = *reinterpret_cast<const u32x4_t*>(vt_lo + ch * PITCH + tok);
        }
#pragma unroll
        for (int a = 0; a < KCW; ++a)
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
              acc[a][r][c] = mfma_bf16(a_hi[a][r], b_hi[c], acc[a][r][c]);
              if (SPLIT_K) acc[a][r][c] = mfma_bf16(a_lo[a][r], b_hi[c], acc[a][r][c]);
              if (SPLIT_V) acc[a][r][c] = mfma_bf16(a_hi[a][r], b_lo[c], acc[a][r][c]);
            }
      }
    }
    __syncthreads();
  }

  // ---- write the partial summary in fragment layout ------------------------------------
  const int64_t slot = ((int64_t)bh * g.M + blk) * p.splits + split;
  if (mfma_wave) {
#pragma unroll
    for (int a = 0; a < KCW; ++a)
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        const int kc = wr * KCW + a, ct = wc * CTW + c;
        const int off = ((kc * NCT + ct) * 64 + lane) * 8;
        const f32x4_t r0 = acc[a][0][c], r1 = acc[a][1][c];
        if constexpr (OUT_BF16) {   // one token slice: the bf16 stack feeds the MFMA mixing
          st16(p.sb + slot * FRAG + off,
               u32x4_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]),
                       pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])});
        } else {
          float* dst = p.ps + slot * FRAG + off;
          st16(dst, __builtin_bit_cast(u32x4_t, r0));
          st16(dst + 4, __builtin_bit_cast(u32x4_t, r1));
        }
      }
  }

  // ---- deterministic reduction of z (and u) over the token groups ----------------------
  float* red = reinterpret_cast<float*>(smem);          // [TG][D] (aliases the key planes)
  float* red_u = red + TG * D;
  __syncthreads();
  if (loader) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[tgrp * D + 8 * fgrp + e] = zacc[e];
      if (WANT_U) red_u[tgrp * D + 8 * fgrp + e] = uacc[e];
    }
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f, su = 0.f;
    for (int t = 0; t < TG; ++t) {
      s += red[t * D + tid];
      if (WANT_U) su += red_u[t * D + tid];
    }
    p.pz[slot * D + tid] = s;
    if (WANT_U) p.pu[slot * D + tid] = su;
  }
}

template <typename TIn, int D, bool SPLIT_K, bool SPLIT_V, bool WANT_U, bool OUT_BF16 = false>
static hipError_t launch_summary_t(const SummaryParams& p, dim3 grid, hipStream_t stream) {
  using Dm = Dims<D>;
  constexpr int LPR = D / 8, TG_ALL = kThreads / LPR, TG = TG_ALL < 32 ? TG_ALL : 32;
  constexpr int ROUND = TG * 8, PITCH = ROUND + 8;
  size_t lds = (size_t)(Dm::DK * (SPLIT_K ? 2 : 1) + D * (SPLIT_V ? 2 : 1)) * PITCH * 2;
  const size_t red = (size_t)TG * D * 4 * (WANT_U ? 2 : 1);
  if (red > lds) lds = red;
  auto kern = summary_kernel<TIn, D, SPLIT_K, SPLIT_V, WANT_U, OUT_BF16>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t dispatch_flags(const SummaryParams& p, bool split_k, bool split_v, bool want_u,
                                 bool out_bf16, dim3 grid, hipStream_t s) {
  if constexpr (sizeof(TIn) == 2) {
    if (split_v) return hipErrorInvalidValue;   // bf16 V is exact: never split
    if (out_bf16) {
      if (split_k || want_u) return hipErrorInvalidValue;
      return launch_summary_t<TIn, D, false, false, false, true>(p, grid, s);
    }
    if (split_k)
      return want_u ? launch_summary_t<TIn, D, true, false, true>(p, grid, s)
                    : launch_summary_t<TIn, D, true, false, false>(p, grid, s);
    return want_u ? launch_summary_t<TIn, D, false, false, true>(p, grid, s)
                  : launch_summary_t<TIn, D, false, false, false>(p, grid, s);
  } else {
    if (split_k != split_v || out_bf16) return hipErrorInvalidValue;
    if (split_k)
      return want_u ? launch_summary_t<TIn, D, true, true, true>(p, grid, s)
                    : launch_summary_t<TIn, D, true, true, false>(p, grid, s);
    return want_u ? launch_summary_t<TIn, D, false, false, true>(p, grid, s)
                  : launch_summary_t<TIn, D, false, false, false>(p, grid, s);
  }
}

template <typename TIn>
static hipError_t dispatch_d(const SummaryParams& p, int d, bool sk, bool sv, bool wu, bool ob,
                             dim3 grid, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_flags<TIn, 16>(p, sk, sv, wu, ob, grid, s);
    case 32: return dispatch_flags<TIn, 32>(p, sk, sv, wu, ob, grid, s);
    case 64: return dispatch_flags<TIn, 64>(p, sk, sv, wu, ob, grid, s);
    case 128: return dispatch_flags<TIn, 128>(p, sk, sv, wu, ob, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_summary(const SummaryParams& p, int d, bool in_fp32, bool split_k, bool split_v,
                          bool want_u, bool out_bf16, dim3 grid, hipStream_t stream) {
  return in_fp32 ? dispatch_d<float>(p, d, split_k, split_v, want_u, out_bf16, grid, stream)
                 : dispatch_d<uint16_t>(p, d, split_k, split_v, want_u, out_bf16, grid, stream);
}

}  // namespace mhla
