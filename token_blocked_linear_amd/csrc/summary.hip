// Summary kernel: phi(K) in registers, per-block S_b = sum_j phi(K_j) V_j^T on bf16 MFMA with
// fp32 accumulation, z_b = sum_j phi(K_j) (and, for the MALA readout, u = sum_j V_j).
//
// Source: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Method -> Overall framework (local KV summary S_b and normaliser z_b of every block); the
// MALA linear form in "Rectifying Magnitude Neglect in Linear Attention", Method -> Key design,
// also needs sum_j V_j.
//
// Work units are (batch*head, block, token slice); the grid is persistent and each workgroup
// (4 wave64s) strides over units.  Tokens stream in rounds of up to 256: every thread owns 8
// consecutive block-local tokens x 8 consecutive features, issues one 16-byte load per token
// row (D/8 lanes cover a row, so each load instruction reads whole rows), applies phi in fp32,
// and transposes its 8x8 piece in registers so that LDS holds phi(K)^T and V^T with tokens
// contiguous (one 16-byte LDS write per feature).  The MFMA phase reads every operand with one
// 16-byte LDS read.  The next round's loads -- of this unit or the next one -- are in flight
// during the MFMA phase.  z (and u) come from the same MFMAs against an all-ones operand, so
// they carry exactly the operands' rounding and need no cross-thread reduction.
#include <type_traits>

#include "mhla_device.hpp"

namespace mhla {

// TV, the element type of V, is TIn except in the backward, which feeds Q as K and dO (the
// output's type) as V.  TOKW (backward): phi(K_j) is scaled by kscale[j] and the normaliser
// product weights token j by zw[j] instead of 1, so that S = sum_j kscale_j phi(K_j) V_j^T and
// z = sum_j kscale_j zw_j phi(K_j).
// Token groups of 8 per round: as many as the workgroup's threads cover, at most 32 (256 tokens).
// With phi(K) split (hi and lo planes of phi(K)^T in LDS) and bf16 inputs at d <= 64 the rounds
// are shorter (192 tokens: 72 KB of LDS at d = 64, two workgroups per CU instead of one with
// 256-token rounds; MALA image summary 56.6 -> 44.5 us).
#ifndef MHLA_SUMMARY_SPLIT_TG
#define MHLA_SUMMARY_SPLIT_TG 24
#endif
template <typename TIn, int D, bool SPLIT_K>
constexpr int summary_tg() {
  constexpr int all = kThreads / (D / 8);
  constexpr int cap = (SPLIT_K && sizeof(TIn) == 2 && D <= 64) ? MHLA_SUMMARY_SPLIT_TG : 32;
  return all < cap ? all : cap;
}

template <typename TIn, int D, bool SPLIT_K, bool SPLIT_V, bool WANT_U, bool OUT_BF16, int PHI, typename TV,
          bool TOKW>
__global__ __launch_bounds__(kThreads) void summary_kernel(SummaryParams p, int n_units) {
  using Dm = Dims<D>;
  constexpr int DK = Dm::DK, NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int LPR = D / 8;               // threads per token row
  constexpr int TG = summary_tg<TIn, D, SPLIT_K>();   // token groups of 8 per round (<= 256 tokens)
  constexpr int ROUND = TG * 8;            // tokens per round
  constexpr int PITCH = ROUND;             // LDS row pitch (bf16 elements): rows start on 128 B
  static_assert(ROUND >= 64, "the chunk swizzle needs at least 8 chunks per row");
  // MFMA work split: waves form WR x WC over (32-feature chunks, 16-channel tiles).
  constexpr int WR = NKC >= 2 ? 2 : 1;
  constexpr int WC = NCT >= 2 ? 2 : 1;
  constexpr int KCW = NKC / WR;
  constexpr int CTW = NCT / WC;
  constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 1.0
  // LDS bank swizzle: the 16-byte token chunk c of row f lives at chunk c ^ h(f).  phi(K)^T
  // rows are written 8 rows apart (f = 8*fgrp + e) and read as rows {b..b+3, b+8..b+11};
  // V^T rows are written 8 apart and read 8 consecutive.  Both h keep any 8 consecutive
  // lanes of either access on 8 distinct 16-byte bank groups.
  auto hk = [](int f) { return ((f >> 3) & 7) ^ ((f & 3) << 1); };
  auto hv = [](int c) { return (c & 7) ^ ((c >> 3) & 7); };

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* kt_hi = smem;                                   // [DK][PITCH]
  uint16_t* kt_lo = kt_hi + DK * PITCH;                     // [DK][PITCH]   (SPLIT_K)
  uint16_t* vt_hi = kt_lo + (SPLIT_K ? DK * PITCH : 0);     // [D][PITCH]
  uint16_t* vt_lo = vt_hi + D * PITCH;                      // [D][PITCH]    (SPLIT_V)
  float* s_zw = reinterpret_cast<float*>(vt_lo + (SPLIT_V ? D * PITCH : 0));   // [ROUND] (TOKW)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const Geom& g = p.g;
  const int fgrp = tid % LPR;              // features [8*fgrp, 8*fgrp+8)
  const int tgrp = tid / LPR;              // tokens [8*tgrp, 8*tgrp+8) of each round
  const bool loader = tgrp < TG;           // small D: some threads only help with MFMA
  const bool mfma_wave = wave < WR * WC;
  const int wr = wave / WC, wc = wave % WC;
  const int pr = lane & 15, lg = lane >> 4;

  if (DK > D) {  // key rows beyond D stay zero for the whole kernel
    for (int i = tid; i < (DK - D) * PITCH; i += kThreads) {
      kt_hi[D * PITCH + i] = 0;
      if (SPLIT_K) kt_lo[D * PITCH + i] = 0;
    }
  }

  // ---- side job: bf16 operand fragments of M_c for the MFMA mixing kernel -----------------
  if (p.mcf) {
    const int nitp = p.mcf_nitp, nbc = p.mcf_nbc, M = g.M;
    const int total = p.mcf_heads * nitp * nbc * 64;      // lane fragments of 8 elements
    for (int idx = blockIdx.x * kThreads + tid; idx < total; idx += gridDim.x * kThreads) {
      const int l = idx & 63;
      int t = idx >> 6;
      const int bc = t % nbc;
      t /= nbc;
      const int it = t % nitp, hh = t / nitp;
      const int i = 16 * it + (l & 15);
      // W[i][b] = M_c[i][b], or M_c[b][i] for the transposed mixing
      const float* mch = p.mc ? p.mc + (int64_t)hh * p.mc_head_stride : nullptr;
      const int64_t si = p.mcf_transposed ? 1 : M, sb = p.mcf_transposed ? M : 1;
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int b = 32 * bc + 8 * (l >> 4) + e;
        m[e] = (i < M && b < M && !(p.mcf_causal && b >= i)) ? (mch ? mch[i * si + b * sb] : 1.0f)
                                                               : 0.f;   // NULL M_c (M == 1): [1]
      }
      u32x4_t hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h, l;
        split_bf16x2(m[2 * j], m[2 * j + 1], h, l);
        hi[j] = h;
        lo[j] = l;
      }
      st16(p.mcf + (int64_t)idx * 8, hi);
      if (p.mcf_lo) st16(p.mcf_lo + (int64_t)idx * 8, lo);
    }
  }

  // ---- unit bookkeeping --------------------------------------------------------------------
  struct Unit {
    int split, blk, bh;
    int32_t j_begin, j_end, base_tok;
    int64_t head_off;
    BlockGeo bg;
  };
  auto make_unit = [&](int u) {
    Unit U;
    U.split = u % p.splits;
    const int t = u / p.splits;
    U.blk = t % g.M;
    U.bh = t / g.M;
    U.j_begin = U.split * p.tok_per_split;
    U.bg = block_geo(g, U.blk);
    U.j_end = min(U.j_begin + p.tok_per_split, U.bg.n);
    U.base_tok = U.bg.base;
    U.head_off = (int64_t)U.bh * g.N * D;
    return U;
  };

  // When the block's last extent is a multiple of 8, a thread's 8 block-local tokens
  // j0..j0+7 (j0 a multiple of 8) lie in one grid row: their rows are consecutive in memory
  // and one index computation serves all 8 loads.  (Per unit: a ragged edge block may not.)
  // The token-weight loads there read 16 bytes at token t0 and need t0 a multiple of 4:
  // t0 = base + row * G2 + (multiple of 8), so base and G2 must be.
  auto contig8_of = [&](const Unit& U) {
    return (U.bg.e2 & 7) == 0 && (!TOKW || ((U.bg.base & 3) == 0 && (g.G2 & 3) == 0));
  };

  // Loads of one round into a register buffer.  Rows of tokens past the unit's end are zero:
  // they add nothing to S (their V is zero) and z masks them explicitly.
  // Loads go through buffer resources spanning one head; rows past the unit's end get an
  // out-of-range offset and read as zero, with no branch around the loads.
  constexpr uint32_t ES = sizeof(TIn), ESV = sizeof(TV);
  const uint32_t head_bytes = (uint32_t)g.N * D * ES, head_bytes_v = (uint32_t)g.N * D * ESV;
  // tw (TOKW): kscale of the thread's 8 tokens in tw[0..7], zw in tw[8..15]; 0 past the end
  auto issue_loads = [&](In8<TIn> (&rk)[8], In8<TV> (&rv)[8], float (&tw)[16], const Unit& U,
                         int32_t round_base) {
    const Rsrc rsk = make_rsrc(reinterpret_cast<const TIn*>(p.k) + U.head_off, head_bytes);
    const Rsrc rsv = make_rsrc(reinterpret_cast<const TV*>(p.v) + U.head_off, head_bytes_v);
    const int32_t j0 = round_base + 8 * tgrp;
    if (contig8_of(U)) {
      const bool ok = loader && j0 < U.j_end;
      const uint32_t t0 = ok ? (uint32_t)(U.base_tok + block_offset(g, U.bg, (uint32_t)j0)) : 0u;
      const uint32_t e0 = t0 * D + 8 * fgrp;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rk[i].template load_buf<MHLA_SUMMARY_LOAD_CPOL>(rsk, ok ? (e0 + (uint32_t)(i * D)) * ES : kOutOfRange);
        rv[i].template load_buf<MHLA_SUMMARY_LOAD_CPOL>(rsv, ok ? (e0 + (uint32_t)(i * D)) * ESV : kOutOfRange);
      }
      if constexpr (TOKW) {
        // t0 is a multiple of 4 here, and j_end a multiple of 8 (the block's last extent and the
        // slice length are): the 8 tokens are all in the unit or all past its end
        const Rsrc rs = make_rsrc(p.kscale + (int64_t)U.bh * g.N, (uint32_t)g.N * 4u);
        const Rsrc rz = make_rsrc(p.zw + (int64_t)U.bh * g.N, (uint32_t)g.N * 4u);
        const u32x4_t s0 = buf_ld16(rs, ok ? t0 * 4u : kOutOfRange), s1 = buf_ld16(rs, ok ? t0 * 4u + 16u : kOutOfRange);
        const u32x4_t z0 = buf_ld16(rz, ok ? t0 * 4u : kOutOfRange), z1 = buf_ld16(rz, ok ? t0 * 4u + 16u : kOutOfRange);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tw[i] = __uint_as_float(s0[i]);
          tw[4 + i] = __uint_as_float(s1[i]);
          tw[8 + i] = __uint_as_float(z0[i]);
          tw[12 + i] = __uint_as_float(z1[i]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t j = j0 + i;
        const bool ok = loader && j < U.j_end;
        const uint32_t t = ok ? (uint32_t)(U.base_tok + block_offset(g, U.bg, (uint32_t)j)) : 0u;
        const uint32_t e = t * D + 8 * fgrp;
        rk[i].template load_buf<MHLA_SUMMARY_LOAD_CPOL>(rsk, ok ? e * ES : kOutOfRange);
        rv[i].template load_buf<MHLA_SUMMARY_LOAD_CPOL>(rsv, ok ? e * ESV : kOutOfRange);
        if constexpr (TOKW) {
          const int64_t ti = (int64_t)U.bh * g.N + t;
          tw[i] = ok ? p.kscale[ti] : 0.f;
          tw[8 + i] = ok ? p.zw[ti] : 0.f;
        }
      }
    }
  };

  f32x4_t acc[KCW][2][CTW], accz[KCW][2], accu[CTW];
  auto reset = [&]() {
#pragma unroll
    for (int a = 0; a < KCW; ++a)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        accz[a][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CTW; ++c) acc[a][r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int c = 0; c < CTW; ++c) accu[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  reset();

  // One round: phi / split / transpose into LDS, MFMAs, and the unit's epilogue if it ends.
  // `after_lds` runs once the round's registers are in LDS (single-buffer refill point).
  auto process = [&](const In8<TIn> (&rk)[8], const In8<TV> (&rv)[8], const float (&tw)[16], const Unit& U,
                     int32_t rb, auto&& after_lds) {
    if (loader) {
      if (TOKW && fgrp == 0) {   // the round's normaliser weights, one writer per token group
        st16(s_zw + 8 * tgrp, u32x4_t{__float_as_uint(tw[8]), __float_as_uint(tw[9]), __float_as_uint(tw[10]),
                                      __float_as_uint(tw[11])});
        st16(s_zw + 8 * tgrp + 4, u32x4_t{__float_as_uint(tw[12]), __float_as_uint(tw[13]),
                                          __float_as_uint(tw[14]), __float_as_uint(tw[15])});
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = 8 * fgrp + e;
        u32x4_t hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x0 = phi_map<PHI>(rk[2 * i].get(e)), x1 = phi_map<PHI>(rk[2 * i + 1].get(e));
          if (TOKW) {
            x0 *= tw[2 * i];
            x1 *= tw[2 * i + 1];
          }
          if (SPLIT_K) {
            uint32_t h, l;
            split_bf16x2(x0, x1, h, l);
            hi[i] = h;
            lo[i] = l;
          } else {
            hi[i] = pack_bf16x2(x0, x1);
          }
        }
        const int kofs = f * PITCH + 8 * (tgrp ^ hk(f));
        *reinterpret_cast<u32x4_t*>(kt_hi + kofs) = hi;
        if (SPLIT_K) *reinterpret_cast<u32x4_t*>(kt_lo + kofs) = lo;

        u32x4_t vh, vl;
        if constexpr (sizeof(TV) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vh[i] = rv[2 * i].bits(e) | (rv[2 * i + 1].bits(e) << 16);   // exact: no rounding
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = rv[2 * i].get(e), v1 = rv[2 * i + 1].get(e);
            if (SPLIT_V) {
              uint32_t h, l;
              split_bf16x2(v0, v1, h, l);
              vh[i] = h;
              vl[i] = l;
            } else {
              vh[i] = pack_bf16x2(v0, v1);
            }
          }
        }
        const int vofs = f * PITCH + 8 * (tgrp ^ hv(f));
        *reinterpret_cast<u32x4_t*>(vt_hi + vofs) = vh;
        if (SPLIT_V) *reinterpret_cast<u32x4_t*>(vt_lo + vofs) = vl;
      }
    }
    __syncthreads();
    after_lds();

    const int32_t valid_round = min(ROUND, U.j_end - rb);
    if (mfma_wave) {
      const int nsteps = (valid_round + 31) >> 5;
      const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
      for (int ks = 0; ks < nsteps; ++ks) {
        const int chunk = 4 * ks + lg;           // 16-byte chunk of tokens 32ks + 8lg ..
        // token validity as the B operand of the z product (phi(0) = 1 on padding rows); with
        // TOKW the tokens' weights instead, split hi (vmask) + lo (wlo); 0 past the end
        u32x4_t vmask = ones, wlo = {0u, 0u, 0u, 0u};
        if constexpr (TOKW) {
          const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(s_zw + 8 * chunk);
          const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(s_zw + 8 * chunk + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4_t& w = i < 2 ? w0 : w1;
            uint32_t h, l;
            split_bf16x2(__uint_as_float(w[(2 * i) & 3]), __uint_as_float(w[(2 * i + 1) & 3]), h, l);
            vmask[i] = h;
            wlo[i] = l;
          }
        } else {
          const int left = valid_round - 8 * chunk;
          if (left < 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              vmask[i] = (2 * i < left ? 0x3f80u : 0u) | (2 * i + 1 < left ? 0x3f800000u : 0u);
          }
        }
        u32x4_t a_hi[KCW][2], a_lo[KCW][2], b_hi[CTW], b_lo[CTW];
#pragma unroll
        for (int a = 0; a < KCW; ++a) {
          const int kc = wr * KCW + a;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int f = 32 * kc + 8 * (pr >> 2) + 4 * r + (pr & 3);
            const int ofs = f * PITCH + 8 * (chunk ^ hk(f));
            a_hi[a][r] = *reinterpret_cast<const u32x4_t*>(kt_hi + ofs);
            if (SPLIT_K) a_lo[a][r] = *reinterpret_cast<const u32x4_t*>(kt_lo + ofs);
          }
        }
#pragma unroll
        for (int c = 0; c < CTW; ++c) {
          const int ch = 16 * (wc * CTW + c) + pr;
          const int ofs = ch * PITCH + 8 * (chunk ^ hv(ch));
          b_hi[c] = *reinterpret_cast<const u32x4_t*>(vt_hi + ofs);
          if (SPLIT_V) b_lo[c] = *reinterpret_cast<const u32x4_t*>(vt_lo + ofs);
        }
#pragma unroll
        for (int a = 0; a < KCW; ++a)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int c = 0; c < CTW; ++c) {
              acc[a][r][c] = mfma_bf16(a_hi[a][r], b_hi[c], acc[a][r][c]);
              if (SPLIT_K) acc[a][r][c] = mfma_bf16(a_lo[a][r], b_hi[c], acc[a][r][c]);
              if (SPLIT_V) acc[a][r][c] = mfma_bf16(a_hi[a][r], b_lo[c], acc[a][r][c]);
            }
            if (wc == 0) {
              accz[a][r] = mfma_bf16(a_hi[a][r], vmask, accz[a][r]);
              if (SPLIT_K) accz[a][r] = mfma_bf16(a_lo[a][r], vmask, accz[a][r]);
              if (TOKW) accz[a][r] = mfma_bf16(a_hi[a][r], wlo, accz[a][r]);
            }
          }
        if (WANT_U && wr == 0) {
#pragma unroll
          for (int c = 0; c < CTW; ++c) {
            accu[c] = mfma_bf16(ones, b_hi[c], accu[c]);
            if (SPLIT_V) accu[c] = mfma_bf16(ones, b_lo[c], accu[c]);
          }
        }
      }
    }

    // ---- unit epilogue: summary in fragment layout, z, u ------------------------------
    if (rb + ROUND >= U.j_end && mfma_wave) {
      const int64_t slot = ((int64_t)U.bh * g.M + U.blk) * p.splits + U.split;
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
      // z: every column of the validity product holds the row sum; lanes of column 0 store.
      // Row 4g + r of row tile (kc, rt) is key feature 32*kc + 8g + 4*rt + r.
      if (wc == 0 && pr == 0) {
#pragma unroll
        for (int a = 0; a < KCW; ++a)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int f = 32 * (wr * KCW + a) + 8 * lg + 4 * r;
            if (f < D) st16(p.pz + slot * D + f, __builtin_bit_cast(u32x4_t, accz[a][r]));
          }
      }
      // u: every row of the ones-product holds the column sum; lanes of row group 0 store.
      if (WANT_U && wr == 0 && lg == 0) {
#pragma unroll
        for (int c = 0; c < CTW; ++c) p.pu[slot * D + 16 * (wc * CTW + c) + pr] = accu[c][0];
      }
      reset();
    }
    __syncthreads();
  };

  // Advance (unit, round) -> the next round of this unit or the first round of the next unit.
  auto advance = [&](int& unit, Unit& U, int32_t& rb) {
    if (rb + ROUND < U.j_end) {
      rb += ROUND;
    } else {
      unit += gridDim.x;
      if (unit < n_units) {
        U = make_unit(unit);
        rb = U.j_begin;
      }
    }
  };

  int unit = blockIdx.x;
  if (unit >= n_units) return;
  Unit U = make_unit(unit);
  int32_t rb = U.j_begin;

  auto nothing = [] {};
  if constexpr (sizeof(TIn) == 2 && sizeof(TV) == 2 && D <= 64) {
    // Two register buffers: the loads of round r+1 are in flight while round r goes through
    // phi, LDS and MFMA.
    In8<TIn> ka[8], kb[8];
    In8<TV> va[8], vb[8];
    float twa[16], twb[16];
    issue_loads(ka, va, twa, U, rb);
    while (true) {
      int nu = unit;
      Unit NU = U;
      int32_t nrb = rb;
      advance(nu, NU, nrb);
      if (nu < n_units) issue_loads(kb, vb, twb, NU, nrb);
      process(ka, va, twa, U, rb, nothing);
      if (nu >= n_units) break;
      unit = nu;
      U = NU;
      rb = nrb;
      advance(nu, NU, nrb);
      if (nu < n_units) issue_loads(ka, va, twa, NU, nrb);
      process(kb, vb, twb, U, rb, nothing);
      if (nu >= n_units) break;
      unit = nu;
      U = NU;
      rb = nrb;
    }
  } else {
    // One buffer (d = 128 would spill two; fp32 inputs are twice as wide): refilled as soon as
    // the round sits in LDS, so the loads overlap the MFMA phase.
    In8<TIn> ka[8];
    In8<TV> va[8];
    float twa[16];
    issue_loads(ka, va, twa, U, rb);
    while (true) {
      int nu = unit;
      Unit NU = U;
      int32_t nrb = rb;
      advance(nu, NU, nrb);
      process(ka, va, twa, U, rb, [&] {
        if (nu < n_units) issue_loads(ka, va, twa, NU, nrb);
      });
      if (nu >= n_units) break;
      unit = nu;
      U = NU;
      rb = nrb;
    }
  }
}

template <int PHI, typename TIn, int D, bool SPLIT_K, bool SPLIT_V, bool WANT_U, bool OUT_BF16 = false,
          typename TV = TIn, bool TOKW = false>
static hipError_t launch_summary_t(const SummaryParams& p, int n_units, hipStream_t stream) {
  using Dm = Dims<D>;
  constexpr int TG = summary_tg<TIn, D, SPLIT_K>();
  constexpr int ROUND = TG * 8, PITCH = ROUND;
  const size_t lds = (size_t)(Dm::DK * (SPLIT_K ? 2 : 1) + D * (SPLIT_V ? 2 : 1)) * PITCH * 2 +
                    (TOKW ? (size_t)ROUND * 4 : 0);
  auto kern = summary_kernel<TIn, D, SPLIT_K, SPLIT_V, WANT_U, OUT_BF16, PHI, TV, TOKW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  // persistent grid: as many workgroups as fit on the chip at once (LDS-limited), at most
  // one per unit
  const int per_cu = (int)(160 * 1024 / lds) < 1 ? 1 : (int)(160 * 1024 / lds);
  int grid = 256 * (per_cu > 4 ? 4 : per_cu);
  if (grid > n_units) grid = n_units;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, p, n_units);
  return hipGetLastError();
}

template <int PHI, typename TIn, int D>
static hipError_t dispatch_flags(const SummaryParams& p, bool split_k, bool split_v, bool want_u,
                                 bool out_bf16, int n, hipStream_t s) {
  if constexpr (sizeof(TIn) == 2) {
    if (split_v) return hipErrorInvalidValue;   // bf16 V is exact: never split
    if (out_bf16) {
      if (split_k || want_u) return hipErrorInvalidValue;
      return launch_summary_t<PHI, TIn, D, false, false, false, true>(p, n, s);
    }
    if (split_k)
      return want_u ? launch_summary_t<PHI, TIn, D, true, false, true>(p, n, s)
                    : launch_summary_t<PHI, TIn, D, true, false, false>(p, n, s);
    return want_u ? launch_summary_t<PHI, TIn, D, false, false, true>(p, n, s)
                  : launch_summary_t<PHI, TIn, D, false, false, false>(p, n, s);
  } else {
    if (split_k != split_v || out_bf16) return hipErrorInvalidValue;
    if (split_k)
      return want_u ? launch_summary_t<PHI, TIn, D, true, true, true>(p, n, s)
                    : launch_summary_t<PHI, TIn, D, true, true, false>(p, n, s);
    return want_u ? launch_summary_t<PHI, TIn, D, false, false, true>(p, n, s)
                  : launch_summary_t<PHI, TIn, D, false, false, false>(p, n, s);
  }
}

template <int PHI, typename TIn>
static hipError_t dispatch_d(const SummaryParams& p, int d, bool sk, bool sv, bool wu, bool ob,
                             int n, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_flags<PHI, TIn, 16>(p, sk, sv, wu, ob, n, s);
    case 32: return dispatch_flags<PHI, TIn, 32>(p, sk, sv, wu, ob, n, s);
    case 64: return dispatch_flags<PHI, TIn, 64>(p, sk, sv, wu, ob, n, s);
    case 128: return dispatch_flags<PHI, TIn, 128>(p, sk, sv, wu, ob, n, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_summary_dma(const SummaryParams& p, int d, bool split_k, bool want_u, bool out_bf16, int phi,
                              int n_units, hipStream_t stream);

// bf16 inputs stream through LDS (summary_dma.hip) at d = 32 and 64, and at d = 128 when phi(K) is
// split (here its hi and lo planes would leave one workgroup per CU); fp32 inputs, d = 16 and the
// single-operand d = 128 summary run here (on the long-sequence workload this kernel's register
// buffer sustains 123 us against 132 us for the LDS ring, whose load stream alone takes 114 us).
#ifndef MHLA_SUMMARY_DMA
#define MHLA_SUMMARY_DMA 1
#endif

// n_units = splits * M * BH work units; the kernel picks its own persistent grid.
hipError_t launch_summary(const SummaryParams& p, int d, bool in_fp32, bool split_k, bool split_v,
                          bool want_u, bool out_bf16, int phi, int n_units, hipStream_t stream) {
  if (MHLA_SUMMARY_DMA && !in_fp32 && d >= 32 && !split_v && (d <= 64 || split_k))
    return launch_summary_dma(p, d, split_k, want_u, out_bf16, phi, n_units, stream);
  auto go = [&](auto phi_c) {
    constexpr int PHI = decltype(phi_c)::value;
    return in_fp32 ? dispatch_d<PHI, float>(p, d, split_k, split_v, want_u, out_bf16, n_units, stream)
                   : dispatch_d<PHI, uint16_t>(p, d, split_k, split_v, want_u, out_bf16, n_units, stream);
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_summary_dma_tokw(const SummaryParams& p, int d, int phi, int n_units, hipStream_t stream);

// The backward's dS~ = sum_t (phi(q_t) / den_t) dO_t^T and dz~ = sum_t phi(q_t) gden_t, as a
// summary with K := Q scaled per token by kscale = 1/den and V := dO, whose normaliser product
// weights token t by zw = gden_t * den_t = -(dO_t . o_t).  K split; V split when fp32 (bf16 dO
// is exact); fp32 partials; head sizes 32, 64, 128.
hipError_t launch_summary_tokw(const SummaryParams& p, int d, bool in_fp32, bool v_fp32, int phi, int n_units,
                               hipStream_t stream) {
  // bf16 Q and dO stream through the LDS ring (summary_dma.hip), the weights loaded with each stage
  if (MHLA_SUMMARY_DMA && !in_fp32 && !v_fp32 && d >= 32) return launch_summary_dma_tokw(p, d, phi, n_units, stream);
  auto go = [&](auto phi_c) -> hipError_t {
    constexpr int PHI = decltype(phi_c)::value;
    auto by_d = [&](auto tin, auto tv) -> hipError_t {
      using TI = decltype(tin);
      using TV = decltype(tv);
      constexpr bool SV = sizeof(TV) == 4;
      switch (d) {
        case 32: return launch_summary_t<PHI, TI, 32, true, SV, false, false, TV, true>(p, n_units, stream);
        case 64: return launch_summary_t<PHI, TI, 64, true, SV, false, false, TV, true>(p, n_units, stream);
        case 128: return launch_summary_t<PHI, TI, 128, true, SV, false, false, TV, true>(p, n_units, stream);
        default: return hipErrorInvalidValue;
      }
    };
    if (in_fp32) return v_fp32 ? by_d(float{}, float{}) : by_d(float{}, uint16_t{});
    return v_fp32 ? by_d(uint16_t{}, float{}) : by_d(uint16_t{}, uint16_t{});
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhla
