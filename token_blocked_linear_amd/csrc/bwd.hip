// Backward pass of the MHLA forward: gradients of L = sum(dO * O) with respect to Q, K, V and
// M_c.  "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method ->
// Key design 3 trains M_c end to end; the pages give no gradient formulas, so these kernels
// take the chain rule of the forward steps (Overall framework, Key design 2) in reverse:
//   g_t = dO_t / den_t, gden_t = -(dO_t . o_t) / den_t   (normalised; else dO_t, 0)
//   dq~_t = S~_i g_t + z~_i gden_t                         dq_kernel (also 1/den_t, -(dO_t . o_t))
//   dS~_i = sum_{t in i} (q~_t / den_t) dO_t^T              the summary kernel with K := Q scaled
//   dz~_i = sum_{t in i} q~_t gden_t                        per token by 1/den (fp32, then split
//                                                          hi / lo), V := dO, normaliser weights
//                                                          -(dO_t . o_t): no g tensor
//   dS_b = sum_i m_ib dS~_i, dz_b likewise                 the mixing kernel with M_c^T
//   dM_c[i, b] = <dS~_i, S_b> + <dz~_i, z_b>                dmc_kernel, dmc_reduce_kernel
//   dk~_j = dS_b v_j + dz_b, dv_j = dS_b^T k~_j            keyside_kernel
//   dq = dq~ * phi'(q), dk = dk~ * phi'(k).
// MALA ("Rectifying Magnitude Neglect in Linear Attention", Method -> Key design: one block,
// Y_t = u/N + beta_t q~_t^T C with C = S - z u^T / N, s_t = q~_t . z, beta_t = 1 + 1/s_t) takes
// the same kernels with the centred summary in place of S~:
//   p_t = (C^T q~_t) . dO_t, g_t = beta_t dO_t, gden_t = -p_t / s_t^2
//   dq~_t = C g_t + z gden_t                                dq_kernel<MALA>
//   dS = sum_t q~_t g_t^T, dz' = sum_t q~_t gden_t          the summary kernel (kscale = beta_t)
//   dz = dz' - dS u / N, du = -(1/N) sum_t s_t dO_t          mala_stage_kernel (stage 1)
//   dk~_j = dS v_j + dz, dv_j = dS^T k~_j + du              keyside_kernel
// (the centred forms: C g and dz' - dS u / N are the differences that an uncentred S would leave
// to cancel in fp32).
// Every product runs on bf16 MFMA with hi/lo operand splits (about fp32 accuracy).  Head sizes
// 32, 64 and 128.
//
// A summary T staged in fragment layout is the A operand of out[col] = sum_k T[k][col] B[k]
// (frag_lds.hpp).  dq~ = S~ g and dk~ = dS v need the transposed summaries; each workgroup builds
// them in LDS from the staged ones.  Both tile kernels take the per-token operands in the
// readout's layout (lane (t, g) holds features or channels 32c + 8g + 0..7 of token t), and the
// permuted A rows give every lane 8 consecutive outputs of its token, so phi'(x) of the same
// features is in the lane and the stores are 16-byte.
#include <type_traits>

#include "frag_lds.hpp"

namespace mhla {

enum { kBwdNormalized = 0, kBwdUnnormalized = 1, kBwdMala = 2 };

template <int PHI>
__device__ inline float dphi_map(float x) {
  if constexpr (PHI == kPhiRelu) return x > 0.0f ? 1.0f : 0.0f;
  else if constexpr (PHI == kPhiExp) return __expf(x);
  else return x > 0.0f ? 1.0f : __expf(x);
}

// Unit L -> (head, block, token slice), as the readout numbers them.
struct BwdUnit {
  int bh, blk, split;
  int32_t j_begin, j_end, base_tok;
  int n_tiles;
  int64_t head_off, row;
  BlockGeo bg;
};
template <int D>
__device__ inline BwdUnit bwd_unit(const BwdParams& p, int L) {
  const Geom& g = p.g;
  const int per_head = p.splits * g.M;
  int r;
  BwdUnit u;
  if (p.xcd_map) {
    const int xcd = L & 7, s = L >> 3;
    u.bh = (s / per_head) * 8 + xcd;
    r = s % per_head;
  } else {
    u.bh = L / per_head;
    r = L % per_head;
  }
  u.blk = r / p.splits;
  u.split = r % p.splits;
  u.j_begin = u.split * p.tok_per_split;
  u.bg = block_geo(g, u.blk);
  u.j_end = min(u.j_begin + p.tok_per_split, u.bg.n);
  u.base_tok = u.bg.base;
  u.n_tiles = (u.j_end - u.j_begin + 15) >> 4;
  u.head_off = (int64_t)u.bh * g.N * D;
  u.row = (int64_t)u.bh * g.M + u.blk;
  return u;
}

// A fragment-layout summary (hi and lo) from global memory into LDS.
template <int D, int NT>
__device__ inline void stage_frag(const uint16_t* ghi, const uint16_t* glo, uint16_t* s_hi,
                                  uint16_t* s_lo, int tid) {
  constexpr int FRAG = Dims<D>::FRAG, NCT = Dims<D>::NCT;
  constexpr int PER = (FRAG + NT * 8 - 1) / (NT * 8);
  u32x4_t th[PER], tl[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (tid + j * NT) * 8;
    if (i < FRAG) {
      th[j] = ld16(ghi + i);
      tl[j] = ld16(glo + i);
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (tid + j * NT) * 8;
    if (i < FRAG) {
      st16(s_hi + lds_pos<NCT>(i), th[j]);
      st16(s_lo + lds_pos<NCT>(i), tl[j]);
    }
  }
}

// F(T^T) from F(T), both in LDS.  Element (kc, ct, lane, e) of the transposed summary holds
// T[16ct + lane%16][32kc + 8(lane/16) + e].  D >= 32 (no padding rows).
// Work in 8 x 8 blocks: the 8 source chunks of lanes 16g + 8h + j (j = 0..7) of fragment
// (kc, ct) hold T[r0 + e][c0 + j] (r0 = 32kc + 8g, c0 = 16ct + 8h); row r0 + e of the block is
// one destination chunk, so a thread does 8 16-byte reads, an 8 x 8 transpose of 16-bit
// elements in registers and 8 16-byte writes.
template <int D, int NT>
__device__ inline void transpose_frag(const uint16_t* src_hi, const uint16_t* src_lo,
                                      uint16_t* dst_hi, uint16_t* dst_lo, int tid) {
  constexpr int NCT = Dims<D>::NCT, NBLK = Dims<D>::FRAG / 64;
  for (int blk = tid; blk < 2 * NBLK; blk += NT) {   // the hi blocks, then the lo blocks
    const bool lo = blk >= NBLK;
    const int bb = lo ? blk - NBLK : blk;
    const uint16_t* src = lo ? src_lo : src_hi;
    uint16_t* dst = lo ? dst_lo : dst_hi;
    const int h = bb & 1, g = (bb >> 1) & 3, fr = bb >> 3;   // fr = kc * NCT + ct
    const int r0 = 32 * (fr / NCT) + 8 * g, c0 = 16 * (fr % NCT) + 8 * h;
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = *reinterpret_cast<const u32x4_t*>(src + lds_pos<NCT>((fr * 64 + 16 * g + 8 * h + j) * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4_t w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a = v[2 * k][e >> 1], b = v[2 * k + 1][e >> 1];
        w[k] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      const int r = r0 + e;
      const int dchunk = ((c0 >> 5) * NCT + (r >> 4)) * 64 + 16 * ((c0 & 31) >> 3) + (r & 15);
      *reinterpret_cast<u32x4_t*>(dst + lds_pos<NCT>(dchunk * 8)) = w;
    }
  }
}

// out (NCT accumulator tiles, permuted rows) += T^T B with T = the staged summary (hi, lo) and
// B the lane's operands for contraction chunk kc (hi, lo; lo may be zero).  Tiles go in groups
// of four: the group's operand reads are issued together and its MFMAs run in three rounds of
// independent accumulators (hi*hi, lo*hi, hi*lo), so no MFMA waits on the one before it.
template <int D, bool B_LO>
__device__ inline void frag_mfma(f32x4_t (&acc)[Dims<D>::NCT], const uint16_t* s_hi,
                                 const uint16_t* s_lo, AOffsets ao, int kc, u32x4_t bh, u32x4_t bl) {
  constexpr int NCT = Dims<D>::NCT, G = NCT < 4 ? NCT : 4;
#pragma unroll
  for (int c0 = 0; c0 < NCT; c0 += G) {
    u32x4_t ah[G], al[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int ct = c0 + g;
      const int off = (kc * NCT + (ct & ~1)) * 512 + ((ct & 1) ? ao.odd : ao.even);
      ah[g] = *reinterpret_cast<const u32x4_t*>(s_hi + off);
      al[g] = *reinterpret_cast<const u32x4_t*>(s_lo + off);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) acc[c0 + g] = mfma_bf16(ah[g], bh, acc[c0 + g]);
#pragma unroll
    for (int g = 0; g < G; ++g) acc[c0 + g] = mfma_bf16(al[g], bh, acc[c0 + g]);
    if (B_LO) {
#pragma unroll
      for (int g = 0; g < G; ++g) acc[c0 + g] = mfma_bf16(ah[g], bl, acc[c0 + g]);
    }
  }
}

// 8 values of a lane as bf16 hi / lo operand words (x[2i] in the low half of word i).
__device__ inline void split8(const float (&x)[8], u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h, l;
    split_bf16x2(x[2 * i], x[2 * i + 1], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// Value r (0..7) of the lane's output group cgp from permuted accumulator tiles.
template <int NCT>
__device__ inline float acc_out(const f32x4_t (&acc)[NCT], int cgp, int r) {
  return r < 4 ? acc[2 * cgp][r] : acc[2 * cgp + 1][r - 4];
}

// 8 outputs at byte offset `off` of a buffer resource (out of range: dropped)
template <typename T>
__device__ inline void buf_store8(Rsrc r, uint32_t off, const float (&x)[8]) {
  if constexpr (sizeof(T) == 4) {
    buf_st16(r, off, u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
    buf_st16(r, off == kOutOfRange ? kOutOfRange : off + 16u,
             u32x4_t{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
  } else {
    buf_st16(r, off, u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                             pack_bf16x2(x[6], x[7])});
  }
}

// ---- query side: dq, g, dz~ ----------------------------------------------------------------
// Threads per workgroup of the tile kernels: at d = 128 the two staged summaries take 128 KB
// of LDS, one workgroup per CU, so it runs 8 waves instead of 4.
template <int D>
constexpr int bwd_threads() { return D >= 128 ? 512 : kThreads; }

// MALA: the staged summary is C and the normaliser z (see the top of the file); the kernel also
// leaves the unit's sum_t s_t dO_t in du_part.
template <typename TIn, typename TOut, int D, int PHI, bool MALA>
__global__ __launch_bounds__(bwd_threads<D>()) void dq_kernel(BwdParams p, int mode) {
  constexpr int NT = bwd_threads<D>();
  static_assert(D >= 32, "the backward serves head sizes 32, 64 and 128");
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG, ZF = NKC * 512, NG = NCT / 2;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sa_hi = smem;                 // F(S~)
  uint16_t* sa_lo = sa_hi + FRAG;
  uint16_t* sb_hi = sa_lo + FRAG;         // F(S~^T)
  uint16_t* sb_lo = sb_hi + FRAG;
  uint16_t* s_z = sb_lo + FRAG;           // normaliser fragments
  float* s_zt = reinterpret_cast<float*>(s_z + ZF);   // z~ [D]

  const int tid = threadIdx.x, lane = tid & 63, pr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const Geom& geo = p.g;
  const BwdUnit U = bwd_unit<D>(p, blockIdx.x);

  stage_frag<D, NT>(p.st_hi + U.row * FRAG, p.st_lo + U.row * FRAG, sa_hi, sa_lo, tid);
  if (tid < D) s_zt[tid] = p.zt[U.row * D + tid];
  __syncthreads();
  transpose_frag<D, NT>(sa_hi, sa_lo, sb_hi, sb_lo, tid);
  build_zfrag<D>(s_zt, s_z, tid);
  __syncthreads();

  const AOffsets ao = a_offsets(lane);
  constexpr uint32_t ES = sizeof(TIn), EO = sizeof(TOut);
  const Rsrc rq = make_rsrc(reinterpret_cast<const TIn*>(p.q) + U.head_off, (uint32_t)geo.N * D * ES);
  const Rsrc rdo = make_rsrc(reinterpret_cast<const TOut*>(p.dout) + U.head_off, (uint32_t)geo.N * D * EO);

  // Per tile: this lane's token (validity, element offset) and its Q, dO loads.  Two named
  // buffers take turns: the next tile's loads go out after the current tile's MFMAs and before
  // its stores, and a register copy of loaded values (which would wait for them) is never made.
  // The stores go through buffer resources (invalid tokens: out of range, dropped) so that their
  // number is the same on every path and the next wait counts them exactly.
  struct TileBuf {
    In8<TIn> q[NKC];
    In8<TOut> d[NG];
    bool valid;
    uint32_t rel;
  };
  auto load_tile = [&](TileBuf& b, int tile) {
    const int32_t j = U.j_begin + tile * 16 + pr;
    b.valid = tile < U.n_tiles && j < U.j_end;
    b.rel = b.valid ? (uint32_t)(U.base_tok + block_offset(geo, U.bg, (uint32_t)j)) * D : 0u;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      b.q[kc].template load_buf<0>(rq, b.valid ? (b.rel + 32 * kc + 8 * lg) * ES : kOutOfRange);
#pragma unroll
    for (int c = 0; c < NG; ++c)
      b.d[c].template load_buf<0>(rdo, b.valid ? (b.rel + 32 * c + 8 * lg) * EO : kOutOfRange);
  };
  const Rsrc rdq = make_rsrc(reinterpret_cast<TOut*>(p.dq) + U.head_off, (uint32_t)geo.N * D * EO);
  const Rsrc rts = make_rsrc(p.tok_scale + (int64_t)U.bh * geo.N, (uint32_t)geo.N * 4u);
  const Rsrc rtz = make_rsrc(p.tok_zw + (int64_t)U.bh * geo.N, (uint32_t)geo.N * 4u);

  // MALA: this lane's share of sum_t s_t dO_t (its channels 32c + 8lg + r)
  float du_acc[MALA ? NG : 1][8];
#pragma unroll
  for (int c = 0; c < (MALA ? NG : 1); ++c)
#pragma unroll
    for (int r = 0; r < 8; ++r) du_acc[c][r] = 0.f;

  // one tile: `next` is loaded once this tile's MFMAs are issued
  auto process = [&](const TileBuf& cur, TileBuf& next, int next_tile) {
    // phi(q): fp32 values and hi / lo operands
    float ph[NKC][8];
    u32x4_t bqh[NKC], bql[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ph[kc][e] = phi_map<PHI>(cur.q[kc].get(e));
      split8(ph[kc], bqh[kc], bql[kc]);
    }
    // num = S~^T q~, den = q~ . z~
    f32x4_t acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const u32x4_t az = *reinterpret_cast<const u32x4_t*>(s_z + (kc * 64 + lane) * 8);
      accz = mfma_bf16(az, bqh[kc], accz);
      accz = mfma_bf16(az, bql[kc], accz);
      frag_mfma<D, true>(acc, sa_hi, sa_lo, ao, kc, bqh[kc], bql[kc]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float den = accz[0] + accz[1];

    // g and gden over the lane's channels 32c + 8lg + r; the dot dO . o is completed across the
    // four lanes of the token
    float g[NG][8];
    float gden = 0.f, inv = 1.0f, part = 0.f, zw = 0.f;
    if constexpr (MALA) {
      // den = s_t, acc = C^T q~_t; part = p_t; kscale = beta_t, zw = gden_t / beta_t
      const float is = 1.0f / den;
      inv = 1.0f + is;
#pragma unroll
      for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float d_o = cur.d[c].get(r);
          part = fmaf(d_o, acc_out<NCT>(acc, c, r), part);
          g[c][r] = d_o * inv;
          if (cur.valid) du_acc[c][r] = fmaf(den, d_o, du_acc[c][r]);
        }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      gden = -part * is * is;
      zw = gden / inv;
    } else if (mode == kBwdNormalized) {
      inv = 1.0f / den;
#pragma unroll
      for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float d_o = cur.d[c].get(r);
          part = fmaf(d_o, acc_out<NCT>(acc, c, r) * inv, part);
          g[c][r] = d_o * inv;
        }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      gden = -part * inv;
      zw = -part;
    } else {
#pragma unroll
      for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) g[c][r] = cur.d[c].get(r);
    }
    if (!cur.valid) {                 // tokens past the slice contribute nothing
      gden = 0.f;
#pragma unroll
      for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) g[c][r] = 0.f;
    }

    // dq~ = S~ g + z~ gden: contraction over channels, chunk c = the lane's channel group c
    f32x4_t acc2[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc2[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      u32x4_t bgh, bgl;
      split8(g[c], bgh, bgl);
      frag_mfma<D, true>(acc2, sb_hi, sb_lo, ao, c, bgh, bgl);
      __builtin_amdgcn_sched_barrier(0);
    }

    load_tile(next, next_tile);

#pragma unroll
    for (int c = 0; c < NG; ++c) {
      const int f0 = 32 * c + 8 * lg;
      float out[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        out[r] = (acc_out<NCT>(acc2, c, r) + s_zt[f0 + r] * gden) * dphi_map<PHI>(cur.q[c].get(r));
      buf_store8<TOut>(rdq, cur.valid ? (cur.rel + f0) * EO : kOutOfRange, out);
    }
    // the token's weights for dS~ and dz~ (kscale = 1/den, zw = gden * den = -(dO . o); MALA:
    // beta and gden / beta), one lane per token
    const uint32_t toff = (cur.valid && lg == 0) ? (cur.rel / D) * 4u : kOutOfRange;
    buf_st4(rts, toff, __float_as_uint(inv));
    buf_st4(rtz, toff, __float_as_uint(zw));
  };

  constexpr int STEP = NT / 64;
  TileBuf bufA, bufB;
  load_tile(bufA, wave);
  for (int tile = wave; tile < U.n_tiles; tile += 2 * STEP) {
    process(bufA, bufB, tile + STEP);
    if (tile + STEP >= U.n_tiles) break;
    process(bufB, bufA, tile + 2 * STEP);
  }

  if constexpr (MALA) {
    // the unit's sum_t s_t dO_t: over the 16 token lanes of each lane group, then over the waves
    // (through LDS, once every wave is done with the staged summaries)
    __syncthreads();
    float* s_red = reinterpret_cast<float*>(smem);   // [NT / 64][D]
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float x = du_acc[c][r];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if (pr == 0) s_red[wave * D + 32 * c + 8 * lg + r] = x;
      }
    __syncthreads();
    if (tid < D) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < STEP; ++w) a += s_red[w * D + tid];
      p.du_part[(U.row * p.splits + U.split) * D + tid] = a;
    }
  }
}

// ---- key side: dk, dv --------------------------------------------------------------------
template <typename TIn, typename TOut, int D, int PHI>
__global__ __launch_bounds__(bwd_threads<D>()) void keyside_kernel(BwdParams p) {
  constexpr int NT = bwd_threads<D>();
  static_assert(D >= 32, "the backward serves head sizes 32, 64 and 128");
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG, NG = NCT / 2;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s1_hi = smem;                 // F(dS_b)
  uint16_t* s1_lo = s1_hi + FRAG;
  uint16_t* s2_hi = s1_lo + FRAG;         // F(dS_b^T)
  uint16_t* s2_lo = s2_hi + FRAG;
  float* s_dz = reinterpret_cast<float*>(s2_lo + FRAG);   // dz_b [D]
  float* s_du = s_dz + D;                                  // du (MALA) or zeros [D]

  const int tid = threadIdx.x, lane = tid & 63, pr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const Geom& geo = p.g;
  const BwdUnit U = bwd_unit<D>(p, blockIdx.x);

  stage_frag<D, NT>(p.ds_hi + U.row * FRAG, p.ds_lo + U.row * FRAG, s1_hi, s1_lo, tid);
  if (tid < D) {
    s_dz[tid] = p.dz[U.row * D + tid];
    s_du[tid] = p.du ? p.du[(int64_t)U.bh * D + tid] : 0.f;
  }
  __syncthreads();
  transpose_frag<D, NT>(s1_hi, s1_lo, s2_hi, s2_lo, tid);
  __syncthreads();

  const AOffsets ao = a_offsets(lane);
  constexpr uint32_t ES = sizeof(TIn);
  const Rsrc rk = make_rsrc(reinterpret_cast<const TIn*>(p.k) + U.head_off, (uint32_t)geo.N * D * ES);
  const Rsrc rv = make_rsrc(reinterpret_cast<const TIn*>(p.v) + U.head_off, (uint32_t)geo.N * D * ES);

  // two named tile buffers and buffer-resource stores, as in dq_kernel
  struct TileBuf {
    In8<TIn> k[NKC], v[NKC];
    bool valid;
    uint32_t rel;
  };
  auto load_tile = [&](TileBuf& b, int tile) {
    const int32_t j = U.j_begin + tile * 16 + pr;
    b.valid = tile < U.n_tiles && j < U.j_end;
    b.rel = b.valid ? (uint32_t)(U.base_tok + block_offset(geo, U.bg, (uint32_t)j)) * D : 0u;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t off = b.valid ? (b.rel + 32 * kc + 8 * lg) * ES : kOutOfRange;
      b.k[kc].template load_buf<0>(rk, off);
      b.v[kc].template load_buf<0>(rv, off);
    }
  };
  constexpr uint32_t EO = sizeof(TOut);
  const Rsrc rdk = make_rsrc(reinterpret_cast<TOut*>(p.dk) + U.head_off, (uint32_t)geo.N * D * EO);
  const Rsrc rdv = make_rsrc(reinterpret_cast<TOut*>(p.dv) + U.head_off, (uint32_t)geo.N * D * EO);

  auto process = [&](const TileBuf& cur, TileBuf& next, int next_tile) {
    f32x4_t acc1[NCT], acc2[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      acc1[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc2[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      // dv = dS_b^T phi(k): contraction over key features
      float ph[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ph[e] = phi_map<PHI>(cur.k[kc].get(e));
      u32x4_t bh, bl;
      split8(ph, bh, bl);
      frag_mfma<D, true>(acc1, s1_hi, s1_lo, ao, kc, bh, bl);
      // dk~ = dS_b v: contraction over value channels (bf16 V is exact in one operand)
      if constexpr (sizeof(TIn) == 2) {
        frag_mfma<D, false>(acc2, s2_hi, s2_lo, ao, kc, cur.v[kc].w, cur.v[kc].w);
      } else {
        float vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = cur.v[kc].get(e);
        u32x4_t vh, vl;
        split8(vv, vh, vl);
        frag_mfma<D, true>(acc2, s2_hi, s2_lo, ao, kc, vh, vl);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    load_tile(next, next_tile);

#pragma unroll
    for (int c = 0; c < NG; ++c) {
      const int f0 = 32 * c + 8 * lg;
      float dvo[8], dko[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        dvo[r] = acc_out<NCT>(acc1, c, r) + s_du[f0 + r];
        dko[r] = (acc_out<NCT>(acc2, c, r) + s_dz[f0 + r]) * dphi_map<PHI>(cur.k[c].get(r));
      }
      const uint32_t off = cur.valid ? (cur.rel + f0) * EO : kOutOfRange;
      buf_store8<TOut>(rdv, off, dvo);
      buf_store8<TOut>(rdk, off, dko);
    }
  };

  constexpr int STEP = NT / 64;
  TileBuf bufA, bufB;
  load_tile(bufA, wave);
  for (int tile = wave; tile < U.n_tiles; tile += 2 * STEP) {
    process(bufA, bufB, tile + STEP);
    if (tile + STEP >= U.n_tiles) break;
    process(bufB, bufA, tile + 2 * STEP);
  }
}

// ---- dM_c ---------------------------------------------------------------------------------
// dmc[i][b] = sum over (batch-head, position) of dS~_i and S_b (fragment positions, then the D
// normaliser entries), both summed over their token slices while loaded.  A TILE x TILE output
// tile and one chunk of 64-position steps per workgroup; each step is staged through LDS as bf16
// hi / lo, and each wave owns 32 rows x (TILE / 2) columns (2 x TILE / 32 MFMA tiles): A = dS~
// rows, B = S rows, both with 8 consecutive positions per lane.  The next step's loads are in
// flight during the MFMAs.  Positions past FRAG + D (the last step of a (batch, head)) read as
// zero.  Every row is staged once per output tile of its chunk: 128 x 128 tiles (8 waves) once
// M > 64 load and convert each row half as often as 64 x 64 tiles (4 waves).  The kernel is
// bound by its loads (a step's 256-byte row pieces, 64 KB apart in the stack): each load
// instruction covers whole 128-byte lines, and one round of workgroups (one chunk each) keeps
// two steps per CU in flight without a second round's ramp.
constexpr int kDmcK = 64, kDmcPitch = kDmcK + 8;   // positions per step; LDS pitch in bf16 elements

// SINGLE: every summary has one token slice (ssplits = zsplits_d = 1).  The step's loads then
// go straight into registers through buffer resources (rows past M and positions past FRAG + D
// read as zero) and are converted at the LDS store, so they stay in flight during the MFMAs;
// with several slices they are summed as they arrive.
template <bool SINGLE, int TILE>
__global__ __launch_bounds__(TILE * 4) void dmc_kernel(DmcParams p) {
  constexpr int kDmcTile = TILE, WB = TILE / 32;   // WB: MFMA column tiles per wave
  __shared__ __align__(16) uint16_t a_hi[kDmcTile * kDmcPitch], a_lo[kDmcTile * kDmcPitch];
  __shared__ __align__(16) uint16_t b_hi[kDmcTile * kDmcPitch], b_lo[kDmcTile * kDmcPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int M = p.M, FRAG = p.frag, D = p.D;
  const int nt = (M + kDmcTile - 1) / kDmcTile;
  // Workgroup L -> (chunk, output tile): the nt^2 tiles of one chunk read the same rows, so
  // they share an XCD (workgroups are dealt to the 8 XCDs round robin): L = 8 * (c8 * nt^2 +
  // tile) + x with chunk = 8 * c8 + x.  Slots of chunks >= nchunks have nothing to do.
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int tile = slot % (nt * nt), chunk = 8 * (slot / (nt * nt)) + xcd;
  if (chunk >= p.nchunks) return;
  const int i0 = (tile / nt) * kDmcTile, b0 = (tile % nt) * kDmcTile;
  const int grp = blockIdx.y;
  // loader: eight threads per row, 16 bytes each, so that each load instruction of a wave covers
  // eight whole 128-byte lines; thread t holds positions 4 (t % 8) + 32 hf + 0..3 (hf = 0, 1) of
  // the tile's rows t / 8 and t / 8 + TILE / 2
  constexpr int kRowsPass = TILE / 2;
  const int lrow = tid >> 3, lq = (tid & 7) * 4;
  const int wi = (wave >> 1) * 32, wb = (wave & 1) * (TILE / 2);
  const int64_t total_steps = (int64_t)p.group_bh * p.steps_per_bh;
  const int64_t s_begin = (int64_t)chunk * p.steps_per_chunk;
  const int64_t s_end = min(s_begin + p.steps_per_chunk, total_steps);

  // sum over token slices of 4 consecutive values at position pos of summary row (bh, m)
  auto load4 = [&](const float* part, const float* zpart, int zsplits, int bh, int m, int pos, float (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = 0.f;
    if (m >= M || pos >= FRAG + D) return;
    const int64_t r = (int64_t)bh * M + m;
    const bool in_s = pos < FRAG;
    const int ns = in_s ? p.ssplits : zsplits;
    for (int s = 0; s < ns; ++s) {
      const float* src = in_s ? part + (r * p.ssplits + s) * FRAG + pos : zpart + (r * zsplits + s) * D + (pos - FRAG);
      const u32x4_t w = ld16(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += __uint_as_float(w[e]);
    }
  };
  auto load_step = [&](int64_t step, float (&xa)[2][2][4], float (&xb)[2][2][4]) {
    const int j = (int)(step / p.steps_per_bh);
    const int pos0 = (int)(step % p.steps_per_bh) * kDmcK;
    const int bh = p.per_head ? j * p.H + grp : j;
#pragma unroll
    for (int hr = 0; hr < 2; ++hr)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int pos = pos0 + 32 * hf + lq, r = lrow + kRowsPass * hr;
        load4(p.dps, p.dpz, p.zsplits_d, bh, i0 + r, pos, xa[hr][hf]);
        load4(p.ps, p.pz, p.ssplits, bh, b0 + r, pos, xb[hr][hf]);
      }
  };

  // SINGLE: raw words of the step, [hr][hf] as held by the loader
  u32x4_t ra[2][2], rb[2][2];
  auto issue_step = [&](int64_t step) {
    const int j = (int)(step / p.steps_per_bh);
    const int pos0 = (int)(step % p.steps_per_bh) * kDmcK;   // the step is all S or all z
    const int bh = p.per_head ? j * p.H + grp : j;
    const bool in_s = pos0 < FRAG;
    const Rsrc rsa = in_s ? make_rsrc(p.dps + (int64_t)bh * M * FRAG, (uint32_t)M * FRAG * 4u)
                          : make_rsrc(p.dpz + (int64_t)bh * M * D, (uint32_t)M * D * 4u);
    const Rsrc rsb = in_s ? make_rsrc(p.ps + (int64_t)bh * M * FRAG, (uint32_t)M * FRAG * 4u)
                          : make_rsrc(p.pz + (int64_t)bh * M * D, (uint32_t)M * D * 4u);
    const int stride = in_s ? FRAG : D, base = in_s ? 0 : FRAG;
#pragma unroll
    for (int hr = 0; hr < 2; ++hr)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int pos = pos0 + 32 * hf + lq;
        const bool okp = pos < FRAG + D;
        const int ma = i0 + lrow + kRowsPass * hr, mb = b0 + lrow + kRowsPass * hr;
        const uint32_t oa = (okp && ma < M) ? (uint32_t)(ma * stride + pos - base) * 4u : kOutOfRange;
        const uint32_t ob = (okp && mb < M) ? (uint32_t)(mb * stride + pos - base) * 4u : kOutOfRange;
        ra[hr][hf] = buf_ld16(rsa, oa);
        rb[hr][hf] = buf_ld16(rsb, ob);
      }
  };
  auto words = [](const u32x4_t& w, float (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  };
  auto split4 = [](const float (&x)[4], u32x2_t& hi, u32x2_t& lo) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t h, l;
      split_bf16x2(x[2 * i], x[2 * i + 1], h, l);
      hi[i] = h;
      lo[i] = l;
    }
  };

  f32x4_t acc[2][WB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < WB; ++c) acc[a][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  float xa[2][2][4], xb[2][2][4];
  if (s_begin < s_end) {
    if constexpr (SINGLE) issue_step(s_begin);
    else load_step(s_begin, xa, xb);
  }
  for (int64_t step = s_begin; step < s_end; ++step) {
#pragma unroll
    for (int hr = 0; hr < 2; ++hr)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (SINGLE) {
          words(ra[hr][hf], xa[hr][hf]);
          words(rb[hr][hf], xb[hr][hf]);
        }
        u32x2_t ah, al, bhh, bll;
        split4(xa[hr][hf], ah, al);
        split4(xb[hr][hf], bhh, bll);
        const int o = (lrow + kRowsPass * hr) * kDmcPitch + 32 * hf + lq;
        *reinterpret_cast<u32x2_t*>(a_hi + o) = ah;
        *reinterpret_cast<u32x2_t*>(a_lo + o) = al;
        *reinterpret_cast<u32x2_t*>(b_hi + o) = bhh;
        *reinterpret_cast<u32x2_t*>(b_lo + o) = bll;
      }
    // the step's words are in LDS: the next step's loads go out before the barrier (SINGLE),
    // so that they are in flight while the slower waves finish converting
    if constexpr (SINGLE) {
      if (step + 1 < s_end) issue_step(step + 1);
    }
    __syncthreads();
    if constexpr (!SINGLE) {
      if (step + 1 < s_end) load_step(step + 1, xa, xb);
    }
#pragma unroll
    for (int k2 = 0; k2 < kDmcK; k2 += 32) {
      const int kk = k2 + 8 * (lane >> 4);
      u32x4_t fah[2], fal[2], fbh[WB], fbl[WB];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int ra = (wi + 16 * a + (lane & 15)) * kDmcPitch + kk;
        fah[a] = *reinterpret_cast<const u32x4_t*>(a_hi + ra);
        fal[a] = *reinterpret_cast<const u32x4_t*>(a_lo + ra);
      }
#pragma unroll
      for (int c = 0; c < WB; ++c) {
        const int rb = (wb + 16 * c + (lane & 15)) * kDmcPitch + kk;
        fbh[c] = *reinterpret_cast<const u32x4_t*>(b_hi + rb);
        fbl[c] = *reinterpret_cast<const u32x4_t*>(b_lo + rb);
      }
      // three rounds over the independent accumulators
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < WB; ++c) acc[a][c] = mfma_bf16(fah[a], fbh[c], acc[a][c]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < WB; ++c) acc[a][c] = mfma_bf16(fal[a], fbh[c], acc[a][c]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < WB; ++c) acc[a][c] = mfma_bf16(fah[a], fbl[c], acc[a][c]);
    }
    __syncthreads();
  }
  float* out = p.out + ((int64_t)grp * p.nchunks + chunk) * M * M;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < WB; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + wi + 16 * a + 4 * (lane >> 4) + r;
        const int b = b0 + wb + 16 * c + (lane & 15);
        if (i < M && b < M) out[(int64_t)i * M + b] = acc[a][c][r];
      }
}

// dM_c from the chunk partials part[g][c][e].  Many outputs: a workgroup of 8 waves takes 64
// consecutive outputs, wave j sums the chunks c = j, j + 8, ... in order (its lanes over the
// outputs, so each load is coalesced) and the eight sums are added in the order j = 0 .. 7.
// Few outputs: one wave each, lanes striding over the chunks and a fixed shuffle tree.  Both
// orders are fixed for a given shape.
constexpr int kDmcRedWaves = 8;
__global__ __launch_bounds__(64 * kDmcRedWaves) void dmc_reduce_kernel(const float* part, float* dmc, int64_t mm,
                                                                       int groups, int nchunks, int wave_per_output) {
  const int64_t n_out = (int64_t)groups * mm;
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  if (!wave_per_output) {
    __shared__ float sums[kDmcRedWaves][64];
    const int64_t idx = (int64_t)blockIdx.x * 64 + lane;
    float a = 0.f;
    if (idx < n_out) {
      const int64_t g = idx / mm, e = idx % mm;
      const float* src = part + g * nchunks * mm + e;
#pragma unroll 4
      for (int c = j; c < nchunks; c += kDmcRedWaves) a += src[(int64_t)c * mm];   // loads ahead, adds in order
    }
    sums[j][lane] = a;
    __syncthreads();
    if (j == 0 && idx < n_out) {
      float t = sums[0][lane];
#pragma unroll
      for (int k = 1; k < kDmcRedWaves; ++k) t += sums[k][lane];
      dmc[idx] = t;
    }
  } else {
    const int64_t idx = (int64_t)blockIdx.x * kDmcRedWaves + j;
    if (idx >= n_out) return;                      // whole waves leave together
    const int64_t g = idx / mm, e = idx % mm;
    const float* src = part + g * nchunks * mm + e;
    float s = 0.f;
    for (int c = lane; c < nchunks; c += 64) s += src[(int64_t)c * mm];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) dmc[idx] = s;
  }
}

// ---- MALA: sums of the token-slice partials ------------------------------------------------
// One workgroup per (batch, head).  Fragment position pos holds T[k][c] for key feature
// k = 32 kc + 8 (l / 16) + pos % 8 and channel c = 16 ct + l % 16, where l = (pos / 8) % 64 and
// (kc, ct) = (pos / 512) / NCT, (pos / 512) % NCT: 8 consecutive positions are 8 features of
// one channel.  Stage 1 keeps dS in LDS (fp32, fragment order) for dz -= dS u / N.
template <int D>
__global__ __launch_bounds__(kThreads) void mala_stage_kernel(MalaStageParams p) {
  using Dm = Dims<D>;
  constexpr int FRAG = Dm::FRAG, NCT = Dm::NCT;
  extern __shared__ __align__(16) float fsm[];
  float* s_x = fsm;             // dS [FRAG] (stage 1)
  float* s_z = s_x + FRAG;      // [D]
  float* s_u = s_z + D;         // u / N [D]
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int ss = p.ss;
  const float inv_n = 1.0f / (float)p.N;
  if (tid < D) {
    float z = 0.f, u = 0.f;
    for (int s = 0; s < ss; ++s) z += p.pz[(bh * ss + s) * D + tid];
    if (p.stage == 0) {
      for (int s = 0; s < ss; ++s) u += p.pu[(bh * ss + s) * D + tid];
      u *= inv_n;
    } else {
      u = p.ub[bh * D + tid];
      float du = 0.f;
      for (int r = 0; r < p.rs; ++r) du += p.du_part[(bh * p.rs + r) * D + tid];
      p.du[bh * D + tid] = -du * inv_n;
    }
    s_z[tid] = z;
    s_u[tid] = u;
  }
  __syncthreads();
  for (int pos = tid * 8; pos < FRAG; pos += kThreads * 8) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* src = p.ps + bh * ss * FRAG + pos;
    for (int s = 0; s < ss; ++s) {
      const u32x4_t w0 = ld16(src + (int64_t)s * FRAG), w1 = ld16(src + (int64_t)s * FRAG + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] += __uint_as_float(w0[e]);
        a[4 + e] += __uint_as_float(w1[e]);
      }
    }
    if (p.stage == 0) {   // centring: C[k][c] = S[k][c] - z[k] u[c] / N
      const int l = (pos >> 3) & 63, fr = pos >> 9;
      const int k0 = 32 * (fr / NCT) + 8 * (l >> 4), c = 16 * (fr % NCT) + (l & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = fmaf(-s_z[k0 + e], s_u[c], a[e]);
    } else {
      st16(s_x + pos, u32x4_t{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                              __float_as_uint(a[3])});
      st16(s_x + pos + 4, u32x4_t{__float_as_uint(a[4]), __float_as_uint(a[5]), __float_as_uint(a[6]),
                                  __float_as_uint(a[7])});
    }
    u32x4_t hi, lo;
    split8(a, hi, lo);
    st16(p.y_hi + bh * FRAG + pos, hi);
    st16(p.y_lo + bh * FRAG + pos, lo);
  }
  if (p.stage == 0) {
    if (tid < D) {
      p.zo[bh * D + tid] = s_z[tid];
      p.ub_out[bh * D + tid] = s_u[tid];
    }
    return;
  }
  __syncthreads();
  if (tid < D) {   // (dS u / N)[k] over the channels c, in channel order
    const int k = tid, kc = k >> 5, e = k & 7, lgk = (k & 31) >> 3;
    float a = 0.f;
    for (int c = 0; c < D; ++c) {
      const int pos = ((kc * NCT + (c >> 4)) * 64 + 16 * lgk + (c & 15)) * 8 + e;
      a = fmaf(s_x[pos], s_u[c], a);
    }
    p.zo[bh * D + k] = s_z[k] - a;
  }
}

// ---- launches -----------------------------------------------------------------------------
template <int D>
static size_t dq_lds() {
  using Dm = Dims<D>;
  return (size_t)4 * Dm::FRAG * 2 + (size_t)Dm::NKC * 512 * 2 + (size_t)D * 4;
}
template <int D>
static size_t keyside_lds() {
  return (size_t)4 * Dims<D>::FRAG * 2 + (size_t)2 * D * 4;
}

template <int PHI, typename TIn, typename TOut, int D>
static hipError_t launch_bwd_t(const BwdParams& p, int mode, int n_units, bool key_side, hipStream_t s) {
  if (key_side) {
    auto kern = keyside_kernel<TIn, TOut, D, PHI>;
    const size_t lds = keyside_lds<D>();
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_units), dim3(bwd_threads<D>()), lds, s, p);
  } else {
    auto kern = mode == kBwdMala ? dq_kernel<TIn, TOut, D, PHI, true> : dq_kernel<TIn, TOut, D, PHI, false>;
    const size_t lds = dq_lds<D>();
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_units), dim3(bwd_threads<D>()), lds, s, p, mode);
  }
  return hipGetLastError();
}

template <int PHI, typename TIn, typename TOut>
static hipError_t bwd_dispatch_d(const BwdParams& p, int d, int mode, int n, bool ks, hipStream_t s) {
  switch (d) {
    case 32: return launch_bwd_t<PHI, TIn, TOut, 32>(p, mode, n, ks, s);
    case 64: return launch_bwd_t<PHI, TIn, TOut, 64>(p, mode, n, ks, s);
    case 128: return launch_bwd_t<PHI, TIn, TOut, 128>(p, mode, n, ks, s);
    default: return hipErrorInvalidValue;
  }
}

// n_units = splits * M * BH; key_side selects keyside_kernel (dk, dv), else dq_kernel.
hipError_t launch_bwd_tiles(const BwdParams& p, int d, bool in_fp32, bool out_fp32, int mode, int phi,
                            bool key_side, int n_units, hipStream_t stream) {
  auto go = [&](auto phi_c) {
    constexpr int PHI = decltype(phi_c)::value;
    if (in_fp32)
      return out_fp32 ? bwd_dispatch_d<PHI, float, float>(p, d, mode, n_units, key_side, stream)
                      : bwd_dispatch_d<PHI, float, uint16_t>(p, d, mode, n_units, key_side, stream);
    return out_fp32 ? bwd_dispatch_d<PHI, uint16_t, float>(p, d, mode, n_units, key_side, stream)
                    : bwd_dispatch_d<PHI, uint16_t, uint16_t>(p, d, mode, n_units, key_side, stream);
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

// One workgroup per (batch, head); head sizes 32, 64, 128.
hipError_t launch_mala_stage(const MalaStageParams& p, int d, int bh, hipStream_t stream) {
  auto go = [&](auto dc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    const size_t lds = ((size_t)Dims<D>::FRAG + 2 * D) * 4;
    hipError_t e = hipFuncSetAttribute((const void*)mala_stage_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mala_stage_kernel<D>, dim3(bh), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
  };
  switch (d) {
    case 32: return go(std::integral_constant<int, 32>{});
    case 64: return go(std::integral_constant<int, 64>{});
    case 128: return go(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dmc(const DmcParams& p, float* dmc, hipStream_t stream) {
  const int tile = dmc_tile(p.M);
  const int t = (p.M + tile - 1) / tile;
  const int groups = p.per_head ? p.H : 1;
  const int c8 = (p.nchunks + 7) / 8;
  const bool single = p.ssplits == 1 && p.zsplits_d == 1;
  const dim3 grid(8 * c8 * t * t, groups);
  if (tile == 128) {
    if (single) hipLaunchKernelGGL((dmc_kernel<true, 128>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((dmc_kernel<false, 128>), grid, dim3(512), 0, stream, p);
  } else {
    if (single) hipLaunchKernelGGL((dmc_kernel<true, 64>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((dmc_kernel<false, 64>), grid, dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mm = (int64_t)p.M * p.M, n_out = (int64_t)groups * mm;
  const int wave_per_output = n_out < 16384 ? 1 : 0;
  const int64_t per_wg = wave_per_output ? kDmcRedWaves : 64;   // outputs per workgroup
  hipLaunchKernelGGL(dmc_reduce_kernel, dim3((unsigned)((n_out + per_wg - 1) / per_wg)), dim3(64 * kDmcRedWaves), 0,
                     stream, p.out, dmc, mm, groups, p.nchunks, wave_per_output);
  return hipGetLastError();
}

}  // namespace mhla
