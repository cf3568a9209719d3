// Chunkwise-causal MHLA readout over a 1D token sequence.
//
// "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method -> Key
// design 2 (the token-expanded identity q~^T S~_i = sum_t m_{i,b(t)} (q~^T K~_t) V_t^T) and Key
// design 4 (compatible with chunkwise-parallel training and streaming inference).  The pages
// give no causal form; the reading here masks the token-expanded sum at the token level: query
// t sees keys t' <= t with weight m_{b(t),b(t')} (q~_t . k~_t').  For query t of block i:
//   num_t = q~_t^T (S~<_i + m_ii (P_s + R_t)),   den_t = q~_t^T (z~<_i + m_ii (p_s + r_t))
// with S~<_i = sum_{b<i} m_ib S_b (the mixing kernel with the strictly lower part of M_c),
// P_s the summed partial summaries of the block's earlier token slices (an exclusive prefix
// over slices), and R_t = sum of k~_j v_j^T over the slice's tokens j <= t.
//
// One workgroup (4 wave64s, 8 at d = 128) per unit = (batch-head, block, token slice).  The unit's running
// state (S~<_i + m_ii P_s, then + m_ii * each finished sub-chunk) lives in LDS as bf16 hi / lo
// fragments -- the MFMA A operands of the readout, as in the readout kernel -- and in fp32
// accumulators spread over the waves.  The slice is walked in sub-chunks of SUB tokens:
//   1. stage the sub-chunk's phi(K) (row-major, and transposed scaled by m_ii) and V^T in LDS;
//   2. every wave reads out its query tile (channels split between WQ waves): O^T = state^T q~
//      on 16x16x32 MFMAs, plus the in-sub-chunk causal term: scores D[j][t] = phi(k_j).q~_t on
//      16x16x32 MFMAs (keys as A rows), masked to j <= t and scaled by m_ii, which in the
//      16x16x16 MFMA's layout are directly the B operand of V^T P (rows of the 16x16x32
//      result = k of the 16x16x16 operand); the score sums give the in-chunk normaliser;
//   3. the state absorbs the sub-chunk: acc += (m_ii phi(K))^T V on MFMA (permuted A rows so
//      each lane owns 8 consecutive fragment elements), rewritten as hi / lo fragments.
// The readout and update of the state use hi / lo bf16 operand splits (bf16 V is exact).  With
// bf16 inputs the in-sub-chunk scores and V^T P do too; with fp32 inputs they run on fp32 MFMAs
// (16x16x4) over fp32 phi(K) and V tiles, since an output with few keys in view averages no
// rounding error away.
#include <type_traits>

#include "frag_lds.hpp"

namespace mhla {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x16_bf16: A lane l = row l%16, k = 4(l/16) + 0..3; B lane l = k 4(l/16) + 0..3,
// column l%16; D lane l = rows 4(l/16) + 0..3, column l%16 (checked on the MI355X with an
// in-bounds probe against an integer matrix product).
__device__ inline f32x4_t mfma16_bf16(const u32x2_t& a, const u32x2_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                   c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: A lane l = row l%16, k = l/16; B lane l = k l/16, column l%16; D as
// above.
__device__ inline f32x4_t mfma4_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// VSPLIT: fp32 inputs (fp32 phi(K) and V^T tiles in LDS, in the space of the hi / lo planes).  At d = 128 a 64-token sub-chunk fits the LDS with
// bf16 V (156 KB) and halves the sub-chunk steps (and their barriers); fp32 V takes 32.
template <int D, bool VSPLIT>
struct CausalShape {
  static constexpr int NW = D >= 128 ? 8 : 4;      // waves per workgroup
  static constexpr int NT = 64 * NW;               // threads per workgroup
  static constexpr int SUB = D >= 128 && VSPLIT ? 32 : 64;   // tokens per sub-chunk
  static constexpr int QT = SUB / 16;              // query tiles per sub-chunk
  static constexpr int WQ = NW / QT;               // waves per query tile (channel pairs split)
  static constexpr int KP = D + 8;                 // LDS pitch of row-major phi(K) (elements)
  static constexpr int TP = SUB + 8;               // LDS pitch of the transposed tiles
};

template <int D, bool VSPLIT>
constexpr size_t causal_lds_bytes() {
  using CS = CausalShape<D, VSPLIT>;
  return (size_t)2 * (2 * Dims<D>::FRAG + Dims<D>::NKC * 512 + 2 * CS::SUB * CS::KP + 2 * D * CS::TP +
                      (VSPLIT ? 2 : 1) * D * CS::TP);
}

template <typename TOut>
__device__ inline void store8_out(TOut* dst, const float (&x)[8]) {
  if constexpr (sizeof(TOut) == 4) {
    st16(dst, u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
    st16(dst + 4, u32x4_t{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
  } else {
    st16(dst, u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7])});
  }
}

template <typename TIn, typename TOut, int D, int PHI>
__global__ __launch_bounds__((CausalShape<D, sizeof(TIn) == 4>::NT)) void causal_kernel(CausalParams p) {
  static_assert(D >= 32, "the causal readout serves head sizes 32, 64 and 128");
  using Dm = Dims<D>;
  using CS = CausalShape<D, sizeof(TIn) == 4>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int SUB = CS::SUB, QT = CS::QT, WQ = CS::WQ, KP = CS::KP, TP = CS::TP, NW = CS::NW;
  constexpr bool VSPLIT = sizeof(TIn) == 4;     // fp32 V needs hi / lo; bf16 V is exact
  constexpr int NFR = NKC * NCT;                 // state fragments
  // State fragments by wave: WPK waves share a 32-feature chunk kc = wave / WPK, each owning
  // FPW consecutive channel tiles, so a wave reads its phi(K)^T rows once for all of them.
  constexpr int WPK = NW / NKC;                  // waves per feature chunk
  constexpr int FPW = NCT / WPK > 0 ? NCT / WPK : 1;   // fragments (channel tiles) per wave
  constexpr int PPW = NCT / 2 / WQ;              // channel pairs per wave in the readout
  constexpr uint32_t ES = sizeof(TIn);

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* s_hi = smem;                        // state fragments (hi, lo)
  uint16_t* s_lo = s_hi + FRAG;
  uint16_t* s_z = s_lo + FRAG;                  // normaliser fragments
  uint16_t* kr_hi = s_z + NKC * 512;            // phi(K) row-major [SUB][KP]
  uint16_t* kr_lo = kr_hi + SUB * KP;
  uint16_t* kt_hi = kr_lo + SUB * KP;           // m_ii phi(K)^T [D][TP]
  uint16_t* kt_lo = kt_hi + D * TP;
  uint16_t* vt_hi = kt_lo + D * TP;             // V^T [D][TP]
  uint16_t* vt_lo = vt_hi + D * TP;             // (fp32 V only)
  // fp32 inputs: phi(K) row-major [SUB][KP] and V^T [D][TP] as fp32, over the hi / lo planes
  float* kr32 = reinterpret_cast<float*>(kr_hi);
  float* vt32 = reinterpret_cast<float*>(vt_hi);

  // the wave index in a scalar register: the per-wave roles below are uniform branches
  const int tid = threadIdx.x, lane = tid & 63, pr = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Geom& geo = p.g;

  // unit L -> (head, block, token slice); all units of a head on one XCD when BH % 8 == 0
  const int L = blockIdx.x;
  const int per_head = p.splits * geo.M;
  int bh, r;
  if (p.xcd_map) {
    const int xcd = L & 7, sl = L >> 3;
    bh = (sl / per_head) * 8 + xcd;
    r = sl % per_head;
  } else {
    bh = L / per_head;
    r = L % per_head;
  }
  const int blk = r / p.splits, split = r % p.splits;
  const int32_t j_begin = split * p.tok_per_split;
  const BlockGeo bgeo = block_geo(geo, blk);
  const int32_t j_end = min(j_begin + p.tok_per_split, bgeo.n);
  const int32_t base_tok = bgeo.base;
  const int64_t head_off = (int64_t)bh * geo.N * D;
  const int64_t row = (int64_t)bh * geo.M + blk;
  const float mii = p.mc ? p.mc[(int64_t)(bh % p.H) * p.mc_head_stride + (int64_t)blk * geo.M + blk] : 1.0f;

  // ---- state: S~<_i (+ m_ii * earlier slices), fp32 in the owning waves, hi / lo in LDS ----
  const int my_kc = wave / WPK, my_ct0 = (wave % WPK) * FPW;
  const bool updater = my_ct0 < NCT;             // d = 32: two of the four waves
  f32x4_t sacc[FPW][2];
#pragma unroll
  for (int a = 0; a < FPW; ++a) {
    const int fr = my_kc * NCT + my_ct0 + a;
    sacc[a][0] = sacc[a][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!updater) continue;
    const int pos = (fr * 64 + lane) * 8;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (p.st_hi) {
      const u32x4_t h = ld16(p.st_hi + row * FRAG + pos);
      const u32x4_t l = p.st_lo ? ld16(p.st_lo + row * FRAG + pos) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hw = h[e >> 1], lw = l[e >> 1];
        x[e] = ((e & 1) ? bf16hi_to_f32(hw) : bf16lo_to_f32(hw)) + ((e & 1) ? bf16hi_to_f32(lw) : bf16lo_to_f32(lw));
      }
    }
    if (p.pre) {
      const float* pp = p.pre + (row * p.splits + split) * FRAG + pos;
      const u32x4_t w0 = ld16(pp), w1 = ld16(pp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = fmaf(mii, __uint_as_float(w0[e]), x[e]);
        x[4 + e] = fmaf(mii, __uint_as_float(w1[e]), x[4 + e]);
      }
    }
    sacc[a][0] = f32x4_t{x[0], x[1], x[2], x[3]};
    sacc[a][1] = f32x4_t{x[4], x[5], x[6], x[7]};
    store_frag8<true>(s_hi, s_lo, lds_pos<NCT>(pos), x);
  }
  // Normaliser state: wave kc (< NKC) holds z[32kc + 8lg + e] in zacc[e / 4][e % 4] on every lane
  // (the layout of a 16x16x32 result against an all-ones B operand), and writes the normaliser
  // fragment: lane (row 4g + 0) = hi(z), (row 4g + 1) = lo(z), other rows zero.
  const bool zwave = wave % WPK == 0;            // one wave per feature chunk keeps z
  f32x4_t zacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  auto write_zfrag = [&]() {
    float z8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z8[e] = zacc[e >> 2][e & 3];
    u32x4_t w = {0u, 0u, 0u, 0u};
    if ((pr & 3) < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        split_bf16x2(z8[2 * i], z8[2 * i + 1], h, l);
        w[i] = (pr & 3) == 0 ? h : l;
      }
    }
    st16(s_z + (my_kc * 64 + lane) * 8, w);
  };
  if (zwave) {
    const int f0 = 32 * my_kc + 8 * lg;
    float z8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float zz = p.zt ? p.zt[row * D + f0 + e] : 0.f;
      if (p.prez) zz = fmaf(mii, p.prez[(row * p.splits + split) * D + f0 + e], zz);
      z8[e] = zz;
    }
    zacc[0] = f32x4_t{z8[0], z8[1], z8[2], z8[3]};
    zacc[1] = f32x4_t{z8[4], z8[5], z8[6], z8[7]};
    write_zfrag();
  }

  const AOffsets ao = a_offsets(lane);
  // query tile and channel pairs of this wave.  Waves w and w + 4 share a SIMD, so waves 4 .. 7
  // take the query tiles in reverse order: every SIMD then walks the same number of in-sub-chunk
  // key tiles (query tile qt reads qt + 1 of them).
  const int qt = ((wave >> 2) & 1) ? QT - 1 - wave % QT : wave % QT, cp = wave / QT;
  const Rsrc rq = make_rsrc(reinterpret_cast<const TIn*>(p.q) + head_off, (uint32_t)geo.N * D * ES);
  const Rsrc rk = make_rsrc(reinterpret_cast<const TIn*>(p.k) + head_off, (uint32_t)geo.N * D * ES);
  const Rsrc rv = make_rsrc(reinterpret_cast<const TIn*>(p.v) + head_off, (uint32_t)geo.N * D * ES);

  // Staging role: 2 consecutive tokens x 8 features (lanes run over the token pairs, so the
  // transposed 4-byte LDS writes of a wave fill consecutive words of one row).
  constexpr int FG = D / 8, NPAIR = SUB / 2;
  const int tp = tid % NPAIR, fg = tid / NPAIR;
  const bool stager = fg < FG;
  In8<TIn> ck[2], cv[2];     // the sub-chunk's K and V rows of this thread (prefetched)
  In8<TIn> cq[NKC];          // the wave's query features (prefetched)
  auto issue_kv = [&](int32_t j0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int32_t j = j0 + 2 * tp + i;
      const bool ok = stager && j < j_end;
      const uint32_t t = ok ? (uint32_t)(base_tok + block_offset(geo, bgeo, (uint32_t)j)) : 0u;
      const uint32_t off = ok ? (t * D + 8 * fg) * ES : kOutOfRange;
      ck[i].template load_buf<0>(rk, off);
      cv[i].template load_buf<0>(rv, off);
    }
  };
  auto issue_q = [&](In8<TIn> (&dst)[NKC], int32_t j0) {
    const int32_t jq = j0 + 16 * qt + pr;
    const bool ok = jq < j_end;
    const uint32_t rel = ok ? (uint32_t)(base_tok + block_offset(geo, bgeo, (uint32_t)jq)) * D : 0u;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) dst[kc].template load_buf<0>(rq, ok ? (rel + 32 * kc + 8 * lg) * ES : kOutOfRange);
  };
  issue_kv(j_begin);
  issue_q(cq, j_begin);
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  for (int32_t j0 = j_begin; j0 < j_end; j0 += SUB) {
    // ---- stage the sub-chunk from the prefetched registers, then prefetch the next one ----
    if (stager) {
      float kf[2][8];                         // [token][feature]; tokens past the end: 0
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = j0 + 2 * tp + i < j_end;
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[i][e] = ok ? phi_map<PHI>(ck[i].get(e)) : 0.f;
        if constexpr (VSPLIT) {
          float* dst = kr32 + (2 * tp + i) * KP + 8 * fg;
          *reinterpret_cast<float4*>(dst) = make_float4(kf[i][0], kf[i][1], kf[i][2], kf[i][3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(kf[i][4], kf[i][5], kf[i][6], kf[i][7]);
        } else {
          store_frag8<true>(kr_hi, kr_lo, (2 * tp + i) * KP + 8 * fg, kf[i]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int at = (8 * fg + e) * TP + 2 * tp;
        uint32_t h, l;
        split_bf16x2(mii * kf[0][e], mii * kf[1][e], h, l);
        *reinterpret_cast<uint32_t*>(kt_hi + at) = h;
        *reinterpret_cast<uint32_t*>(kt_lo + at) = l;
        if constexpr (VSPLIT) {
          *reinterpret_cast<float2*>(vt32 + at) = make_float2(cv[0].get(e), cv[1].get(e));
        } else {
          *reinterpret_cast<uint32_t*>(vt_hi + at) = cv[0].bits(e) | (cv[1].bits(e) << 16);   // exact
        }
      }
    }
    issue_kv(j0 + SUB);                        // past the end: out-of-range loads read zero
    __syncthreads();

    // ---- readout of query tile qt, channel pairs [cp * PPW, (cp + 1) * PPW) ----
    const int32_t jq = j0 + 16 * qt + pr;
    const bool qvalid = jq < j_end;
    const uint32_t qrel = qvalid ? (uint32_t)(base_tok + block_offset(geo, bgeo, (uint32_t)jq)) * D : 0u;
    u32x4_t bq_hi[NKC], bq_lo[NKC];
    float qf[NKC][8];                          // fp32 inputs: phi(q) for the in-sub-chunk scores
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        const float q0 = phi_map<PHI>(cq[kc].get(2 * i)), q1 = phi_map<PHI>(cq[kc].get(2 * i + 1));
        if constexpr (VSPLIT) {
          qf[kc][2 * i] = q0;
          qf[kc][2 * i + 1] = q1;
        }
        split_bf16x2(q0, q1, h, l);
        bq_hi[kc][i] = h;
        bq_lo[kc][i] = l;
      }
    // cq is free now: the next sub-chunk's queries go straight into it (a register copy of
    // loaded values would make the loop wait for every outstanding load and store); with fp32
    // inputs once the scores are done, so that phi(q) takes cq's registers meanwhile
    if constexpr (!VSPLIT) issue_q(cq, j0 + SUB);
    f32x4_t accz = {0.f, 0.f, 0.f, 0.f};
    f32x4_t acc[2 * PPW];
#pragma unroll
    for (int t = 0; t < 2 * PPW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const u32x4_t az = *reinterpret_cast<const u32x4_t*>(s_z + (kc * 64 + lane) * 8);
      accz = mfma_bf16(az, bq_hi[kc], accz);
      accz = mfma_bf16(az, bq_lo[kc], accz);
      u32x4_t ah[2 * PPW], al[2 * PPW];
#pragma unroll
      for (int t = 0; t < 2 * PPW; ++t) {
        const int ct = 2 * cp * PPW + t;
        const int off = (kc * NCT + (ct & ~1)) * 512 + ((ct & 1) ? ao.odd : ao.even);
        ah[t] = *reinterpret_cast<const u32x4_t*>(s_hi + off);
        al[t] = *reinterpret_cast<const u32x4_t*>(s_lo + off);
      }
#pragma unroll
      for (int t = 0; t < 2 * PPW; ++t) acc[t] = mfma_bf16(ah[t], bq_hi[kc], acc[t]);
#pragma unroll
      for (int t = 0; t < 2 * PPW; ++t) acc[t] = mfma_bf16(al[t], bq_hi[kc], acc[t]);
#pragma unroll
      for (int t = 0; t < 2 * PPW; ++t) acc[t] = mfma_bf16(ah[t], bq_lo[kc], acc[t]);
    }
    // in-sub-chunk causal term over key tiles 0 .. qt
    float dsum = 0.f;
    for (int kt = 0; kt <= qt; ++kt) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int off = (16 * kt + pr) * KP + 32 * kc + 8 * lg;
        if constexpr (VSPLIT) {
          // k index lg of step e = feature 32 kc + 8 lg + e, on both operands
          const float4 k0 = *reinterpret_cast<const float4*>(kr32 + off);
          const float4 k1 = *reinterpret_cast<const float4*>(kr32 + off + 4);
          sc = mfma4_f32(k0.x, qf[kc][0], sc);
          sc = mfma4_f32(k0.y, qf[kc][1], sc);
          sc = mfma4_f32(k0.z, qf[kc][2], sc);
          sc = mfma4_f32(k0.w, qf[kc][3], sc);
          sc = mfma4_f32(k1.x, qf[kc][4], sc);
          sc = mfma4_f32(k1.y, qf[kc][5], sc);
          sc = mfma4_f32(k1.z, qf[kc][6], sc);
          sc = mfma4_f32(k1.w, qf[kc][7], sc);
        } else {
          const u32x4_t kh = *reinterpret_cast<const u32x4_t*>(kr_hi + off);
          const u32x4_t kl = *reinterpret_cast<const u32x4_t*>(kr_lo + off);
          sc = mfma_bf16(kh, bq_hi[kc], sc);
          sc = mfma_bf16(kl, bq_hi[kc], sc);
          sc = mfma_bf16(kh, bq_lo[kc], sc);
        }
      }
      // lane: keys 16kt + 4lg + r, query 16qt + pr (positions within the sub-chunk)
      float pv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        pv[rr] = (16 * kt + 4 * lg + rr <= 16 * qt + pr) ? mii * sc[rr] : 0.f;
        dsum += pv[rr];
      }
      if constexpr (VSPLIT) {
#pragma unroll
        for (int t = 0; t < 2 * PPW; ++t) {
          const int ct = 2 * cp * PPW + t;
          const int c = 32 * (ct >> 1) + 8 * (pr >> 2) + 4 * (ct & 1) + (pr & 3);
          // step rr: k index lg = key 16 kt + 4 lg + rr, the lane's own score pv[rr]
          const float4 vv = *reinterpret_cast<const float4*>(vt32 + c * TP + 16 * kt + 4 * lg);
          acc[t] = mfma4_f32(vv.x, pv[0], acc[t]);
          acc[t] = mfma4_f32(vv.y, pv[1], acc[t]);
          acc[t] = mfma4_f32(vv.z, pv[2], acc[t]);
          acc[t] = mfma4_f32(vv.w, pv[3], acc[t]);
        }
      } else {
        u32x2_t ph, pl;
        {
          uint32_t h0, l0, h1, l1;
          split_bf16x2(pv[0], pv[1], h0, l0);
          split_bf16x2(pv[2], pv[3], h1, l1);
          ph = u32x2_t{h0, h1};
          pl = u32x2_t{l0, l1};
        }
#pragma unroll
        for (int t = 0; t < 2 * PPW; ++t) {
          const int ct = 2 * cp * PPW + t;
          // A row pr of tile ct is channel 32 (ct / 2) + 8 (pr / 4) + 4 (ct % 2) + pr % 4, so that
          // lane (t, g) ends with channels 8g .. 8g+7 of its pair, as in the state product
          const int c = 32 * (ct >> 1) + 8 * (pr >> 2) + 4 * (ct & 1) + (pr & 3);
          const int off = c * TP + 16 * kt + 4 * lg;
          const u32x2_t vh = *reinterpret_cast<const u32x2_t*>(vt_hi + off);
          acc[t] = mfma16_bf16(vh, ph, acc[t]);
          acc[t] = mfma16_bf16(vh, pl, acc[t]);
        }
      }
    }
    if constexpr (VSPLIT) issue_q(cq, j0 + SUB);
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    if (qvalid) {
      const float den = accz[0] + accz[1] + dsum;
      const float scale = p.normalized ? 1.0f / den : 1.0f;
#pragma unroll
      for (int pp = 0; pp < PPW; ++pp) {
        float o[8];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          o[rr] = acc[2 * pp][rr] * scale;
          o[4 + rr] = acc[2 * pp + 1][rr] * scale;
        }
        const int c0 = 32 * (cp * PPW + pp) + 8 * lg;
        store8_out(reinterpret_cast<TOut*>(p.o) + head_off + qrel + c0, o);
      }
    }
    if (j0 + SUB >= j_end) break;   // the last sub-chunk: no later readout needs the state
    __syncthreads();   // the readout is done with the state fragments and the staged tiles

    // ---- the state absorbs the sub-chunk: sacc += (m_ii phi(K))^T V, z += (m_ii phi(K))^T 1 ----
    if (updater) {
#pragma unroll
      for (int ks = 0; ks < SUB / 32; ++ks) {
        u32x4_t ah[2], al[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int f = 32 * my_kc + 8 * (pr >> 2) + 4 * rt + (pr & 3);
          const int ka = f * TP + 32 * ks + 8 * lg;
          ah[rt] = *reinterpret_cast<const u32x4_t*>(kt_hi + ka);
          al[rt] = *reinterpret_cast<const u32x4_t*>(kt_lo + ka);
        }
#pragma unroll
        for (int a = 0; a < FPW; ++a) {
          const int cb = (16 * (my_ct0 + a) + pr) * TP + 32 * ks + 8 * lg;
          u32x4_t bh, bl;
          if constexpr (VSPLIT) {
            const float4 v0 = *reinterpret_cast<const float4*>(vt32 + cb);
            const float4 v1 = *reinterpret_cast<const float4*>(vt32 + cb + 4);
            uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
            split_bf16x2(v0.x, v0.y, h0, l0);
            split_bf16x2(v0.z, v0.w, h1, l1);
            split_bf16x2(v1.x, v1.y, h2, l2);
            split_bf16x2(v1.z, v1.w, h3, l3);
            bh = u32x4_t{h0, h1, h2, h3};
            bl = u32x4_t{l0, l1, l2, l3};
          } else {
            bh = *reinterpret_cast<const u32x4_t*>(vt_hi + cb);
          }
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) sacc[a][rt] = mfma_bf16(ah[rt], bh, sacc[a][rt]);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) sacc[a][rt] = mfma_bf16(al[rt], bh, sacc[a][rt]);
          if constexpr (VSPLIT) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) sacc[a][rt] = mfma_bf16(ah[rt], bl, sacc[a][rt]);
          }
        }
        if (zwave) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            zacc[rt] = mfma_bf16(ah[rt], ones, zacc[rt]);
            zacc[rt] = mfma_bf16(al[rt], ones, zacc[rt]);
          }
        }
      }
#pragma unroll
      for (int a = 0; a < FPW; ++a) {
        const float x[8] = {sacc[a][0][0], sacc[a][0][1], sacc[a][0][2], sacc[a][0][3],
                            sacc[a][1][0], sacc[a][1][1], sacc[a][1][2], sacc[a][1][3]};
        store_frag8<true>(s_hi, s_lo, lds_pos<NCT>(((my_kc * NCT + my_ct0 + a) * 64 + lane) * 8), x);
      }
      if (zwave) write_zfrag();
    }
    __syncthreads();
  }
}

// Exclusive prefix over the token slices of each block, in place:
// part[row][s] <- sum_{s' < s} part[row][s'] for the FRAG summary positions and the D normaliser
// entries; fixed order.
__global__ __launch_bounds__(kThreads) void slice_prefix_kernel(float* ps, float* pz, int64_t rows, int splits,
                                                                int frag, int d) {
  const int64_t per_row = (int64_t)frag + d;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * per_row) return;
  const int64_t rw = idx / per_row, pos = idx % per_row;
  float run = 0.f;
  for (int s = 0; s < splits; ++s) {
    float* x = pos < frag ? ps + (rw * splits + s) * frag + pos : pz + (rw * splits + s) * d + (pos - frag);
    const float v = *x;
    *x = run;
    run += v;
  }
}

template <int PHI, typename TIn, typename TOut, int D>
static hipError_t launch_causal_t(const CausalParams& p, int n_units, hipStream_t s) {
  auto kern = causal_kernel<TIn, TOut, D, PHI>;
  const size_t lds = causal_lds_bytes<D, sizeof(TIn) == 4>();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_units), dim3(CausalShape<D, sizeof(TIn) == 4>::NT), lds, s, p);
  return hipGetLastError();
}

template <int PHI, typename TIn, typename TOut>
static hipError_t causal_dispatch_d(const CausalParams& p, int d, int n, hipStream_t s) {
  switch (d) {
    case 32: return launch_causal_t<PHI, TIn, TOut, 32>(p, n, s);
    case 64: return launch_causal_t<PHI, TIn, TOut, 64>(p, n, s);
    case 128: return launch_causal_t<PHI, TIn, TOut, 128>(p, n, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_causal_slice(const CausalParams& p, int d, bool out_fp32, int phi, int n_units, hipStream_t stream);

// bf16 inputs: the slice kernel (causal_slice.hip); fp32 inputs: the kernel above.
#ifndef MHLA_CAUSAL_SLICE
#define MHLA_CAUSAL_SLICE 1
#endif

// n_units = splits * M * BH.
hipError_t launch_causal(const CausalParams& p, int d, bool in_fp32, bool out_fp32, int phi, int n_units,
                         hipStream_t stream) {
  if (MHLA_CAUSAL_SLICE && !in_fp32 && p.tok_per_split <= 256)
    return launch_causal_slice(p, d, out_fp32, phi, n_units, stream);
  auto go = [&](auto phi_c) {
    constexpr int PHI = decltype(phi_c)::value;
    if (in_fp32)
      return out_fp32 ? causal_dispatch_d<PHI, float, float>(p, d, n_units, stream)
                      : causal_dispatch_d<PHI, float, uint16_t>(p, d, n_units, stream);
    return out_fp32 ? causal_dispatch_d<PHI, uint16_t, float>(p, d, n_units, stream)
                    : causal_dispatch_d<PHI, uint16_t, uint16_t>(p, d, n_units, stream);
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_slice_prefix(float* ps, float* pz, int64_t rows, int splits, int frag, int d, hipStream_t stream) {
  const int64_t n = rows * ((int64_t)frag + d);
  hipLaunchKernelGGL(slice_prefix_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     ps, pz, rows, splits, frag, d);
  return hipGetLastError();
}

}  // namespace mhla
