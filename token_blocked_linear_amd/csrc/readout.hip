// Readout kernels: for every query token t of block i,
//   normalised    o_t = phi(q_t)^T S~_i / phi(q_t)^T z~_i
//   unnormalised  o_t = phi(q_t)^T S~_i
//   MALA          o_t = u/N + (1 + 1/s_t) phi(q_t)^T C,   s_t = phi(q_t)^T z
// Sources: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Method -> Overall framework (flowchart readout) and Key design 2 (mixing S~_i = sum_b m_ib S_b;
// the normaliser may be dropped); "Rectifying Magnitude Neglect in Linear Attention", Method ->
// Key design (beta, gamma and the linear form, with C = S - z u^T / N so that
// Y = u/N + beta q~^T C exactly).
//
// One workgroup (4 wave64s) serves one unit: a token slice of one query block of one
// (batch, head).  The block's mixed summary sits in LDS in fragment layout (each MFMA A operand
// is one 16-byte LDS read), together with one extra "normaliser" fragment per 32-feature chunk
// whose rows 4g+0 hold hi(z~[k]) and rows 4g+1 hold lo(z~[k]) for every lane group g.  The mixed
// summary either comes from the mixing kernel (all of a thread's loads in flight at once), or --
// for few blocks, and for MALA -- is formed in the prologue:
//   FUSE_BF16      S~_i = sum_b m_ib S_b from the bf16 stack, z~_i likewise, in fp32;
//   FUSE_PARTIALS  from the fp32 token-slice partials: S_b = sum of slices, then the mixing
//                  (MHLA) or the centring C = S - z u^T / N (MALA), split into bf16 hi + lo.
// With all units of a head on one XCD (workgroups are dealt to the 8 XCDs round-robin), a head's
// summaries are fetched from HBM once and then hit in that XCD's L2.
// Per 16-token tile: the lane owning token t = lane%16 and key features 32*kc + 8*(lane/16) + 0..7
// loads them with one 16-byte read (issued a tile ahead), applies phi in fp32, and MFMAs compute
// O^T = S~^T phi(Q)^T, with the normaliser fragment leaving phi(q_t)^T z~ = D[4g] + D[4g+1] in
// every lane of token t with no cross-lane reduction.  Output channels are taken 32 at a time as
// two MFMA tiles h = 0, 1 whose A row m is channel 8*(m/4) + 4h + m%4 of the group, so lane
// (t, g) ends with the 8 consecutive channels 8g .. 8g+7 of token t: 16-byte stores, and the four
// lane groups of a token write 64 (bf16) or 128 (fp32) contiguous bytes.  In LDS, bit 2 of a
// fragment's lane index is flipped when bit 3 is set, so that every 8 lanes of these operand
// reads cover all banks once.
#include <type_traits>

#include "frag_lds.hpp"

namespace mhla {

enum { kModeNormalized = 0, kModeUnnormalized = 1, kModeMala = 2 };
enum { kFuseNone = 0, kFuseBf16 = 1, kFusePartials = 2 };

// NT 16-token tiles at once: phi(Q) -> MFMAs against the staged summary (each A operand read
// from LDS feeds the NT tiles) -> scale -> 16-byte stores.  cur[t] holds this lane's query
// features of tile t; coff[t] the element offset of its token row in Q / O.
template <typename TIn, typename TOut, int D, bool SPLIT, int NT, int PHI>
__device__ __forceinline__ void readout_tiles(const In8<TIn> (&cur)[NT][Dims<D>::NKC],
                                              const bool (&cvalid)[NT], const int64_t (&coff)[NT],
                                              const uint16_t* s_hi, const uint16_t* s_lo,
                                              const uint16_t* s_z, const float* s_ub, AOffsets ao,
                                              int lane, int mode, void* out) {
  using Dm = Dims<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT;
  const int lg = lane >> 4;
  f32x4_t acc[NT][NCT], accz[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    accz[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    // phi on every lane, no branch: tokens past the slice (their loads read zero) give finite
    // values whose output columns are never stored, and key rows k >= D (d = 16) meet zero rows
    // of the summary and normaliser fragments
    u32x4_t b_hi[NT], b_lo[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = phi_map<PHI>(cur[t][kc].get(2 * i)), x1 = phi_map<PHI>(cur[t][kc].get(2 * i + 1));
        if (SPLIT) {
          uint32_t h, l;
          split_bf16x2(x0, x1, h, l);
          b_hi[t][i] = h;
          b_lo[t][i] = l;
        } else {
          b_hi[t][i] = pack_bf16x2(x0, x1);
        }
      }
    const u32x4_t az = *reinterpret_cast<const u32x4_t*>(s_z + (kc * 64 + lane) * 8);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      accz[t] = mfma_bf16(az, b_hi[t], accz[t]);
      if (SPLIT) accz[t] = mfma_bf16(az, b_lo[t], accz[t]);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int off = NCT >= 2 ? (kc * NCT + (ct & ~1)) * 512 + ((ct & 1) ? ao.odd : ao.even)
                               : (kc * 64 + lane) * 8;
      const u32x4_t a_hi = *reinterpret_cast<const u32x4_t*>(s_hi + off);
      u32x4_t a_lo;
      if (SPLIT) a_lo = *reinterpret_cast<const u32x4_t*>(s_lo + off);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][ct] = mfma_bf16(a_hi, b_hi[t], acc[t][ct]);
        if (SPLIT) {
          acc[t][ct] = mfma_bf16(a_lo, b_hi[t], acc[t][ct]);
          acc[t][ct] = mfma_bf16(a_hi, b_lo[t], acc[t][ct]);
        }
      }
    }
    // keep each chunk's LDS operand reads next to their MFMAs: hoisting all of them would
    // cost NKC*NCT*4 registers and halve the waves per SIMD at d = 128
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!cvalid[t]) continue;
    const float den = accz[t][0] + accz[t][1];      // phi(q_t)^T z~  (hi row + lo row)
    float scale = 1.f;
    if (mode == kModeNormalized) scale = 1.0f / den;
    else if (mode == kModeMala) scale = 1.0f + 1.0f / den;
    // lane (t, g) holds channels c0 + 0..7 of each 32-channel group (d = 16: channels 4g..4g+3)
    constexpr int NG = NCT >= 2 ? NCT / 2 : 1;      // channel groups
    constexpr int W = NCT >= 2 ? 8 : 4;             // channels per lane and group
#pragma unroll
    for (int cgp = 0; cgp < NG; ++cgp) {
      const int c0 = NCT >= 2 ? 32 * cgp + 8 * lg : 4 * lg;
      float o[W];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = acc[t][NCT >= 2 ? 2 * cgp : 0][r] * scale;
        if constexpr (W == 8) o[4 + r] = acc[t][2 * cgp + 1][r] * scale;
      }
      if (mode == kModeMala) {
#pragma unroll
        for (int j = 0; j < W; j += 4) {
          const u32x4_t ub = *reinterpret_cast<const u32x4_t*>(s_ub + c0 + j);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[j + r] += __uint_as_float(ub[r]);
        }
      }
      const int64_t dst = coff[t] + c0;
      if constexpr (sizeof(TOut) == 4) {
#pragma unroll
        for (int j = 0; j < W; j += 4)
          st16_pol<MHLA_READOUT_STORE_NT>(
              reinterpret_cast<float*>(out) + dst + j,
              u32x4_t{__float_as_uint(o[j]), __float_as_uint(o[j + 1]), __float_as_uint(o[j + 2]),
                      __float_as_uint(o[j + 3])});
      } else if constexpr (W == 8) {
        st16_pol<MHLA_READOUT_STORE_NT>(
            reinterpret_cast<uint16_t*>(out) + dst,
            u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7])});
      } else {
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(out) + dst) =
            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
  }
}

// A unit's coordinates.  Unit L -> (head, block, token slice); with xcd_map (B*H % 8 == 0), unit
// L belongs to head 8 * ((L/8) / per_head) + L%8, so that the units of a head share an XCD.
struct RdUnit {
  int bh, blk;
  int32_t j_begin, j_end, base_tok;
  int n_tiles;
  int64_t head_off, row;
  BlockGeo bg;
};
template <int D>
__device__ inline RdUnit rd_unit(const ReadoutParams& p, int L) {
  const Geom& g = p.g;
  const int per_head = p.splits * g.M;
  int r;
  RdUnit u;
  if (p.xcd_map) {
    const int xcd = L & 7, s = L >> 3;
    u.bh = (s / per_head) * 8 + xcd;
    r = s % per_head;
  } else {
    u.bh = L / per_head;
    r = L % per_head;
  }
  u.blk = r / p.splits;
  const int split = r % p.splits;
  u.j_begin = split * p.tok_per_split;
  u.bg = block_geo(g, u.blk);
  u.j_end = min(u.j_begin + p.tok_per_split, u.bg.n);
  u.base_tok = u.bg.base;
  u.n_tiles = (u.j_end - u.j_begin + 15) >> 4;
  u.head_off = (int64_t)u.bh * g.N * D;
  u.row = (int64_t)u.bh * g.M + u.blk;
  return u;
}

// Issue the query loads of tile t of unit u into `dst` through a buffer resource over the
// unit's head: tokens past the slice and key features beyond D (d = 16) read as zero.
template <typename TIn, int D, int QPOL>
__device__ inline void rd_issue(const ReadoutParams& p, const RdUnit& u, int t, int lane,
                                In8<TIn> (&dst)[Dims<D>::NKC], bool& v, int64_t& off) {
  constexpr uint32_t ES = sizeof(TIn);
  const int pr = lane & 15, lg = lane >> 4;
  const int32_t j = u.j_begin + t * 16 + pr;
  v = j < u.j_end;
  off = v ? u.head_off + (int64_t)(u.base_tok + block_offset(p.g, u.bg, (uint32_t)j)) * D : 0;
  const Rsrc rsq = make_rsrc(reinterpret_cast<const TIn*>(p.q) + u.head_off, (uint32_t)p.g.N * D * ES);
  const uint32_t rel = (uint32_t)(off - u.head_off);
#pragma unroll
  for (int kc = 0; kc < Dims<D>::NKC; ++kc) {
    const int k0 = 32 * kc + 8 * lg;
    dst[kc].template load_buf<QPOL>(rsq, (v && k0 < D) ? (rel + k0) * ES : kOutOfRange);
  }
}

// Query tiles per wave and step: two (each staged A operand feeds two MFMAs) where the registers
// allow it at 4 waves per SIMD; one at d = 128 and for fp32 inputs.
template <typename TIn, int D>
constexpr int readout_tiles_per_step() { return sizeof(TIn) == 2 && D <= 64 ? MHLA_READOUT_TILES : 1; }
// waves per SIMD the register allocation must allow (fp32 inputs at d = 128 need more registers;
// the bf16 mixing prologue at d <= 64 is held to 8)
template <typename TIn, int D, int FUSE = 0>
constexpr int readout_waves() {
  return FUSE == kFuseBf16 && sizeof(TIn) == 2 && D <= 64 ? 8 : (sizeof(TIn) == 4 && D == 128 ? 3 : 4);
}

// QPOL: cache policy of the query loads (MHLA_READOUT_LOAD_CPOL, or 2 = nt when the queries
// of one launch are larger than about half the infinity cache and would only evict the
// summaries from it).
template <typename TIn, typename TOut, int D, bool SPLIT, int FUSE, int PHI, int QPOL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    readout_waves<TIn, D, FUSE>()))) void readout_kernel(
    ReadoutParams p, int mode) {
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const Geom& g = p.g;
  const RdUnit U = rd_unit<D>(p, blockIdx.x);
  const int bh = U.bh, blk = U.blk;

  // NT tiles per wave and step (tiles wave, wave + 4, ...); the first step's query loads go out
  // before the prologue, each later step's during the previous step
  constexpr int NT = readout_tiles_per_step<TIn, D>();
  constexpr int WSTEP = kThreads / 64;
  In8<TIn> raw[NT][NKC];
  bool valid[NT];
  int64_t toff[NT];
  auto issue_step = [&](int t0) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      valid[j] = false;
      toff[j] = 0;
      if (t0 + j * WSTEP < U.n_tiles) {
        rd_issue<TIn, D, QPOL>(p, U, t0 + j * WSTEP, lane, raw[j], valid[j], toff[j]);
      } else {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) raw[j][kc].zero();
      }
    }
  };
  int tile = wave;
  issue_step(tile);

  // ---- prologue: mixed summary (loaded or formed here), z~, mean of V ------------------
  const int M = g.M;
  // fragment chunks of 8 elements per thread; the prologues take PC of them per pass
  constexpr int PER = (FRAG + kThreads * 8 - 1) / (kThreads * 8);
  // (the mixing prologues take one: fewer loads in flight per thread leave registers for more
  // waves, 8 per SIMD for the bf16 one at d <= 64, and more waves hide a unit's prologue behind
  // the other units' query streams)
  constexpr int PC = FUSE != kFuseNone ? 1 : (PER < 2 ? PER : 2);
  if constexpr (FUSE == kFuseNone) {
    // the mixing kernel's output: every chunk of this thread in flight at once
    const Rsrc rhi = make_rsrc(p.st_hi + U.row * FRAG, FRAG * 2u);
    const Rsrc rlo = make_rsrc(SPLIT ? p.st_lo + U.row * FRAG : p.st_hi, SPLIT ? FRAG * 2u : 0u);
    u32x4_t th[PER], tl[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (tid + j * kThreads) * 8;
      const uint32_t off = i < FRAG ? (uint32_t)i * 2u : kOutOfRange;
      th[j] = buf_ld16(rhi, off);
      if (SPLIT) tl[j] = buf_ld16(rlo, off);
    }
    if (tid < D) s_zt[tid] = p.zt[U.row * D + tid];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (tid + j * kThreads) * 8;
      if (i < FRAG) {
        st16(s_hi + lds_pos<NCT>(i), th[j]);
        if (SPLIT) st16(s_lo + lds_pos<NCT>(i), tl[j]);
      }
    }
  } else if constexpr (FUSE == kFuseBf16) {
    // S~_i = sum_b m_ib S_b and z~_i = sum_b m_ib z_b in fp32 (NULL M_c: M == 1, weight 1)
    const float* mrow =
        p.mc ? p.mc + (int64_t)(bh % p.H) * p.mc_head_stride + (int64_t)blk * M : nullptr;
    // blocks are taken 8 at a time with all 8 loads in flight; blocks >= M read as zero
    // through the buffer resource and carry the weight 0
    const Rsrc rss = make_rsrc(p.sb + (int64_t)bh * M * FRAG, (uint32_t)M * FRAG * 2u);
    auto weight = [&](int b) { return b < M ? (mrow ? mrow[b] : 1.0f) : 0.0f; };
    for (int j0 = 0; j0 < PER; j0 += PC) {
      float a[PC][8];
#pragma unroll
      for (int c = 0; c < PC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[c][e] = 0.f;
      for (int b0 = 0; b0 < M; b0 += 8) {
        u32x4_t w[PC][8];
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          const int i = (tid + (j0 + c) * kThreads) * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            w[c][j] = buf_ld16(rss, (b0 + j < M && i < FRAG) ? (uint32_t)((b0 + j) * FRAG + i) * 2u
                                                             : kOutOfRange);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float m = weight(b0 + j);
#pragma unroll
          for (int c = 0; c < PC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t x = w[c][j][e >> 1];
              a[c][e] = fmaf(m, (e & 1) ? bf16hi_to_f32(x) : bf16lo_to_f32(x), a[c][e]);
            }
        }
      }
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        const int i = (tid + (j0 + c) * kThreads) * 8;
        if (i < FRAG) store_frag8<false>(s_hi, s_lo, lds_pos<NCT>(i), a[c]);
      }
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
      for (int j0 = 0; j0 < PER; j0 += PC) {
        // slices 4 at a time, PC chunks each, all loads in flight; slices >= ss read as zero
        float a[PC][8];
#pragma unroll
        for (int c = 0; c < PC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) a[c][e] = 0.f;
        for (int s0 = 0; s0 < ss; s0 += 4) {
          u32x4_t w[PC][4][2];
#pragma unroll
          for (int c = 0; c < PC; ++c) {
            const int i = (tid + (j0 + c) * kThreads) * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool ok = s0 + j < ss && i < FRAG;
              const uint32_t off = (uint32_t)((s0 + j) * FRAG + i) * 4u;
              w[c][j][0] = buf_ld16(rsp, ok ? off : kOutOfRange);
              w[c][j][1] = buf_ld16(rsp, ok ? off + 16u : kOutOfRange);
            }
          }
#pragma unroll
          for (int c = 0; c < PC; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                a[c][e] += __uint_as_float(w[c][j][0][e]);
                a[c][4 + e] += __uint_as_float(w[c][j][1][e]);
              }
        }
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          const int pos = (tid + (j0 + c) * kThreads) * 8;
          if (pos >= FRAG) continue;
          const int l = (pos >> 3) & 63, fr = pos >> 9;
          const int kc = fr / NCT, ct = fr % NCT;
          const int k0 = 32 * kc + 8 * (l >> 4);
          const float uc = s_ub[16 * ct + (l & 15)] * inv_n;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int k = k0 + e;
            a[c][e] -= (k < D ? s_zt[k] : 0.f) * uc;
          }
          store_frag8<SPLIT>(s_hi, s_lo, lds_pos<NCT>(pos), a[c]);
        }
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
  build_zfrag<D>(s_zt, s_z, tid);
  __syncthreads();

  const AOffsets ao = a_offsets(lane);
  for (; tile < U.n_tiles; tile += NT * WSTEP) {
    In8<TIn> cur[NT][NKC];
    bool cvalid[NT];
    int64_t coff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) cur[j][kc] = raw[j][kc];
      cvalid[j] = valid[j];
      coff[j] = toff[j];
    }
    if (tile + NT * WSTEP < U.n_tiles) issue_step(tile + NT * WSTEP);
    readout_tiles<TIn, TOut, D, SPLIT, NT, PHI>(cur, cvalid, coff, s_hi, s_lo, s_z, s_ub, ao, lane, mode, p.o);
  }
}

template <int PHI, typename TIn, typename TOut, int D, bool SPLIT, int FUSE, int QPOL = MHLA_READOUT_LOAD_CPOL>
static hipError_t launch_t(const ReadoutParams& p, int mode, int n_wg, hipStream_t s) {
  using Dm = Dims<D>;
  const size_t lds = (size_t)Dm::FRAG * 2 * (SPLIT ? 2 : 1) + (size_t)Dm::NKC * 512 * 2 + 2 * D * 4;
  hipLaunchKernelGGL((readout_kernel<TIn, TOut, D, SPLIT, FUSE, PHI, QPOL>), dim3(n_wg), dim3(kThreads), lds,
                     s, p, mode);
  return hipGetLastError();
}

// Valid (split, fuse) pairs: the bf16-stack fusion exists for bf16 operands only; the others
// for both operand precisions.
template <int PHI, typename TIn, typename TOut, int D>
static hipError_t dispatch_fuse(const ReadoutParams& p, int mode, bool split, int fuse, bool q_stream,
                                int n_wg, hipStream_t s) {
  if (split) {
    if (fuse == kFuseNone) return launch_t<PHI, TIn, TOut, D, true, kFuseNone>(p, mode, n_wg, s);
    if (fuse == kFusePartials) return launch_t<PHI, TIn, TOut, D, true, kFusePartials>(p, mode, n_wg, s);
    return hipErrorInvalidValue;
  }
  if constexpr (sizeof(TIn) == 2) {   // the streamed-query variant: bf16 stacks of many blocks
    if (fuse == kFuseNone && q_stream) return launch_t<PHI, TIn, TOut, D, false, kFuseNone, 2>(p, mode, n_wg, s);
  }
  if (fuse == kFuseNone) return launch_t<PHI, TIn, TOut, D, false, kFuseNone>(p, mode, n_wg, s);
  if (fuse == kFusePartials) return launch_t<PHI, TIn, TOut, D, false, kFusePartials>(p, mode, n_wg, s);
  if constexpr (sizeof(TIn) == 2) {
    if (fuse == kFuseBf16) return launch_t<PHI, TIn, TOut, D, false, kFuseBf16>(p, mode, n_wg, s);
  }
  return hipErrorInvalidValue;
}

template <int PHI, typename TIn, typename TOut>
static hipError_t dispatch_d(const ReadoutParams& p, int d, int mode, bool split, int fuse, bool qs,
                             int n_wg, hipStream_t s) {
  switch (d) {
    case 16: return dispatch_fuse<PHI, TIn, TOut, 16>(p, mode, split, fuse, qs, n_wg, s);
    case 32: return dispatch_fuse<PHI, TIn, TOut, 32>(p, mode, split, fuse, qs, n_wg, s);
    case 64: return dispatch_fuse<PHI, TIn, TOut, 64>(p, mode, split, fuse, qs, n_wg, s);
    case 128: return dispatch_fuse<PHI, TIn, TOut, 128>(p, mode, split, fuse, qs, n_wg, s);
    default: return hipErrorInvalidValue;
  }
}

// n_wg = splits * M * BH workgroups (one-dimensional grid).  q_stream: load the queries with the
// non-temporal policy (bf16 inputs, single bf16 operands, a mixing kernel of its own).
hipError_t launch_readout(const ReadoutParams& p, int d, bool in_fp32, bool out_fp32, int mode,
                          bool split, int fuse, bool q_stream, int phi, int n_wg, hipStream_t stream) {
  auto go = [&](auto phi_c) {
    constexpr int PHI = decltype(phi_c)::value;
    if (in_fp32)
      return out_fp32 ? dispatch_d<PHI, float, float>(p, d, mode, split, fuse, q_stream, n_wg, stream)
                      : dispatch_d<PHI, float, uint16_t>(p, d, mode, split, fuse, q_stream, n_wg, stream);
    return out_fp32 ? dispatch_d<PHI, uint16_t, float>(p, d, mode, split, fuse, q_stream, n_wg, stream)
                    : dispatch_d<PHI, uint16_t, uint16_t>(p, d, mode, split, fuse, q_stream, n_wg, stream);
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhla
