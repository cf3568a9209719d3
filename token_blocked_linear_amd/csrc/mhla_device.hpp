// Device-side building blocks shared by the three gfx950 kernels of the MHLA forward:
// launch parameter structs, the block geometry, fast integer division, bf16 packing,
// the feature map and the 16x16x32 bf16 MFMA wrapper.
//
// Summary-stack fragment layout (written by the summary kernel, consumed by mix and readout).
// For head_dim D let NKC = max(D,32)/32 (32-feature chunks of the key dimension k) and
// NCT = D/16 (16-channel tiles of the value dimension c).  Element (kc, ct, lane, e) of a
// d x d summary S holds
//     S[k = 32*kc + 8*(lane/16) + e][c = 16*ct + lane%16],     e = 0..7,
// at flat index ((kc*NCT + ct)*64 + lane)*8 + e.  One (kc, ct) fragment is therefore exactly
// the per-lane A operand of a v_mfma_f32_16x16x32_bf16 whose rows are the 16 channels c and
// whose contraction runs over the 32 key features k, so the readout loads it with one
// 16-byte read per lane.  Rows k >= D (only when D = 16) are zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

// Cache policy (the aux operand of buffer loads; 2 = nt: lines are kept only briefly) for the
// data each kernel streams once, and whether the readout's output stores are non-temporal.
#ifndef MHLA_SUMMARY_LOAD_CPOL
#define MHLA_SUMMARY_LOAD_CPOL 2      // K, V
#endif
#ifndef MHLA_MIX_LOAD_CPOL
#define MHLA_MIX_LOAD_CPOL 0          // the summary stack (default: it is read from the infinity cache)
#endif
#ifndef MHLA_READOUT_LOAD_CPOL
#define MHLA_READOUT_LOAD_CPOL 0      // Q
#endif
#ifndef MHLA_READOUT_TILES
#define MHLA_READOUT_TILES 1          // 16-token query tiles per readout wave and step (d <= 64)
#endif
#ifndef MHLA_READOUT_STORE_NT
#define MHLA_READOUT_STORE_NT 0       // O
#endif

namespace mhla {

constexpr int kThreads = 256;  // every kernel runs 4 wave64s per workgroup

template <int D> struct Dims {
  static constexpr int DK = D < 32 ? 32 : D;   // key dimension padded to the MFMA K=32 chunk
  static constexpr int NKC = DK / 32;
  static constexpr int NCT = D / 16;
  static constexpr int FRAG = NKC * NCT * 512; // elements of one fragment-layout summary
};

// Token-grid geometry, padded to 3 axes with leading extents of 1.
struct Geom {
  int32_t G1, G2;          // grid extents of axes 1 and 2
  int32_t B0, B1, B2;      // block extents (of a whole block)
  int32_t NB1, NB2;        // block-grid extents of axes 1 and 2 (rounded up)
  FastDiv fB2, fB1;        // divide block-local token indices of a whole block
  int32_t n_b;             // tokens of a whole block (the most a block holds)
  int32_t N;               // tokens per head (the CLS token included)
  int32_t M;               // blocks per head (the CLS block included)
  int32_t G0;              // grid extent of axis 0
  int32_t cls;             // 1: token 0 is a CLS token forming block 0; grid tokens follow
};

// One block's place in the sequence: first token, token count, extents along axes 1 and 2 and
// their divisors.  With ragged blocks the last block along an axis keeps what is left of the
// grid; the CLS block is its one token.
struct BlockGeo {
  int32_t base, n, e1, e2;
  FastDiv f2, f1;
};
__device__ inline BlockGeo block_geo(const Geom& g, int32_t b) {
  BlockGeo r;
  if (g.cls) {
    if (b == 0) {
      r.base = 0;
      r.n = 1;
      r.e1 = r.e2 = 1;
      r.f2 = r.f1 = FastDiv{1u, 1u, 0u};
      return r;
    }
    --b;
  }
  const int32_t b2 = b % g.NB2, t = b / g.NB2;
  const int32_t b1 = t % g.NB1, b0 = t / g.NB1;
  const int32_t c0 = b0 * g.B0, c1 = b1 * g.B1, c2 = b2 * g.B2;
  const int32_t e0 = min(g.B0, g.G0 - c0);
  r.e1 = min(g.B1, g.G1 - c1);
  r.e2 = min(g.B2, g.G2 - c2);
  r.base = g.cls + (c0 * g.G1 + c1) * g.G2 + c2;
  r.n = e0 * r.e1 * r.e2;
  r.f2 = r.e2 == g.B2 ? g.fB2 : make_fastdiv((uint32_t)r.e2);
  r.f1 = r.e1 == g.B1 ? g.fB1 : make_fastdiv((uint32_t)r.e1);
  return r;
}

// Raster token index of block-local token j (0 <= j < n) relative to the block's first token.
__device__ inline int32_t block_offset(const Geom& g, const BlockGeo& bg, uint32_t j) {
  const uint32_t q2 = fdiv(j, bg.f2);
  const uint32_t j2 = j - q2 * (uint32_t)bg.e2;
  const uint32_t j0 = fdiv(q2, bg.f1);
  const uint32_t j1 = q2 - j0 * (uint32_t)bg.e1;
  return (int32_t)((j0 * (uint32_t)g.G1 + j1) * (uint32_t)g.G2 + j2);
}

// ---------------------------------------------------------------------------------------
// Launch parameters
// ---------------------------------------------------------------------------------------
struct SummaryParams {
  const void* k;           // [BH][N][D] of the input dtype
  const void* v;
  uint16_t* sb;            // bf16 summaries [BH][M][FRAG] (one token slice, bf16 operands)
  float* ps;               // partial summaries  [BH][M][splits][FRAG]   (fp32)
  float* pz;               // partial normaliser [BH][M][splits][D]      (fp32)
  float* pu;               // partial sum of V   [BH][M][splits][D]      (fp32, MALA only)
  Geom g;
  int32_t splits;          // token slices per block
  int32_t tok_per_split;
  // Side job for the MFMA mixing path: convert M_c (fp32) once per forward into bf16 operand
  // fragments mcf[(h*nitp + it)*nbc + bc][lane][8] = M_c[h][16 it + lane%16][32 bc + 8(lane/16) + e]
  // (zero outside M x M).  mcf == nullptr: nothing to convert.
  const float* mc;
  int64_t mc_head_stride;
  uint16_t* mcf;
  uint16_t* mcf_lo;        // non-null: also the low parts (M_c = hi + lo, for the split mixing)
  int32_t mcf_transposed;  // 1: fragments of M_c^T (the backward's mixing)
  int32_t mcf_causal;      // 1: only the strictly lower part of M_c (entries b >= i are zero)
  int32_t mcf_heads, mcf_nitp, mcf_nbc;
  // Per-token weights (the backward's summary): phi(K_j) scaled by kscale[j], the normaliser
  // product weighted by zw[j]; [BH][N] fp32 each.
  const float* kscale;
  const float* zw;
};

// Launch shape of the MFMA mixing kernel for M blocks: nbc 32-block chunks of the contraction,
// itw 16-row i-tiles per wave, wave_rows waves sharing a row group's i-tiles, row_groups
// workgroups per column tile.  Shared by the host plan and the kernel launcher.  `split`: fp32
// partials and M_c as hi + lo; `wlo`: the bf16 stack against M_c as hi + lo (both hold twice the
// W fragments, so beyond 128 blocks they take the 8-wave shape).
struct MixShape {
  int nbc, itw, wave_rows, row_groups, nitp, nw;
};
inline MixShape mix_shape(int M, bool split, bool wlo = false) {
  MixShape s;
  const int nbc = (M + 31) / 32;
  s.nbc = nbc <= 1 ? 1 : nbc <= 2 ? 2 : nbc <= 4 ? 4 : 8;
  const int nit = (M + 15) / 16;
  s.nw = 4;
  if ((split || wlo) && s.nbc == 8) {
    // split, M > 128: one workgroup of 8 waves x 2 i-tiles covers all 256 rows, so the tile is
    // loaded, split and transposed once (four 4-wave row groups would each do it)
    s.nw = 8;
    s.itw = 2;
    s.wave_rows = 8;
    s.row_groups = 1;
    s.nitp = 16;
    return s;
  }
  const int itw = nit <= 4 || split ? 1 : (nit + 3) / 4;   // split: one i-tile per wave
  s.itw = itw <= 1 ? 1 : itw <= 2 ? 2 : 4;
  s.wave_rows = 4;
  while (s.wave_rows > 1 && (s.wave_rows / 2) * s.itw >= nit) s.wave_rows /= 2;
  const int rows_per_wg = s.wave_rows * s.itw * 16;
  s.row_groups = (M + rows_per_wg - 1) / rows_per_wg;
  s.nitp = s.row_groups * s.wave_rows * s.itw;
  return s;
}

struct MixParams {
  const float* ps;
  const float* pz;
  const float* pu;
  const float* mc;         // fp32 [M][M] or [H][M][M]
  int64_t mc_head_stride;  // 0 or M*M
  uint16_t* st_hi;         // mixed summaries, bf16 bits [BH][M][FRAG]
  uint16_t* st_lo;         // low parts (split accuracy) or nullptr
  float* zt;               // mixed normaliser [BH][M][D]
  int32_t M;
  int32_t splits;          // token slices per block of ps
  int32_t H;
  int32_t N;
  int32_t zsplits;         // token slices per block of pz
  int32_t mc_transposed;   // 1: mix with M_c^T (the backward's dS_b = sum_i m_ib dS~_i)
  int32_t causal;          // 1: weights m_ib with b >= i are taken as zero
};

// Backward pass (chain rule of the forward steps; see csrc/bwd.hip).
struct BwdParams {
  const void* q;           // [BH][N][D] input type
  const void* k;
  const void* v;
  const void* dout;        // [BH][N][D] output type
  void* dq;                // [BH][N][D] output type
  void* dk;
  void* dv;
  const uint16_t* st_hi;   // mixed summaries S~ (fragments, bf16 hi / lo) [BH][M][FRAG]
  const uint16_t* st_lo;
  const float* zt;         // z~ [BH][M][D]
  const uint16_t* ds_hi;   // dS = M_c^T dS~ (fragments, hi / lo) [BH][M][FRAG]
  const uint16_t* ds_lo;
  const float* dz;         // dz [BH][M][D]
  float* tok_scale;        // per token 1/den (1 unnormalised) [BH][N]
  float* tok_zw;           // per token -(dO . o) (0 unnormalised) [BH][N]
  float* du_part;          // MALA: per unit sum_t s_t dO_t over its tokens [BH][splits][D]
  const float* du;         // MALA: dL/du added to every dv [BH][D]; NULL otherwise
  Geom g;
  int32_t splits;          // token slices per block (readout slicing)
  int32_t tok_per_split;
  int32_t BH;
  int32_t xcd_map;
};

// MALA backward, one block per (batch, head): sums of the token-slice partials into fragments.
//   stage 0 (forward):  C = S - z u^T / N (hi / lo), z, u / N
//   stage 1 (backward): dS (hi / lo), dz = dz' - dS (u / N), du = -(1/N) sum over units of du_part
struct MalaStageParams {
  const float* ps;         // fp32 fragment partials [BH][ss][FRAG]: S (stage 0) or dS (stage 1)
  const float* pz;         // [BH][ss][D]: z or dz'
  const float* pu;         // stage 0: [BH][ss][D] partials of u
  const float* ub;         // stage 1: u / N [BH][D]
  const float* du_part;    // stage 1: [BH][rs][D]
  uint16_t* y_hi;          // [BH][FRAG]
  uint16_t* y_lo;
  float* zo;               // [BH][D]
  float* ub_out;           // stage 0: u / N [BH][D]
  float* du;               // stage 1: [BH][D]
  int32_t ss;              // token slices of the partials
  int32_t rs;              // units per head of du_part
  int32_t N;
  int32_t stage;
};

// dM_c partials per (batch, head): dmc[bh][i][b] = <dS~_i, S_b> + <dz~_i, z_b>, summaries summed
// over their token slices on the fly.
// The contraction runs over (batch-head, position) pairs of a group: every (batch, head) for a
// shared M_c, every batch item of head g for a per-head one (bh = j*H + g).  It is cut into
// `nchunks` chunks of `steps_per_chunk` 64-position steps, each chunk giving one partial.
// dM_c output tile (rows and columns) of one workgroup: 128 once M > 64, else 64.
__host__ __device__ constexpr int dmc_tile(int M) { return M > 64 ? 128 : 64; }

struct DmcParams {
  const float* dps;        // dS~ partials [BH][M][ssplits][FRAG]
  const float* ps;         // S partials   [BH][M][ssplits][FRAG]
  const float* dpz;        // dz~ partials [BH][M][zsplits_d][D]
  const float* pz;         // z partials   [BH][M][ssplits][D]
  float* out;              // partials [groups][nchunks][M][M]
  int32_t M, frag, D, ssplits, zsplits_d;
  int32_t H, per_head, group_bh;           // group_bh: (batch, head) pairs per group
  int32_t steps_per_bh;                    // ceil((FRAG + D) / 64)
  int32_t nchunks, steps_per_chunk;
};

// Chunkwise-causal readout of a 1D sequence: query t of block i sees the earlier blocks through
// S~<_i = sum_{b<i} m_ib S_b (the mixing kernel with the strictly lower part of M_c), the earlier
// token slices of its own block through their summed partials, and its own slice causally.
struct CausalParams {
  const void* q;           // [BH][N][D] input type
  const void* k;
  const void* v;
  void* o;                 // [BH][N][D] output type
  const uint16_t* st_hi;   // S~<_i fragments (hi, lo) [BH][M][FRAG]; NULL when M == 1
  const uint16_t* st_lo;   // NULL also after the bf16 mixing (single bf16 operands)
  const float* zt;         // z~<_i [BH][M][D]; NULL when M == 1
  const float* pre;        // exclusive prefix over token slices of the block's partial summaries
  const float* prez;       //   [BH][M][splits][FRAG] and [..][D]; NULL with one slice per block
  const float* mc;         // M_c (for m_ii); NULL when M == 1
  int64_t mc_head_stride;
  int32_t H;
  Geom g;
  int32_t splits;          // token slices per block
  int32_t tok_per_split;
  int32_t BH;
  int32_t xcd_map;
  int32_t normalized;
  int32_t split;           // 1: split (hi / lo) operands throughout (the slice kernel's precision)
};

// Streaming decode step (one token per (batch, head)); the state layout is in decode.hip.
struct DecodeParams {
  float* state;            // per (batch, head): (M + 2) * (D*D + slices*D) floats
  const void* q;           // [BH][D] of the input dtype (the new token)
  const void* k;
  const void* v;
  void* o;                 // [BH][D] of the output dtype
  const float* mc;         // M_c; NULL when M == 1
  int64_t mc_head_stride;
  int64_t t;               // the token's position
  int32_t H, M, nb, BH;    // nb: tokens per block
  int32_t normalized;
  int32_t log2_c;          // channels per workgroup = 2^log2_c (8 .. D); D >> log2_c workgroups per head
  int32_t cls;             // 1: position 0 is a CLS token, a block of its own; blocks of nb follow
};

// The decode state after positions 0 .. n-1, from a chunkwise causal forward over them: its
// summaries (fp32 slice partials) and its mixing with the strictly lower M_c (hi + lo).
struct PrefillStateParams {
  float* state;            // the decode state (layout of decode_step_kernel)
  const float* part;       // fp32 partials [BH][Mp][splits][FRAG] (fragment layout)
  const float* pz;         // fp32 partials [BH][Mp][splits][D]
  const uint16_t* st_hi;   // mixed summaries [BH][Mp][FRAG] (hi, lo); NULL when Mp == 1
  const uint16_t* st_lo;
  const float* zt;         // mixed normalisers [BH][Mp][D]; NULL when Mp == 1
  int32_t splits, BH, Mp, M;   // Mp: blocks of the prefix (the last one holds position n - 1); M: the plan's
  int32_t frag, log2_c;
};

// MFMA mixing of a bf16 summary stack: Y[i] = sum_b M_c[i][b] X[b] over fragment positions,
// plus the fp32 normaliser mixing z~[i] = sum_b M_c[i][b] z[b].
struct MixMfmaParams {
  const uint16_t* x;       // bf16 [BH][M][FRAG] (bf16 kernel)
  const float* xf;         // fp32 partials [BH][M][xsplits][FRAG] (split kernel)
  const float* z;          // fp32 partials [BH][M][zsplits][D]
  const uint16_t* mcf;     // bf16 W operand fragments (see SummaryParams); hi part if split
  const uint16_t* mcf_lo;  // low part (split kernel, and the bf16 kernel with W as hi + lo)
  int32_t mcf_per_head;    // 1: fragments per head, 0: shared
  uint16_t* y;             // bf16 [BH][M][FRAG]; hi part if split
  uint16_t* y_lo;          // low part (split kernel)
  float* zt;               // fp32 [BH][M][D]
  int32_t xsplits, zsplits;
  int32_t M;
  int32_t H;
  int32_t D;
  int32_t frag;
  int32_t n_wg_x;          // workgroups per (head, row group) striding over column tiles
  int32_t wave_rows;       // waves sharing the i-tiles of a row group (1, 2 or 4)
};

struct ReadoutParams {
  const void* q;           // [BH][N][D] of the input dtype
  void* o;                 // [BH][N][D] of the output dtype
  const uint16_t* st_hi;   // mixed summaries from the mixing kernel (not fused)
  const uint16_t* st_lo;
  const float* zt;
  Geom g;
  int32_t splits;          // token slices per query block
  int32_t tok_per_split;
  int32_t BH;
  int32_t xcd_map;         // 1: all workgroups of a head on one XCD (BH % 8 == 0)
  // inputs of a mixing step fused into the prologue
  const uint16_t* sb;      // bf16 summary stack [BH][M][FRAG]                 (bf16 fusion)
  const float* ps;         // fp32 partial summaries [BH][M][ssplits][FRAG]     (partials fusion)
  const float* pz;         // normaliser partials [BH][M][ssplits][D]
  const float* pu;         // sum of V partials   [BH][M][ssplits][D]           (MALA)
  const float* mc;         // fp32 [M][M] or [H][M][M]; NULL when M == 1
  int64_t mc_head_stride;
  int32_t H;
  int32_t ssplits;         // token slices of the summary kernel
};

// ---------------------------------------------------------------------------------------
// Numerics helpers
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even (gfx950 converts natively); returns the 16-bit pattern.
__device__ inline uint32_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (RNE) in one word, `lo` in the low half: one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// hi = bf16(x), lo = bf16(x - hi): x == hi + lo to about 2^-17 relative.
__device__ inline void split_bf16(float x, uint32_t& hi_bits, uint32_t& lo_bits) {
  hi_bits = f32_to_bf16_bits(x);
  lo_bits = f32_to_bf16_bits(x - __uint_as_float(hi_bits << 16));
}

// split_bf16 of two values at once, packed like pack_bf16x2 (x0 in the low halves).
__device__ inline void split_bf16x2(float x0, float x1, uint32_t& hi2, uint32_t& lo2) {
  hi2 = pack_bf16x2(x0, x1);
  lo2 = pack_bf16x2(x0 - __uint_as_float(hi2 << 16), x1 - __uint_as_float(hi2 & 0xffff0000u));
}

// Feature maps ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// Background: a positive phi; "Rectifying Magnitude Neglect in Linear Attention", Ablation: ELU+1,
// ReLU and exp work alike).  Numbering as mhla_phi in include/mhla.h.
enum { kPhiElu1 = 0, kPhiRelu = 1, kPhiExp = 2 };

// ELU(x) + 1 with alpha = 1.
__device__ inline float phi_elu1(float x) {
  return x > 0.0f ? x + 1.0f : __expf(x);
}

template <int PHI>
__device__ inline float phi_map(float x) {
  if constexpr (PHI == kPhiRelu) return fmaxf(x, 0.0f);
  else if constexpr (PHI == kPhiExp) return __expf(x);
  else return phi_elu1(x);
}

__device__ inline f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16-byte global loads and stores.
__device__ inline u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ inline void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
template <bool NT>
__device__ inline void st16_pol(void* p, u32x4_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
  else *reinterpret_cast<u32x4_t*>(p) = v;
}

// Buffer resources (V#): a base address and a byte range.  A raw buffer load whose offset lies
// outside the range returns zeros instead of touching memory, so guarded loads need no branch
// (branches around loads make the compiler wait for every outstanding load).  The last word
// is the gfx9-family untyped-buffer configuration.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;   // >= every range used here (ranges < 2^31)

__device__ inline Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
template <int CPOL = 0>
__device__ inline u32x4_t buf_ld16(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CPOL));
}
__device__ inline u32x2_t buf_ld8(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}
// Buffer store: a store whose offset lies outside the range is dropped, so a lane with nothing
// to write needs no branch.  (The vector-memory counter counts stores as well as loads and
// drains in issue order; with a branch around stores the count differs between paths and the
// compiler waits on the smallest count, i.e. for those stores too.)
template <int CPOL = 0>
__device__ inline void buf_st16(Rsrc r, uint32_t byte_off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, CPOL);
}
__device__ inline void buf_st4(Rsrc r, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_off, 0, 0);
}

// Input element loaders: 8 consecutive elements starting at element index `idx` as fp32.
template <typename T> struct In8;
template <> struct In8<uint16_t> {       // bf16 bits
  u32x4_t w;
  __device__ inline void load(const void* base, int64_t idx) {
    w = ld16(reinterpret_cast<const uint16_t*>(base) + idx);
  }
  template <int CPOL>
  __device__ inline void load_buf(Rsrc r, uint32_t byte_off) { w = buf_ld16<CPOL>(r, byte_off); }
  __device__ inline void zero() { w = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ inline float get(int e) const {
    uint32_t x = w[e >> 1];
    return (e & 1) ? bf16hi_to_f32(x) : bf16lo_to_f32(x);
  }
  __device__ inline uint32_t bits(int e) const {   // exact bf16 bits (no rounding needed)
    uint32_t x = w[e >> 1];
    return (e & 1) ? (x >> 16) : (x & 0xffffu);
  }
};
template <> struct In8<float> {
  u32x4_t w0, w1;
  __device__ inline void load(const void* base, int64_t idx) {
    const float* p = reinterpret_cast<const float*>(base) + idx;
    w0 = ld16(p);
    w1 = ld16(p + 4);
  }
  template <int CPOL>
  __device__ inline void load_buf(Rsrc r, uint32_t byte_off) {
    w0 = buf_ld16<CPOL>(r, byte_off);
    w1 = buf_ld16<CPOL>(r, byte_off == kOutOfRange ? kOutOfRange : byte_off + 16u);
  }
  __device__ inline void zero() {
    w0 = u32x4_t{0u, 0u, 0u, 0u};
    w1 = w0;
  }
  __device__ inline float get(int e) const { return __uint_as_float(e < 4 ? w0[e] : w1[e - 4]); }
};

}  // namespace mhla
