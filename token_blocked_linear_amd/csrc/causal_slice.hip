// Chunkwise-causal MHLA readout for bf16 inputs: each token slice is read out against the slice's
// start state plus the masked products inside the slice.
//
// "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method -> Key
// design 2 (the token-expanded identity q~^T S~_i = sum_t m_{i,b(t)} (q~^T K~_t) V_t^T) and Key
// design 4 (chunkwise-parallel training).  Query t of block i, in the slice [j0, j1) of its block:
//   num_t = q~_t^T S0 + sum_{j0 <= j <= t} (q~_t . m_ii k~_j) v_j
//   den_t = q~_t^T z0 + sum_{j0 <= j <= t} (q~_t . m_ii k~_j)
// with S0 = S~<_i + m_ii P_s (the mixing kernel's strictly lower part of M_c, plus the exclusive
// prefix of the block's earlier slices) and z0 likewise -- the quantities of causal.hip, grouped
// so that no running state is rewritten inside the slice and the waves own disjoint query tiles.
//
// A persistent grid (one 8-wave workgroup per CU; two at d = 32) walks the units (batch-head,
// block, slice of at most 256 tokens = 16 query tiles); wave w owns query tiles w and 15 - w, so
// every wave meets 17 (query, key) tile pairs of a full slice.  Per unit:
//   1. phi(q) of the wave's tiles, from LDS (loaded there for this unit by direct-to-LDS DMA while
//      the previous unit was computed), becomes MFMA B operands in registers.  den0 = q~ . z0
//      follows on a few MFMAs whose A operand (rows 4g: hi(z0), 4g + 1: lo(z0)) is built from a
//      z0 row that the previous unit DMA'd into a per-wave slot of the V space; it seeds the
//      normaliser sum.  The wave then starts the DMA of its tiles of the next unit.
//   2. The slice's keys go to LDS in phases of 128 (d = 128) or 256 keys: m_ii phi(K) rows (hi /
//      lo with split operands) and V (bf16, exact), both with 16-byte chunks XOR-swizzled by row
//      so that the operand reads and the transposing reads are conflict-free.  The registers
//      that fed a phase load the next one (or the next unit's first) meanwhile.  With two
//      phases, phase ph takes the slice's 32-key pairs 2p + ph: every wave then has about the
//      same number of active pairs in each phase, which the barrier between phases needs.  Per
//      key tile kt <= t: scores D[j][t] = m_ii phi(k_j) . q~_t on 16x16x32 MFMAs (keys as A
//      rows), masked to j <= t on the diagonal tile; a lane then holds keys 4g .. 4g+3 of query
//      t, the B operand of V^T P as it stands.  Two key tiles form one 16x16x32 step of V^T P
//      whose A operand (channel rows, keys 4g .. 4g+3 of each tile) is two ds_read_b64_tr_b16 of
//      V.
//   3. The readout against S0: O^T += S0^T q~ with permuted A rows (lane (t, g) ends with
//      channels 8g .. 8g+7 of each 32-channel pair).  An S0 that is a bf16 fragment stack read
//      with single operands is DMA'd into the LDS space that the keys' low parts would take
//      (unused then), in the readout kernel's bank-spreading order, at the unit's last phase;
//      otherwise the A operands come straight from global memory (the unit's waves share them
//      in L2) and are combined and split in registers.
//   4. o_t = num_t / den_t (normalised) or num_t, 16-byte stores.
// SPLIT (the plan's split accuracy) takes every product on hi / lo operand pairs.  Otherwise
// phi(q) and m_ii phi(K) are single bf16 operands, the precision at which the non-causal forward
// reads out bf16 ELU+1 inputs (scores and the readout of S0 on one MFMA each); P stays split in
// both: the weighted sums of V cancel (V has both signs), so a rounding of the weights by up to
// 2^-8 relative grows with the number of keys and alone would exceed the causal readout's bar.
#include <type_traits>

#include "frag_lds.hpp"

namespace mhla {

namespace {

typedef short cs16x4_t __attribute__((ext_vector_type(4)));
typedef int32_t cs_i32x4_t __attribute__((ext_vector_type(4)));
#define MHLA_CS_LDS __attribute__((address_space(3)))

// Two transposing LDS reads (4 rows x 16 columns each, 16-lane groups) as one 8 x bf16 operand.
__device__ inline u32x4_t cs_tr_pair(const MHLA_CS_LDS char* p0, const MHLA_CS_LDS char* p1) {
  const cs16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MHLA_CS_LDS cs16x4_t*)p0);
  const cs16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MHLA_CS_LDS cs16x4_t*)p1);
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

// A buffer resource as four scalar words for the inline assembly (as make_rsrc).
__device__ inline cs_i32x4_t cs_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return cs_i32x4_t{(int32_t)(uint32_t)a, (int32_t)(uint32_t)((a >> 32) & 0xffffu), (int32_t)bytes, 0x00020000};
}

// One 16-byte load per lane into LDS at lds_byte + 16 * lane (lds_byte wave-uniform); voff is the
// lane's byte offset into the resource (out of range: the lane writes zeros).  No register
// output; completion is awaited with vmcnt.
__device__ inline void cs_dma16(uint32_t lds_byte, uint32_t voff, cs_i32x4_t rs) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rs)
               : "memory");
}

// vmcnt(N) alone; lgkmcnt(0) alone (gfx9 s_waitcnt encodings, other counters at their maxima)
template <int N>
__device__ inline void cs_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ inline void cs_wait_vm0() { cs_wait_vm<0>(); }
__device__ inline void cs_wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace

template <int D>
struct SliceShape {
  static constexpr int NW = 8, NT = 64 * NW;         // waves, threads per workgroup
  static constexpr int KH = D >= 128 ? 128 : 256;    // keys per phase
  static constexpr int KT = KH / 16;                 // key tiles per phase
  static constexpr int NPH = 256 / KH;               // phases of a full (256-token) slice
  static constexpr int NCH = D / 8;                  // 16-byte chunks per token row
  static constexpr int RPT = KH * NCH / NT;          // K (and V) chunks staged per thread per phase
  static constexpr int QDMA = 16 * NCH / 64;         // DMA instructions per query tile
  // LDS: m_ii phi(K) hi, lo and V for one phase, then the query rows of the 16 tiles
  static constexpr size_t K_BYTES = (size_t)KH * D * 2;
  static constexpr size_t Q_OFF = 3 * K_BYTES;
  static constexpr size_t LDS = Q_OFF + (size_t)256 * D * 2;
  static constexpr int PER_CU = LDS * 2 <= 160 * 1024 ? 2 : 1;   // workgroups per CU
};

// Row swizzle of the query and key rows: the 16 rows that one operand read meets (16 lanes, one
// chunk each) land on 16 different bank groups.
template <int D>
__device__ inline int row_swz(int r) {
  if constexpr (D == 128) return r & 15;
  else if constexpr (D == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}
// V row r: chunk c at c ^ v_swz(r) (the 16 lanes of a transposing read meet 4 rows x 4 chunks)
template <int D>
__device__ inline int v_swz(int r) {
  if constexpr (D == 128) return (r & 3) << 2;
  else if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  else return 0;
}

// S0_PLAIN: S0 comes from the bf16 stack alone (no low parts, no slice prefix) and is exact in
// bf16, so its A operands are the stack's words as they are.
template <typename TOut, int D, int PHI, bool S0_PLAIN, bool SPLIT>
__global__ __launch_bounds__(SliceShape<D>::NT) void causal_slice_kernel(CausalParams p, int n_units) {
  static_assert(D >= 32, "head sizes 32, 64 and 128");
  using Dm = Dims<D>;
  using SS = SliceShape<D>;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG, NG = NCT / 2;
  constexpr int NT = SS::NT, KH = SS::KH, KT = SS::KT, NCH = SS::NCH, RPT = SS::RPT, QDMA = SS::QDMA;
  constexpr int NPH = SS::NPH;
  static_assert(RPT >= 1 && KH * NCH % NT == 0 && QDMA >= 1, "staging shape");
  constexpr int NST = 2 * NG * (sizeof(TOut) == 4 ? 2 : 1);   // output stores per wave and unit

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* k_hi = smem;                          // m_ii phi(K) [KH][D] (chunks swizzled)
  uint16_t* k_lo = k_hi + KH * D;
  uint16_t* v_s = k_lo + KH * D;                  // V [KH][D] (chunks swizzled)
  uint16_t* q_s = v_s + KH * D;                   // raw queries [16 tiles][16][D] (chunks swizzled)
  const uint32_t q_lds = (uint32_t)(uintptr_t)(MHLA_CS_LDS char*)smem + (uint32_t)SS::Q_OFF;
  // S0 through LDS: the space of the keys' low parts (FRAG <= KH * D elements)
  constexpr bool S0_LDS = S0_PLAIN && !SPLIT;
  static_assert(FRAG <= KH * D, "S0 space");
  uint16_t* s0_s = k_lo;
  const uint32_t s0_lds = (uint32_t)(uintptr_t)(MHLA_CS_LDS char*)smem + (uint32_t)SS::K_BYTES;

  // the wave index in a scalar register: the per-wave branches below are uniform ones.  The
  // thread index is made opaque at the start of every unit (tid_v) so that the compiler
  // recomputes lane-dependent offsets there instead of keeping dozens of them live (and spilled)
  // across the whole loop.
  int tid_v = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid_v >> 6);
  const int qtile[2] = {wave, 15 - wave};
  const Geom& geo = p.g;

  struct Unit {
    int bh, split;
    int32_t j_begin, j_end, base;   // slice [j_begin, j_end) of a block starting at token base
    int n_tiles;
    int64_t head_off, row;
    float mii;
  };
  auto decode = [&](int L) {
    const int per_head = p.splits * geo.M;
    int r;
    Unit U;
    if (p.xcd_map) {
      const int xcd = L & 7, sl = L >> 3;
      U.bh = (sl / per_head) * 8 + xcd;
      r = sl % per_head;
    } else {
      U.bh = L / per_head;
      r = L % per_head;
    }
    const int blk = r / p.splits;
    U.split = r % p.splits;
    const BlockGeo bg = block_geo(geo, blk);
    U.j_begin = U.split * p.tok_per_split;
    U.j_end = min(U.j_begin + p.tok_per_split, bg.n);
    U.base = bg.base;                 // a 1D block: its tokens are consecutive
    U.n_tiles = (U.j_end - U.j_begin + 15) >> 4;
    U.head_off = (int64_t)U.bh * geo.N * D;
    U.row = (int64_t)U.bh * geo.M + blk;
    // m_ii through the scalar cache (an input the kernel never writes, at a uniform address), so
    // that the next unit's value waits in a scalar register rather than a vector one
    typedef const __attribute__((address_space(4))) float ConstF;
    U.mii = p.mc ? *(ConstF*)(p.mc + (int64_t)(U.bh % p.H) * p.mc_head_stride + (int64_t)blk * geo.M + blk) : 1.0f;
    return U;
  };
  constexpr uint32_t ES = 2;
  const uint32_t head_bytes = (uint32_t)geo.N * D * ES;
  // element offset (within the head) of slice-relative token j
  auto tok = [&](const Unit& U, int32_t j) -> uint32_t { return (uint32_t)(U.base + U.j_begin + j) * D; };

  // the wave's query tiles of unit U into LDS (rows past the slice read as zero)
  auto dma_q = [&](const Unit& U) {
    const int lane = tid_v & 63;
    const cs_i32x4_t rs = cs_rsrc_words(reinterpret_cast<const uint16_t*>(p.q) + U.head_off, head_bytes);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (qtile[t] >= U.n_tiles) continue;   // uniform
#pragma unroll
      for (int i = 0; i < QDMA; ++i) {
        const int idx = i * 64 + lane, rr = idx / NCH, c = (idx % NCH) ^ row_swz<D>(rr);
        const int32_t j = 16 * qtile[t] + rr;
        const uint32_t voff = U.j_begin + j < U.j_end ? (tok(U, j) + 8 * c) * ES : kOutOfRange;
        cs_dma16(q_lds + (uint32_t)((qtile[t] * 16 * D + i * 512) * 2), voff, rs);
      }
    }
  };
  // Phases take the slice's key pairs (32 keys, two tiles) round robin: local pair kp of phase ph
  // is pair kp * NPH + ph.  Every wave then meets about the same number of active pairs in each
  // phase (its two query tiles w and 15 - w see the causal triangle's short and long rows), where
  // consecutive key ranges would load the waves' barriers unevenly.  Slice-relative key of local
  // key row rr of phase ph:
  auto key_of = [](int ph, int rr) -> int32_t { return 32 * ((rr >> 5) * NPH + ph) + (rr & 31); };
  // K and V of phase ph of unit U into registers (rows past the slice read as zero)
  In8<uint16_t> ck[RPT], cv[RPT];
  auto issue_kv = [&](const Unit& U, int ph) {
    const int tid = tid_v;
    const Rsrc rk = make_rsrc(reinterpret_cast<const uint16_t*>(p.k) + U.head_off, head_bytes);
    const Rsrc rv = make_rsrc(reinterpret_cast<const uint16_t*>(p.v) + U.head_off, head_bytes);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int idx = tid + i * NT, rr = idx / NCH, c = idx % NCH;
      const int32_t j = key_of(ph, rr);
      const uint32_t off = U.j_begin + j < U.j_end ? (tok(U, j) + 8 * c) * ES : kOutOfRange;
      ck[i].template load_buf<0>(rk, off);
      cv[i].template load_buf<0>(rv, off);
    }
  };

  // z0 of unit X (the slice's start normaliser: the mixed z~ row plus m_ii times the in-block
  // prefix of earlier slices) into the wave's own 2 KB slot of the V space: the z~ row at +0, the
  // prefix row at +1 KB (one 16-byte DMA per lane each; lanes past the row write zeros).  Issued
  // where no wave reads the V space until the next unit's first staging, older than the wave's
  // output stores, so that the wait at the top of the next unit covers it.
  float* const z_slot = reinterpret_cast<float*>(v_s) + wave * 512;
  const uint32_t z_lds = (uint32_t)(uintptr_t)(MHLA_CS_LDS char*)smem + (uint32_t)(2 * SS::K_BYTES) + (uint32_t)wave * 2048u;
  static_assert(8 * 2048 <= SS::K_BYTES, "z0 slots");
  auto dma_z = [&](const Unit& X) {
    const int lane = tid_v & 63;
    const uint32_t voff = lane < D / 4 ? (uint32_t)lane * 16u : kOutOfRange;
    if (p.zt) cs_dma16(z_lds, voff, cs_rsrc_words(p.zt + X.row * D, D * 4u));
    if (p.prez) cs_dma16(z_lds + 1024u, voff, cs_rsrc_words(p.prez + (X.row * p.splits + X.split) * D, D * 4u));
  };

  int L = blockIdx.x;
  Unit U = decode(L);
  dma_q(U);
  issue_kv(U, 0);
  dma_z(U);

  for (;;) {
    asm volatile("" : "+v"(tid_v));
    const int tid = tid_v, lane = tid & 63, pr = lane & 15, lg = lane >> 4;
    const int Ln = L + gridDim.x;
    const bool has_next = Ln < n_units;
    // this unit's query rows (DMA) and first K, V phase have landed: only the previous unit's
    // NST output stores may be newer (none before the first unit)
    if (L == (int)blockIdx.x) cs_wait_vm0();
    else cs_wait_vm<NST>();

    // ---- 1. phi(q) as hi / lo B operands (lane: token pr, features 32kc + 8lg + 0..7) ----
    bool qv[2];
    u32x4_t bqh[2][NKC], bql[2][SPLIT ? NKC : 1];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      qv[t] = qtile[t] < U.n_tiles;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        In8<uint16_t> x;
        x.w = *reinterpret_cast<const u32x4_t*>(q_s + (qtile[t] * 16 + pr) * D + 8 * ((4 * kc + lg) ^ row_swz<D>(pr)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = phi_map<PHI>(x.get(2 * i)), b = phi_map<PHI>(x.get(2 * i + 1));
          if constexpr (SPLIT) {
            uint32_t h, l;
            split_bf16x2(a, b, h, l);
            bqh[t][kc][i] = h;
            bql[t][kc][i] = l;
          } else {
            bqh[t][kc][i] = pack_bf16x2(a, b);
          }
        }
      }
    }
    // den0 = phi(q) . z0 on the matrix cores, from the wave's z0 slot (landed: the wait above).
    // Normaliser operand: rows 4g = hi(z0), 4g + 1 = lo(z0); every lane gets its token's den0,
    // which seeds the in-slice sum on the lg = 0 lanes only (that sum is reduced over lg).
    float dsum[2] = {0.f, 0.f};
    if (p.zt || p.prez) {   // either may be absent (no mixing; one slice per block)
      f32x4_t accz[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        float z8[8];
        {
          f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = a;
          if (p.zt) {
            a = *reinterpret_cast<const f32x4_t*>(z_slot + 32 * kc + 8 * lg);
            b = *reinterpret_cast<const f32x4_t*>(z_slot + 32 * kc + 8 * lg + 4);
          }
          if (p.prez) {
            const f32x4_t c = *reinterpret_cast<const f32x4_t*>(z_slot + 256 + 32 * kc + 8 * lg);
            const f32x4_t d = *reinterpret_cast<const f32x4_t*>(z_slot + 256 + 32 * kc + 8 * lg + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] = fmaf(U.mii, c[e], a[e]);
              b[e] = fmaf(U.mii, d[e], b[e]);
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z8[e] = a[e];
            z8[4 + e] = b[e];
          }
        }
        u32x4_t az = {0u, 0u, 0u, 0u};
        if ((pr & 3) < 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t h, l;
            split_bf16x2(z8[2 * i], z8[2 * i + 1], h, l);
            az[i] = (pr & 3) == 0 ? h : l;
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          accz[t] = mfma_bf16(az, bqh[t][kc], accz[t]);
          if constexpr (SPLIT) accz[t] = mfma_bf16(az, bql[t][kc], accz[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) dsum[t] = lg == 0 ? accz[t][0] + accz[t][1] : 0.f;
    }
    Unit Un = U;
    if (has_next) {
      Un = decode(Ln);
      cs_wait_lgkm0();   // the query rows are in registers before the DMA may overwrite them
      dma_q(Un);
    }

    f32x4_t acc[2][NCT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[t][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int max_qt = qv[1] ? qtile[1] : (qv[0] ? qtile[0] : -1);   // uniform
    const float mii = U.mii;

    // ---- 2. the slice's keys, a phase at a time ----
    const int n_ph = min(NPH, (U.n_tiles + 1) >> 1);   // phases that hold a key pair
    for (int ph = 0; ph < n_ph; ++ph) {
      __syncthreads();   // the previous phase (or unit) is done with the key space (and S0)
      if (S0_LDS && ph == n_ph - 1 && p.st_hi) {
        // S0 = this unit's bf16 stack fragments: LDS chunk u holds stack chunk u ^ (bit 3 of u
        // moved to bit 2), the order of lds_pos (an involution).  Issued at the last phase, so
        // that the loads the phases before it wait for do not queue behind it
        constexpr int NDMA = FRAG / 512;        // 1 KB instructions
        const cs_i32x4_t rs = cs_rsrc_words(p.st_hi + U.row * FRAG, FRAG * 2u);
        for (int i = wave; i < NDMA; i += SS::NW) {
          const int u = i * 64 + lane, g = NCT >= 2 ? (u ^ (((u >> 3) & 1) << 2)) : u;
          cs_dma16(s0_lds + (uint32_t)(i * 1024), (uint32_t)g * 16u, rs);
        }
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int idx = tid + i * NT, rr = idx / NCH, c = idx % NCH;
        const bool ok = U.j_begin + key_of(ph, rr) < U.j_end;
        float kf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[e] = ok ? mii * phi_map<PHI>(ck[i].get(e)) : 0.f;
        store_frag8<SPLIT>(k_hi, k_lo, rr * D + 8 * (c ^ row_swz<D>(rr)), kf);
        st16(v_s + rr * D + 8 * (c ^ v_swz<D>(rr)), cv[i].w);   // bf16 V: exact
      }
      if (ph + 1 < n_ph) issue_kv(U, ph + 1);
      else if (has_next) issue_kv(Un, 0);
      __syncthreads();

      for (int kp = 0; kp < KT / 2; ++kp) {
        const int kt0 = 2 * (kp * NPH + ph);      // key tiles kt0, kt0 + 1 (slice-relative)
        if (kt0 > max_qt || kt0 >= U.n_tiles) break;
        // Query tile t takes part when kt0 <= its index; tile 1 (15 - w) ranks above tile 0, so
        // the cases are: both, tile 1 alone, or (a short slice without tile 1) tile 0 alone.
        auto pair = [&](auto a0c, auto a1c) {
          constexpr bool A0 = decltype(a0c)::value, A1 = decltype(a1c)::value;
          constexpr bool ACT[2] = {A0, A1};
          // scores of both key tiles (a key tile past the slice holds zeros) for the active tiles
          f32x4_t sc[2][2];                       // [key tile][query tile]
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t) sc[h][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            u32x4_t kh[2], kl[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int krow = (2 * kp + h) * 16 + pr;
              const int off = krow * D + 8 * ((4 * kc + lg) ^ row_swz<D>(krow));
              kh[h] = *reinterpret_cast<const u32x4_t*>(k_hi + off);
              if constexpr (SPLIT) kl[h] = *reinterpret_cast<const u32x4_t*>(k_lo + off);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              if (!ACT[t]) continue;   // folded: t is unrolled
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                sc[h][t] = mfma_bf16(kh[h], bqh[t][kc], sc[h][t]);
                if constexpr (SPLIT) {
                  sc[h][t] = mfma_bf16(kl[h], bqh[t][kc], sc[h][t]);
                  sc[h][t] = mfma_bf16(kh[h], bql[t][kc], sc[h][t]);
                }
              }
            }
          }
          // P = masked scores (lane: keys 16kt + 4lg + rr, query 16 qtile[t] + pr), as the
          // 16x16x32 B operand of the pair (keys of tile kt0 in words 0..1, of kt0 + 1 in 2..3)
          u32x4_t bh[2], bl[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (!ACT[t]) continue;   // folded: t is unrolled
            const int q_rel = 16 * qtile[t] + pr;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int k_rel = 16 * (kt0 + h) + 4 * lg;
              float pv[4];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) pv[rr] = k_rel + rr <= q_rel ? sc[h][t][rr] : 0.f;
              uint32_t h0, l0, h1, l1;
              split_bf16x2(pv[0], pv[1], h0, l0);
              split_bf16x2(pv[2], pv[3], h1, l1);
              bh[t][2 * h] = h0;
              bh[t][2 * h + 1] = h1;
              bl[t][2 * h] = l0;
              bl[t][2 * h + 1] = l1;
              dsum[t] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
            }
          }
          // V^T P over the 32 keys: A = V^T rows (permuted channels), two transposed reads
          const MHLA_CS_LDS char* vbase = (const MHLA_CS_LDS char*)(v_s);
          const int r0 = 2 * kp * 16 + 4 * lg + (pr >> 2);   // the row this lane supplies
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const int ch = 4 * (ct >> 1) + (pr & 3);                   // chunk of the 4 channels
            const int hb = 8 * (ct & 1);                               // byte half of the chunk
            const u32x4_t va = cs_tr_pair(vbase + (r0 * D + 8 * (ch ^ v_swz<D>(r0))) * 2 + hb,
                                          vbase + ((r0 + 16) * D + 8 * (ch ^ v_swz<D>(r0 + 16))) * 2 + hb);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              if (!ACT[t]) continue;   // folded: t is unrolled
              acc[t][ct] = mfma_bf16(va, bh[t], acc[t][ct]);
              acc[t][ct] = mfma_bf16(va, bl[t], acc[t][ct]);
            }
          }
        };
        const bool a0 = qv[0] && kt0 <= qtile[0], a1 = qv[1] && kt0 <= qtile[1];   // uniform
        if (a0 && a1) pair(std::true_type{}, std::true_type{});
        else if (a1) pair(std::false_type{}, std::true_type{});
        else pair(std::true_type{}, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- 3. readout against S0, A operands from the fragment-layout summaries in global memory ----
    if constexpr (S0_LDS) {
      // the S0 DMA was issued before the last issue_kv (2 RPT loads), which alone may be newer
      if (has_next) cs_wait_vm<2 * RPT>();
      else cs_wait_vm0();
    }
    __syncthreads();   // every wave's part of S0; no wave reads K or V of this unit any more
    dma_z(Un);         // (with no next unit Un is U: a harmless reload)
    if (max_qt >= 0) {
      const uint16_t* sh = p.st_hi ? p.st_hi + U.row * FRAG : nullptr;
      const uint16_t* sl = p.st_lo ? p.st_lo + U.row * FRAG : nullptr;
      const float* sp = p.pre ? p.pre + (U.row * p.splits + U.split) * FRAG : nullptr;
      const int b3 = (pr >> 2) & 1;
      const AOffsets ao = a_offsets(lane);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          // A row pr of tile ct: channel 32(ct/2) + 8(pr/4) + 4(ct%2) + pr%4, i.e. fragment
          // (kc, ct & ~1 | pr/8), lane 16lg + 8((pr/4)%2) + 4(ct%2) + pr%4
          const int off = ((kc * NCT + (ct & ~1) + (pr >> 3)) * 64 + 16 * lg + 8 * b3 + 4 * (ct & 1) + (pr & 3)) * 8;
          u32x4_t h;
          if constexpr (S0_LDS) {
            h = sh ? *reinterpret_cast<const u32x4_t*>(s0_s + (kc * NCT + (ct & ~1)) * 512 + ((ct & 1) ? ao.odd : ao.even))
                   : u32x4_t{0u, 0u, 0u, 0u};
          } else {
            h = sh ? ld16(sh + off) : u32x4_t{0u, 0u, 0u, 0u};
          }
          if constexpr (S0_PLAIN) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              acc[t][ct] = mfma_bf16(h, bqh[t][kc], acc[t][ct]);
              if constexpr (SPLIT) acc[t][ct] = mfma_bf16(h, bql[t][kc], acc[t][ct]);
            }
          } else {
            const u32x4_t l = sl ? ld16(sl + off) : u32x4_t{0u, 0u, 0u, 0u};
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t hw = h[e >> 1], lw = l[e >> 1];
              x[e] = ((e & 1) ? bf16hi_to_f32(hw) : bf16lo_to_f32(hw)) + ((e & 1) ? bf16hi_to_f32(lw) : bf16lo_to_f32(lw));
            }
            if (sp) {
              const u32x4_t w0 = ld16(sp + off), w1 = ld16(sp + off + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[e] = fmaf(mii, __uint_as_float(w0[e]), x[e]);
                x[4 + e] = fmaf(mii, __uint_as_float(w1[e]), x[4 + e]);
              }
            }
            u32x4_t ah, al;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t hh, ll;
              split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
              ah[i] = hh;
              al[i] = ll;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              acc[t][ct] = mfma_bf16(ah, bqh[t][kc], acc[t][ct]);
              if constexpr (SPLIT) {
                acc[t][ct] = mfma_bf16(al, bqh[t][kc], acc[t][ct]);
                acc[t][ct] = mfma_bf16(ah, bql[t][kc], acc[t][ct]);
              }
            }
          }
          if (ct & 1) __builtin_amdgcn_sched_barrier(0);   // two tiles' loads in flight at a time
        }
      }
    }


    // ---- 4. o = num / den: a fixed number of buffer stores per wave (idle lanes and tiles out of
    //      range, dropped), so that the next unit's wait can leave them outstanding ----
    const Rsrc ro = make_rsrc(reinterpret_cast<TOut*>(p.o) + U.head_off, (uint32_t)geo.N * D * (uint32_t)sizeof(TOut));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float ds = dsum[t];
      ds += __shfl_xor(ds, 16);
      ds += __shfl_xor(ds, 32);
      const int32_t j = 16 * qtile[t] + pr;
      const bool ok = qv[t] && U.j_begin + j < U.j_end;
      const float scale = p.normalized ? 1.0f / ds : 1.0f;   // ds includes den0
      const uint32_t rel = ok ? tok(U, j) : 0u;
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        float o[8];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          o[rr] = acc[t][2 * c][rr] * scale;
          o[4 + rr] = acc[t][2 * c + 1][rr] * scale;
        }
        const uint32_t off = ok ? (rel + 32 * c + 8 * lg) * (uint32_t)sizeof(TOut) : kOutOfRange;
        if constexpr (sizeof(TOut) == 4) {
          buf_st16(ro, off, u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])});
          buf_st16(ro, ok ? off + 16u : kOutOfRange,
                   u32x4_t{__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])});
        } else {
          buf_st16(ro, off, u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                    pack_bf16x2(o[6], o[7])});
        }
      }
    }
    if (!has_next) break;
    L = Ln;
    U = Un;
  }
  cs_wait_vm0();   // nothing may still be writing LDS when the workgroup ends
}

template <int PHI, typename TOut, int D>
static hipError_t launch_slice_t(const CausalParams& p, int n_units, hipStream_t s) {
  const bool plain = p.st_lo == nullptr && p.pre == nullptr;
  auto kern = p.split ? (plain ? causal_slice_kernel<TOut, D, PHI, true, true> : causal_slice_kernel<TOut, D, PHI, false, true>)
                      : (plain ? causal_slice_kernel<TOut, D, PHI, true, false> : causal_slice_kernel<TOut, D, PHI, false, false>);
  const size_t lds = SliceShape<D>::LDS;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // persistent grid: the workgroups one pass of the chip holds, a multiple of 8 so that a
  // workgroup stays on its XCD's units (unit L and workgroup L % grid share L & 7)
  int grid = 256 * SliceShape<D>::PER_CU;
  if (n_units < grid) grid = n_units;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(SliceShape<D>::NT), lds, s, p, n_units);
  return hipGetLastError();
}

// bf16 inputs, head sizes 32, 64, 128, token slices of at most 256 tokens of a 1D sequence;
// n_units = splits * M * BH.
hipError_t launch_causal_slice(const CausalParams& p, int d, bool out_fp32, int phi, int n_units, hipStream_t stream) {
  if (p.tok_per_split > 256 || n_units < 1) return hipErrorInvalidValue;
  auto go = [&](auto phi_c) -> hipError_t {
    constexpr int PHI = decltype(phi_c)::value;
    auto by_d = [&](auto tout) -> hipError_t {
      using TO = decltype(tout);
      switch (d) {
        case 32: return launch_slice_t<PHI, TO, 32>(p, n_units, stream);
        case 64: return launch_slice_t<PHI, TO, 64>(p, n_units, stream);
        case 128: return launch_slice_t<PHI, TO, 128>(p, n_units, stream);
        default: return hipErrorInvalidValue;
      }
    };
    return out_fp32 ? by_d(float{}) : by_d(uint16_t{});
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhla
