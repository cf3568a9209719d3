// Summary kernel for bf16 inputs, streamed through LDS: S_b = sum_j phi(K_j) V_j^T on bf16 MFMA with
// fp32 accumulation, z_b = sum_j phi(K_j), and for the MALA readout u = sum_j V_j.
//
// Source: "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method ->
// Overall framework (local KV summary S_b and normaliser z_b of every block); the MALA linear form
// in "Rectifying Magnitude Neglect in Linear Attention", Method -> Key design, also needs sum_j V_j.
//
// Same work units, outputs and fragment layout as summary.hip; what differs is how tokens reach the
// MFMAs.  Each workgroup (4 wave64s, one per CU) keeps a ring of NS stages in LDS; a stage holds T
// tokens of K and of V row-major (16 KB each).  The tiles arrive by 16-byte buffer loads that write
// LDS directly (lane L of an instruction fills bytes 16 L .. 16 L + 15 of a 1 KB block), NS - 1
// stages ahead of the one being computed, so no register holds data in flight and the memory
// stream does not stop while a stage is transposed or multiplied.  The MFMA operands are read from
// the row-major tiles with the 16-bit transposing LDS read: in each group of 16 lanes, lane l names
// row l/4 and columns 4 (l%4) .. +3 of a 4 x 16 tile, and afterwards lane j holds column j; two
// such reads give a lane the 8 consecutive tokens of one feature (A = phi(K)^T, rows permuted as in
// summary.hip so that the output is in fragment layout) or of one channel (B = V).  phi is applied
// to the A operand in registers (hi + lo when phi(K) is split, at no extra LDS cost).  Rows are
// stored with their 16-byte chunks XOR-swizzled by the token (sigma below), so that the 16 lanes of
// a transposing read touch 16 different bank pairs.
//
// The backward's token-weighted summary (TOKW: K := Q scaled per token by kscale, normaliser product
// weighted by zw, V := dO) takes the same ring: each slot also receives the stage's kscale and zw
// through 4-byte direct-to-LDS loads (lane L of wave w: stage token 64 (w % NTW) + L, gathered by
// its token index, so any block geometry works); the lanes scale phi(Q) before the hi / lo split
// and feed zw (hi + lo) as the normaliser's B operand.
//
// Work split: wave w takes the 32-feature chunk kc = w % NKC and, when NKC < 4, every WK-th 32-token
// step of a stage (WK = 4 / NKC waves share a chunk); their partial sums are added through LDS at
// the end of a unit.  The loads are written in inline assembly (the compiler cannot tell which LDS
// bytes a direct-to-LDS load writes and would wait for all of them before every LDS read); they
// have no output registers, and each wave waits for its own loads with an explicit count.
#include <type_traits>

#include "mhla_device.hpp"

namespace mhla {

namespace {

// Ring shape per head size: stages of SB bytes (K + V), NS of them, sized so that two workgroups
// fit on a CU (two waves per SIMD: one wave's VALU work overlaps the other's MFMAs and LDS reads).
#ifndef MHLA_DMA_STAGE_BYTES
#define MHLA_DMA_STAGE_BYTES 16384
#endif
// TOKW (the backward's token-weighted summary): each slot also holds the stage's per-token weights,
// kscale and zw as fp32 (one 4-byte load per lane, NTW loads of 64 tokens per array); at d = 128 a
// ring of 4 such slots keeps two workgroups per CU.
template <int D, bool TOKW = false> struct DmaRing {
  static constexpr int SB = MHLA_DMA_STAGE_BYTES;
  static constexpr int NS = D == 128 ? (TOKW ? 4 : 5) : 3;   // 80 KB at d = 128; d < 128 also holds a reduction area
  static constexpr int T = SB / (4 * D);                     // tokens per stage
  static constexpr int NTW = TOKW ? (T + 63) / 64 : 0;
  static constexpr int WB = NTW * 256;                       // bytes of one weight array per slot
  static constexpr int SLOT = SB + 2 * WB;
};

// vmcnt(n) alone (expcnt and lgkmcnt at their maxima): the gfx9 s_waitcnt encoding.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt for `ahead` newer loads and n epilogues of `nst` stores, capped at the counter's range (a
// lower count only waits longer).
constexpr int vm_count(int ahead, int nst, int n) { return ahead + n * nst < 63 ? ahead + n * nst : 63; }

// A buffer resource as four scalar words (for the inline assembly): base, range in bytes, the
// gfx9-family untyped-buffer configuration word (as make_rsrc).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ inline i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int32_t)(uint32_t)a, (int32_t)(uint32_t)((a >> 32) & 0xffffu), (int32_t)bytes, 0x00020000};
}

// One 4-byte load per lane into LDS at lds_byte + 4 * lane (lds_byte wave-uniform; out of range:
// the lane writes zero), default cache policy.
__device__ inline void dma4(uint32_t lds_byte, uint32_t voff, i32x4_t rs) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(rs) : "memory");
}

// One 16-byte load per lane into LDS at lds_byte + 16 * lane (lds_byte is wave-uniform); voff is the
// lane's byte offset into the resource (out of range: the lane writes zeros).  Non-temporal: K and V
// are streamed once.
__device__ inline void dma16(uint32_t lds_byte, uint32_t voff, i32x4_t rs) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(m0), "v"(voff), "s"(rs)
               : "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define MHLA_LDS __attribute__((address_space(3)))

// Two transposing reads (rows t0 .. t0 + 3 and t0 + 4 .. t0 + 7 of the lane group's tile) packed as
// one 8 x bf16 MFMA operand.
__device__ inline u32x4_t tr_pair(const MHLA_LDS char* p0, const MHLA_LDS char* p1) {
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MHLA_LDS s16x4_t*)p0);
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MHLA_LDS s16x4_t*)p1);
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

// Chunk swizzle of token row t (stage-relative): chunk c of the row lives at c ^ sigma(t).
template <int D>
__device__ inline int sigma(int t) {
  if constexpr (D == 128) return (t & 3) << 2;
  else if constexpr (D == 64) return ((t >> 1) & 1) << 2;
  else return 0;
}

}  // namespace

template <int D, bool SPLIT_K, bool WANT_U, bool OUT_BF16, int PHI, bool TOKW = false>
__global__ __launch_bounds__(kThreads) void summary_dma_kernel(SummaryParams p, int n_units) {
  using Dm = Dims<D>;
  using Ring = DmaRing<D, TOKW>;
  static_assert(D >= 32, "d = 16 runs on summary_kernel");
  static_assert(!TOKW || (SPLIT_K && !WANT_U && !OUT_BF16), "token weights: split phi(K), fp32 partials");
  constexpr int kStages = Ring::NS, kStageBytes = Ring::SB, kSlotBytes = Ring::SLOT;
  constexpr int NKC = Dm::NKC, NCT = Dm::NCT, FRAG = Dm::FRAG;
  constexpr int T = kStageBytes / (4 * D);          // tokens per stage
  constexpr int KS = T / 32;                        // 32-token MFMA steps per stage
  constexpr int WK = 4 / NKC;                       // waves sharing a feature chunk
  constexpr int KSW = KS / WK;                      // steps per wave and stage
  constexpr int ROWB = 2 * D;                       // bytes of one token row
  constexpr int LPR = D / 8;                        // 16-byte chunks (lanes) per row
  constexpr int DMA_PER = (kStageBytes / 2) / (kThreads * 16);   // loads per thread and tensor
  constexpr int LPS = 2 * DMA_PER + (TOKW ? 2 : 0);              // loads per thread and stage
  constexpr int VM_AHEAD = LPS * (kStages - 2);                  // loads issued after a stage's
  constexpr int NST = NCT * (OUT_BF16 ? 1 : 2) + 2 + (WANT_U ? NCT : 0);   // stores per epilogue
  constexpr uint32_t kOnes = 0x3f803f80u;
  static_assert(KSW >= 1 && KSW * WK == KS, "steps split evenly over the waves of a chunk");

  extern __shared__ __align__(16) char smem[];
  // ring: kStages x [K (SB / 2) | V (SB / 2) | TOKW: kscale (WB) | zw (WB)]; then the reduction
  // area for WK > 1
  float* red = reinterpret_cast<float*>(smem + kStages * kSlotBytes);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(MHLA_LDS char*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int kc = wave % NKC, kh = wave / NKC;
  const int g = lane >> 4, lam = lane & 15;
  const Geom& geo = p.g;

  // ---- side job: bf16 operand fragments of M_c for the MFMA mixing kernel (as summary.hip) ----
  if (p.mcf) {
    const int nitp = p.mcf_nitp, nbc = p.mcf_nbc, M = geo.M;
    const int total = p.mcf_heads * nitp * nbc * 64;
    for (int idx = blockIdx.x * kThreads + tid; idx < total; idx += gridDim.x * kThreads) {
      const int l = idx & 63;
      int t = idx >> 6;
      const int bc = t % nbc;
      t /= nbc;
      const int it = t % nitp, hh = t / nitp;
      const int i = 16 * it + (l & 15);
      const float* mch = p.mc ? p.mc + (int64_t)hh * p.mc_head_stride : nullptr;
      const int64_t si = p.mcf_transposed ? 1 : M, sb = p.mcf_transposed ? M : 1;
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int b = 32 * bc + 8 * (l >> 4) + e;
        m[e] = (i < M && b < M && !(p.mcf_causal && b >= i)) ? (mch ? mch[i * si + b * sb] : 1.0f) : 0.f;
      }
      u32x4_t hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h, l2;
        split_bf16x2(m[2 * j], m[2 * j + 1], h, l2);
        hi[j] = h;
        lo[j] = l2;
      }
      st16(p.mcf + (int64_t)idx * 8, hi);
      if (p.mcf_lo) st16(p.mcf_lo + (int64_t)idx * 8, lo);
    }
  }

  // ---- units and stages ----------------------------------------------------------------------
  struct Unit {
    int bh, blk, split;
    int32_t j_begin, j_end, base_tok;
    int64_t head_off;
    BlockGeo bg;
  };
  auto make_unit = [&](int u) {
    Unit U;
    U.split = u % p.splits;
    const int t = u / p.splits;
    U.blk = t % geo.M;
    U.bh = t / geo.M;
    U.j_begin = U.split * p.tok_per_split;
    U.bg = block_geo(geo, U.blk);
    U.j_end = min(U.j_begin + p.tok_per_split, U.bg.n);
    U.base_tok = U.bg.base;
    U.head_off = (int64_t)U.bh * geo.N * D;
    return U;
  };
  // A cursor over the workgroup's (unit, stage) sequence; past the last unit it yields empty stages.
  struct Cursor {
    int unit;
    int32_t sb;     // first block-local token of the stage
    Unit U;
  };
  auto cursor_start = [&](Cursor& c) {
    c.unit = blockIdx.x;
    if (c.unit < n_units) {
      c.U = make_unit(c.unit);
      c.sb = c.U.j_begin;
    }
  };
  auto cursor_next = [&](Cursor& c) {
    if (c.unit >= n_units) return;
    if (c.sb + T < c.U.j_end) {
      c.sb += T;
    } else {
      c.unit += gridDim.x;
      if (c.unit < n_units) {
        c.U = make_unit(c.unit);
        c.sb = c.U.j_begin;
      }
    }
  };

  // Issue the loads of the cursor's stage into ring slot `slot`: DMA_PER 1 KB blocks of K and of V
  // per wave; lane L of block b holds row t = (1024 b + 16 L) / ROWB, chunk position
  // (16 L % ROWB) / 16, fetched from chunk position ^ sigma(t) of token t's row.
  constexpr uint32_t kES = 2;
  auto issue = [&](const Cursor& c, int slot) {
    const bool live = c.unit < n_units;
    const uint32_t hb = (uint32_t)geo.N * D * kES;
    const i32x4_t rk = rsrc_words(live ? reinterpret_cast<const uint16_t*>(p.k) + c.U.head_off : p.k, live ? hb : 0u);
    const i32x4_t rv = rsrc_words(live ? reinterpret_cast<const uint16_t*>(p.v) + c.U.head_off : p.v, live ? hb : 0u);
    const uint32_t slot_lds = ring_lds + (uint32_t)(slot * kSlotBytes);
#pragma unroll
    for (int i = 0; i < DMA_PER; ++i) {
      const int blk = i * 4 + wave;
      const int byte = blk * 1024 + lane * 16;
      const int t = byte / ROWB, pos = (byte % ROWB) / 16;
      const int ch = pos ^ sigma<D>(t);
      uint32_t off = kOutOfRange;
      if (live) {
        const int32_t j = c.sb + t;
        if (j < c.U.j_end)
          off = ((uint32_t)(c.U.base_tok + block_offset(geo, c.U.bg, (uint32_t)j)) * D + 8u * ch) * kES;
      }
      dma16(slot_lds + (uint32_t)(blk * 1024), off, rk);
      dma16(slot_lds + (uint32_t)(kStageBytes / 2 + blk * 1024), off, rv);
    }
    if constexpr (TOKW) {
      // stage token tau = 64 (wave % NTW) + lane: waves w and w + NTW load the same tokens into the
      // same bytes (same values), so that every wave issues the same number of loads
      const int part = wave % Ring::NTW, tau = 64 * part + lane;
      uint32_t woff = kOutOfRange;
      if (live && tau < T) {
        const int32_t j = c.sb + tau;
        if (j < c.U.j_end) woff = (uint32_t)(c.U.base_tok + block_offset(geo, c.U.bg, (uint32_t)j)) * 4u;
      }
      const int64_t tb = live ? (int64_t)c.U.bh * geo.N : 0;
      const uint32_t wbytes = live ? (uint32_t)geo.N * 4u : 0u;
      dma4(slot_lds + (uint32_t)(kStageBytes + 256 * part), woff, rsrc_words(p.kscale + tb, wbytes));
      dma4(slot_lds + (uint32_t)(kStageBytes + Ring::WB + 256 * part), woff, rsrc_words(p.zw + tb, wbytes));
    }
  };

  f32x4_t acc[2][NCT], accz[2], accu[NCT];
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      accz[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCT; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) accu[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  reset();

  // MFMAs of one stage (slot), `valid` tokens of which belong to the unit.
  auto compute = [&](int slot, int32_t valid) {
    const MHLA_LDS char* ks_base = (const MHLA_LDS char*)smem + slot * kSlotBytes;
    const MHLA_LDS char* vs_base = ks_base + kStageBytes / 2;
    const MHLA_LDS float* ws_base = (const MHLA_LDS float*)(ks_base + kStageBytes);   // TOKW: kscale
    const MHLA_LDS float* wz_base = ws_base + Ring::WB / 4;                            // TOKW: zw
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
      const int step = s * WK + kh;                   // this wave's 32-token step
      const int t0 = 32 * step + 8 * g + (lam >> 2);  // the lane's row in the first read
      const int t1 = t0 + 4;
      // TOKW: kscale and zw of the lane's 8 tokens 32 step + 8 g + 0..7 (broadcast reads)
      float sc[8], zwv[8];
      if constexpr (TOKW) {
        const int tb = 32 * step + 8 * g;
        const f32x4_t s0 = *(const MHLA_LDS f32x4_t*)(ws_base + tb), s1 = *(const MHLA_LDS f32x4_t*)(ws_base + tb + 4);
        const f32x4_t z0 = *(const MHLA_LDS f32x4_t*)(wz_base + tb), z1 = *(const MHLA_LDS f32x4_t*)(wz_base + tb + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[i] = s0[i];
          sc[4 + i] = s1[i];
          zwv[i] = z0[i];
          zwv[4 + i] = z1[i];
        }
      }
      // A: phi(K)^T rows of tile r = features 32 kc + 8 q + 4 r + 0..3 of lane group quarter q
      u32x4_t a_hi[2], a_lo[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int c = 4 * kc + (lam & 3);
        const u32x4_t raw = tr_pair(ks_base + t0 * ROWB + 16 * (c ^ sigma<D>(t0)) + 8 * r,
                                    ks_base + t1 * ROWB + 16 * (c ^ sigma<D>(t1)) + 8 * r);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x0 = phi_map<PHI>(bf16lo_to_f32(raw[i])), x1 = phi_map<PHI>(bf16hi_to_f32(raw[i]));
          if constexpr (TOKW) {
            x0 *= sc[2 * i];
            x1 *= sc[2 * i + 1];
          }
          if constexpr (SPLIT_K) {
            uint32_t h, l;
            split_bf16x2(x0, x1, h, l);
            a_hi[r][i] = h;
            a_lo[r][i] = l;
          } else {
            a_hi[r][i] = pack_bf16x2(x0, x1);
          }
        }
      }
      // validity of the 8 tokens 32 step + 8 g + 0..7: the B operand of the normaliser product
      // (rows past the unit's end hold phi(0) != 0 or stale bytes); in a partial stage the A and B
      // operands of those tokens are also cleared, so that nothing left in the ring can enter a sum
      u32x4_t vmask = {kOnes, kOnes, kOnes, kOnes};
      u32x4_t tmask = {~0u, ~0u, ~0u, ~0u};
      const bool partial = valid < T;         // uniform: the whole workgroup's stage
      if (partial) {
        const int left = valid - (32 * step + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vmask[i] = (2 * i < left ? 0x3f80u : 0u) | (2 * i + 1 < left ? 0x3f800000u : 0u);
          tmask[i] = (2 * i < left ? 0xffffu : 0u) | (2 * i + 1 < left ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          a_hi[r] &= tmask;
          if constexpr (SPLIT_K) a_lo[r] &= tmask;
        }
      }
      // TOKW: the normaliser product weights token t by zw_t, split hi (vmask) + lo (wlo)
      u32x4_t wlo = {0u, 0u, 0u, 0u};
      if constexpr (TOKW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t h, l;
          split_bf16x2(zwv[2 * i], zwv[2 * i + 1], h, l);
          vmask[i] = h;
          wlo[i] = l;
        }
        vmask &= tmask;
        wlo &= tmask;
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        accz[r] = mfma_bf16(a_hi[r], vmask, accz[r]);
        if constexpr (SPLIT_K) accz[r] = mfma_bf16(a_lo[r], vmask, accz[r]);
        if constexpr (TOKW) accz[r] = mfma_bf16(a_hi[r], wlo, accz[r]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        // B: V rows, channels 16 ct + 4 q' .. +3 of lane group quarter q' (two chunks per tile)
        const int c = 2 * ct + ((lam & 3) >> 1);
        const int bsub = 8 * (lam & 1);
        u32x4_t b = tr_pair(vs_base + t0 * ROWB + 16 * (c ^ sigma<D>(t0)) + bsub,
                            vs_base + t1 * ROWB + 16 * (c ^ sigma<D>(t1)) + bsub);
        if (partial) b &= tmask;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          acc[r][ct] = mfma_bf16(a_hi[r], b, acc[r][ct]);
          if constexpr (SPLIT_K) acc[r][ct] = mfma_bf16(a_lo[r], b, acc[r][ct]);
        }
        if constexpr (WANT_U) {
          if (kc == 0) accu[ct] = mfma_bf16(u32x4_t{kOnes, kOnes, kOnes, kOnes}, b, accu[ct]);
        }
      }
    }
  };

  // End of a unit: sum the WK partial results of each chunk (through LDS), then the chunk's
  // first wave writes the summary in fragment layout, z and u.
  constexpr int RED_ACC = 2 * NCT * 64 * 4;   // floats of one wave's acc
  auto epilogue = [&](const Unit& U) {
    if constexpr (WK > 1) {
      if (kh > 0) {
        float* dst = red + (size_t)(kh - 1) * NKC * (RED_ACC + 2 * 64 * 4 + NCT * 64 * 4) +
                     (size_t)kc * (RED_ACC + 2 * 64 * 4 + NCT * 64 * 4);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            *reinterpret_cast<f32x4_t*>(dst + ((r * NCT + c) * 64 + lane) * 4) = acc[r][c];
#pragma unroll
        for (int r = 0; r < 2; ++r) *reinterpret_cast<f32x4_t*>(dst + RED_ACC + (r * 64 + lane) * 4) = accz[r];
        if constexpr (WANT_U) {
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            *reinterpret_cast<f32x4_t*>(dst + RED_ACC + 2 * 64 * 4 + (c * 64 + lane) * 4) = accu[c];
        }
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int k2 = 1; k2 < WK; ++k2) {
          const float* src = red + (size_t)(k2 - 1) * NKC * (RED_ACC + 2 * 64 * 4 + NCT * 64 * 4) +
                             (size_t)kc * (RED_ACC + 2 * 64 * 4 + NCT * 64 * 4);
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              acc[r][c] += *reinterpret_cast<const f32x4_t*>(src + ((r * NCT + c) * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < 2; ++r) accz[r] += *reinterpret_cast<const f32x4_t*>(src + RED_ACC + (r * 64 + lane) * 4);
          if constexpr (WANT_U) {
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              accu[c] += *reinterpret_cast<const f32x4_t*>(src + RED_ACC + 2 * 64 * 4 + (c * 64 + lane) * 4);
          }
        }
      }
    }
    // Outputs through buffer resources, every wave issuing the same NST stores (a wave or lane
    // with nothing to write gets an out-of-range offset, which drops the store): the main loop's
    // wait counts them exactly.
    const int64_t slot = ((int64_t)U.bh * geo.M + U.blk) * p.splits + U.split;
    const bool writer = kh == 0;
    const Rsrc rs_s = OUT_BF16 ? make_rsrc(p.sb + slot * FRAG, FRAG * 2u) : make_rsrc(p.ps + slot * FRAG, FRAG * 4u);
    const Rsrc rs_z = make_rsrc(p.pz + slot * D, D * 4u);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const uint32_t off = writer ? (uint32_t)(((kc * NCT + c) * 64 + lane) * 8) : kOutOfRange;
      const f32x4_t r0 = acc[0][c], r1 = acc[1][c];
      if constexpr (OUT_BF16) {
        buf_st16(rs_s, writer ? off * 2u : kOutOfRange,
                 u32x4_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]), pack_bf16x2(r1[0], r1[1]),
                         pack_bf16x2(r1[2], r1[3])});
      } else {
        buf_st16(rs_s, writer ? off * 4u : kOutOfRange, __builtin_bit_cast(u32x4_t, r0));
        buf_st16(rs_s, writer ? off * 4u + 16u : kOutOfRange, __builtin_bit_cast(u32x4_t, r1));
      }
    }
    // z: row 4 g + j of tile r is feature 32 kc + 8 g + 4 r + j; every column holds it
#pragma unroll
    for (int r = 0; r < 2; ++r)
      buf_st16(rs_z, (writer && lam == 0) ? (uint32_t)(32 * kc + 8 * g + 4 * r) * 4u : kOutOfRange,
               __builtin_bit_cast(u32x4_t, accz[r]));
    if constexpr (WANT_U) {
      const Rsrc rs_u = make_rsrc(p.pu + slot * D, D * 4u);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
        buf_st4(rs_u, (writer && kc == 0 && g == 0) ? (uint32_t)(16 * c + lam) * 4u : kOutOfRange,
                __float_as_uint(accu[c][0]));
    }
    reset();
  };

  if ((int)blockIdx.x >= n_units) return;
  Cursor cc, ic;          // compute cursor, issue cursor (kStages - 1 stages ahead)
  cursor_start(cc);
  cursor_start(ic);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) {
    issue(ic, s);
    cursor_next(ic);
  }
  // epi: bit i set when the epilogue ran i + 1 iterations ago.  The loads of stage s were issued
  // kStages - 1 iterations before its compute (or in the prologue); newer than them are the loads
  // of the kStages - 2 stages after it (VM_AHEAD) and NST stores per epilogue of the last
  // kStages - 1 iterations.  Loads and stores retire in issue order, so waiting until no more than
  // that many are outstanding means stage s has landed.
  uint32_t epi = 0;
  for (int s = 0;; ++s) {
    switch (__builtin_popcount(epi & ((1u << (kStages - 1)) - 1u))) {
      case 0: wait_vm<VM_AHEAD>(); break;
      case 1: wait_vm<vm_count(VM_AHEAD, NST, 1)>(); break;
      case 2: wait_vm<vm_count(VM_AHEAD, NST, 2)>(); break;
      case 3: wait_vm<vm_count(VM_AHEAD, NST, 3)>(); break;
      default: wait_vm<vm_count(VM_AHEAD, NST, 4)>(); break;
    }
    __syncthreads();                          // every wave's loads of stage s, and every wave is
                                              // done with the slot the next issue overwrites
    issue(ic, (s + kStages - 1) % kStages);
    cursor_next(ic);
    const Unit U = cc.U;
    const int32_t valid = min(T, U.j_end - cc.sb);
    compute(s % kStages, valid);
    const bool unit_end = cc.sb + T >= U.j_end;
    if (unit_end) epilogue(U);
    epi = (epi << 1) | (unit_end ? 1u : 0u);
    cursor_next(cc);
    if (cc.unit >= n_units) break;
  }
  wait_vm<0>();           // no load of an empty stage may still be writing LDS at the exit
}

template <int PHI, int D, bool SPLIT_K, bool WANT_U, bool OUT_BF16, bool TOKW = false>
static hipError_t launch_dma_t(const SummaryParams& p, int n_units, hipStream_t stream) {
  constexpr int NKC = D / 32, NCT = D / 16, WK = 4 / NKC;
  constexpr size_t red_floats = WK > 1 ? (size_t)(WK - 1) * NKC * (2 * NCT * 64 * 4 + 2 * 64 * 4 + NCT * 64 * 4) : 0;
  const size_t lds = (size_t)DmaRing<D, TOKW>::NS * DmaRing<D, TOKW>::SLOT + red_floats * 4;
  auto kern = summary_dma_kernel<D, SPLIT_K, WANT_U, OUT_BF16, PHI, TOKW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int per_cu = (int)(160 * 1024 / lds) < 1 ? 1 : ((int)(160 * 1024 / lds) > 2 ? 2 : (int)(160 * 1024 / lds));
  int grid = 256 * per_cu;             // persistent: as many workgroups as fit at once (LDS), at most 2 per CU
  if (grid > n_units) grid = n_units;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, p, n_units);
  return hipGetLastError();
}

template <int PHI, int D>
static hipError_t dma_flags(const SummaryParams& p, bool split_k, bool want_u, bool out_bf16, int n,
                            hipStream_t s) {
  if (out_bf16) {
    if (split_k || want_u) return hipErrorInvalidValue;
    return launch_dma_t<PHI, D, false, false, true>(p, n, s);
  }
  if (split_k)
    return want_u ? launch_dma_t<PHI, D, true, true, false>(p, n, s) : launch_dma_t<PHI, D, true, false, false>(p, n, s);
  return want_u ? launch_dma_t<PHI, D, false, true, false>(p, n, s) : launch_dma_t<PHI, D, false, false, false>(p, n, s);
}

// bf16 inputs, d in {32, 64, 128}: the LDS-streamed summary (n_units as launch_summary).
hipError_t launch_summary_dma(const SummaryParams& p, int d, bool split_k, bool want_u, bool out_bf16, int phi,
                              int n_units, hipStream_t stream) {
  auto go = [&](auto phi_c) -> hipError_t {
    constexpr int PHI = decltype(phi_c)::value;
    switch (d) {
      case 32: return dma_flags<PHI, 32>(p, split_k, want_u, out_bf16, n_units, stream);
      case 64: return dma_flags<PHI, 64>(p, split_k, want_u, out_bf16, n_units, stream);
      case 128: return dma_flags<PHI, 128>(p, split_k, want_u, out_bf16, n_units, stream);
      default: return hipErrorInvalidValue;
    }
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

// The backward's token-weighted summary (K := Q scaled by kscale, normaliser weights zw, V := dO)
// for bf16 Q and dO, d in {32, 64, 128}: split phi(K), fp32 partials.
hipError_t launch_summary_dma_tokw(const SummaryParams& p, int d, int phi, int n_units, hipStream_t stream) {
  if (!p.kscale || !p.zw) return hipErrorInvalidValue;
  auto go = [&](auto phi_c) -> hipError_t {
    constexpr int PHI = decltype(phi_c)::value;
    switch (d) {
      case 32: return launch_dma_t<PHI, 32, true, false, false, true>(p, n_units, stream);
      case 64: return launch_dma_t<PHI, 64, true, false, false, true>(p, n_units, stream);
      case 128: return launch_dma_t<PHI, 128, true, false, false, true>(p, n_units, stream);
      default: return hipErrorInvalidValue;
    }
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhla
