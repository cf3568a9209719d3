// MFMA mixing kernel: S~_i = sum_b m_ib S_b over a stack of summaries, and the fp32 normaliser
// mixing z~_i = sum_b m_ib z_b ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head", Method -> Key design 2: the mixing is one product of M_c with the stack of
// summaries; row i of M_c belongs to query block i).  The backward runs the same product with
// M_c^T (dS_b = sum_i m_ib dS~_i, the chain rule of this step).
//
// Per (batch, head) the summaries form X[M][P] (P = fragment positions of a d x d summary) and
// the kernel computes Y = W X (W = M_c or M_c^T) as Y^T = X^T W^T on v_mfma_f32_16x16x32_bf16:
//   A = X^T   16 positions x 32 blocks, read from an LDS tile that holds X transposed
//             (blocks contiguous; filled with 16-byte global loads and an 8x8 register
//             transpose, like the summary kernel);
//   B = W^T   32 blocks x 16 query blocks, bf16 operand fragments prepared by the summary
//             kernel, held in registers for the workgroup's lifetime;
//   D         16 positions x 16 query blocks.
// The columns are taken 32 at a time as two MFMA tiles pt = 0, 1 whose 16 A rows are the
// positions 8*(m/4) + 4*pt + m%4, m = 0..15.  Over the two tiles lane (g, l) then holds the 8
// consecutive positions 8g .. 8g+7 of row i = 16*it + l: one 16-byte store, and the four lane
// groups of a row write 64 contiguous bytes.
// The contraction over blocks is padded to a multiple of 32 with zero rows.  The normaliser
// rides along as extra column tiles: z_b enters as interleaved bf16 (hi, lo) column pairs
// (z = hi + lo to about 2^-17) and leaves as fp32 z~ = Y[hi col] + Y[lo col].
//
// Two precisions:
//   SPLIT = false  bf16 stack (one token slice per block): the bf16 forward.  With WLO, W enters
//                  as bf16 hi + lo (two MFMAs per product, W to about 2^-17): rounding M_c to one
//                  bf16 would perturb every mixing weight by up to 2^-8 relative, and since S~_i
//                  averages many summaries of both signs, that error does not average away
//                  (it is the largest rounding of the bf16 path);
//   SPLIT = true   fp32 partial summaries, summed over their token slices as they are loaded,
//                  and W, both as bf16 hi + lo; three MFMAs per product (hi*hi + lo*hi + hi*lo,
//                  about 2^-16 relative) and Y leaves as bf16 hi and lo.  One i-tile per wave
//                  keeps the doubled W fragments in registers.
#include "mhla_device.hpp"

namespace mhla {

// Columns (fragment positions) of a staged tile: 16384 / MPAD, so a tile holds 16384 bf16 values.
// The bf16 kernel with 4 waves and at most 64 blocks stages half as many, so that each workgroup
// walks two tiles or more and the next tile's loads overlap the current one's MFMAs (the
// mixing of video3d's 64 blocks: 14.2 -> 12.2 us).
__host__ __device__ constexpr int mix_tile_cols(int nbc, bool split, int nw) {
  return ((!split && nw == 4 && nbc <= 2) ? 8192 : 16384) / (32 * nbc);
}

// NBC: 32-block chunks of the contraction (M <= 32*NBC); ITW: 16-row i-tiles per wave; NW:
// waves per workgroup.  With NW = 8 (the split kernel and the bf16 kernel with WLO at M > 128),
// and with the half-size tiles, a loader thread takes 8 rows x 4 columns of the tile instead of
// 8 x 8, so that the tile's registers halve (and the loader threads still cover its rows once).
template <int NBC, int ITW, bool SPLIT, int NW = 4, bool WLO = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void mix_mfma_kernel(
    MixMfmaParams p) {
  constexpr int MPAD = 32 * NBC;
  constexpr int PB = mix_tile_cols(NBC, SPLIT, NW);   // columns (fragment positions) per staged tile
  constexpr int NCG = PB / 32;            // 32-column groups per staged tile
  constexpr int XP = MPAD;                // LDS pitch (elements) of one transposed column
  constexpr int LC = (NW == 8 || PB * MPAD < 16384) ? 4 : 8;   // tile columns per loader thread
  constexpr int CG = PB / LC;             // column groups per tile
  static_assert(NW * 64 / CG * 8 == MPAD, "the loader threads cover the padded blocks once");
  static_assert(NW == 4 || SPLIT || WLO, "8 waves: W as hi + lo only");
  constexpr bool HAS_LO = SPLIT || WLO;   // W fragments as hi + lo
  // LDS bank swizzle on the 16-byte chunks (8 blocks) of a transposed column r: columns are
  // written 8 apart (r = 8*cg + e) and read 8 consecutive (r = 16*pt + pr).  With >= 8 chunks
  // per column, chunk c lives at c ^ ((r & 7) ^ ((r >> 3) & 7)); a 64-byte column (MPAD = 32)
  // has 4 chunks and two columns share each 128-byte bank row, so the low two bits are used.
  auto swz = [](int r, int c) {
    if constexpr (MPAD >= 64) return c ^ ((r & 7) ^ ((r >> 3) & 7));
    else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
  };

  extern __shared__ __align__(16) uint16_t xt[];   // [PB][XP] (hi), then [PB][XP] (lo) if SPLIT
  uint16_t* xt_lo = xt + PB * XP;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int pr = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.z;
  const int M = p.M;
  // ---------------- wave roles -------------------------------------------------------------
  // `wave_rows` waves split the workgroup's i-tiles; the remaining factor splits columns.
  const int WI = p.wave_rows;
  const int WPW = NW / WI;
  const int wi = wave % WI, wp = wave / WI;
  const int it0 = (blockIdx.y * WI + wi) * ITW;     // first i-tile of this wave
  const int nit = (M + 15) >> 4;
  const int nitp = gridDim.y * WI * ITW;

  // W^T operand fragments: lane holds W[16*it + pr][32*bc + 8*lg + e], e = 0..7, one 16-byte
  // load each.
  const int64_t fofs = (int64_t)(p.mcf_per_head ? bh % p.H : 0) * nitp * NBC * 512;
  u32x4_t bfrag[ITW][NBC], bfrag_lo[HAS_LO ? ITW : 1][HAS_LO ? NBC : 1];
#pragma unroll
  for (int a = 0; a < ITW; ++a)
#pragma unroll
    for (int bc = 0; bc < NBC; ++bc) {
      const int64_t o = fofs + (((int64_t)(it0 + a) * NBC + bc) * 64 + lane) * 8;
      bfrag[a][bc] = ld16(p.mcf + o);
      if constexpr (HAS_LO) bfrag_lo[a][bc] = ld16(p.mcf_lo + o);
    }

  const int P = p.frag;
  const int n_tiles = P / PB;
  uint16_t* y = p.y + (int64_t)bh * M * P;
  uint16_t* y_lo = SPLIT ? p.y_lo + (int64_t)bh * M * P : nullptr;

  const int cg = tid % CG, rg = tid / CG;           // loader role: rows 8*rg.., columns LC*cg..
  // raw: bf16 [row][8 columns], or for SPLIT fp32 [row][LC/4][4 columns] summed over token
  // slices
  constexpr int RW = SPLIT ? LC / 4 : 1;            // words of a row
  u32x4_t raw[8 * RW];
  // the stack of this head through a buffer resource: rows b >= M read as zero, no branch
  const Rsrc rsx = SPLIT ? make_rsrc(p.xf + (int64_t)bh * M * p.xsplits * P, (uint32_t)M * p.xsplits * P * 4u)
                         : make_rsrc(p.x + (int64_t)bh * M * P, (uint32_t)M * P * 2u);
  auto issue = [&](int tile) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int b = 8 * rg + r;
        const uint32_t o0 = b < M ? (uint32_t)((b * p.xsplits) * P + tile * PB + LC * cg) * 4u : kOutOfRange;
        // default cache policy: the row groups of a column tile run on one XCD and share it
#pragma unroll
        for (int w = 0; w < RW; ++w) raw[RW * r + w] = buf_ld16(rsx, b < M ? o0 + 16u * w : kOutOfRange);
      }
      for (int s = 1; s < p.xsplits; ++s) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int b = 8 * rg + r;
          const uint32_t o0 = b < M ? (uint32_t)((b * p.xsplits + s) * P + tile * PB + LC * cg) * 4u : kOutOfRange;
#pragma unroll
          for (int w = 0; w < RW; ++w) {
            const u32x4_t x = buf_ld16(rsx, b < M ? o0 + 16u * w : kOutOfRange);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              raw[RW * r + w][j] = __float_as_uint(__uint_as_float(raw[RW * r + w][j]) + __uint_as_float(x[j]));
          }
        }
      }
    } else if constexpr (LC == 8) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int b = 8 * rg + r;
        raw[r] = buf_ld16<MHLA_MIX_LOAD_CPOL>(rsx, b < M ? (uint32_t)(b * P + tile * PB + 8 * cg) * 2u : kOutOfRange);
      }
    } else {   // 4 bf16 columns per row: words 0 and 1 (the transpose reads no others)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int b = 8 * rg + r;
        const u32x2_t w = buf_ld8(rsx, b < M ? (uint32_t)(b * P + tile * PB + 4 * cg) * 2u : kOutOfRange);
        raw[r] = u32x4_t{w[0], w[1], 0u, 0u};
      }
    }
  };

  // tiles n_tiles .. n_tiles + n_ztiles - 1 hold the normaliser: within z tile j, column 2c is
  // hi(z_b[j*PB/2 + c]) and column 2c + 1 its low part
  const int D = p.D;
  const int n_ztiles = (2 * D + PB - 1) / PB;
  const int last = n_tiles + n_ztiles;            // one past the last tile
  // z partials of this head through a buffer resource (rows b >= M read as zero)
  const int zsp = SPLIT ? p.zsplits : 1;
  const Rsrc rsz = make_rsrc(p.z + (int64_t)bh * M * zsp * D, (uint32_t)M * zsp * D * 4u);
  constexpr int ZW = LC / 2;                        // z values per thread and row
  auto z_off = [&](int zj, int b, int s) -> uint32_t {
    const int c0 = zj * (PB / 2) + ZW * cg;
    return (b < M && c0 < D) ? (uint32_t)((b * zsp + s) * D + c0) * 4u : kOutOfRange;
  };
  auto z_load = [&](uint32_t off, float (&x)[ZW]) {
    if constexpr (ZW == 4) {
      const u32x4_t w = buf_ld16(rsz, off);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(w[j]);
    } else {
      const u32x2_t w = buf_ld8(rsz, off);
      x[0] = __uint_as_float(w[0]);
      x[1] = __uint_as_float(w[1]);
    }
  };
  // A z tile is formed at once (z tiles are few): z_b[c0 .. c0 + ZW - 1] of each of the thread's
  // rows, summed over the token slices, as (hi, lo) bf16 pairs.  Its loads are waited for here,
  // so it leaves nothing in flight.
  auto issue_z = [&](int zj) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int b = 8 * rg + r;
      float zs[ZW];
#pragma unroll
      for (int j = 0; j < ZW; ++j) zs[j] = 0.f;
      for (int s = 0; s < zsp; ++s) {
        float x[ZW];
        z_load(z_off(zj, b, s), x);
#pragma unroll
        for (int j = 0; j < ZW; ++j) zs[j] += x[j];
      }
      u32x4_t w = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < ZW; ++j) {
        uint32_t h, l;
        split_bf16(zs[j], h, l);
        w[j] = h | (l << 16);
      }
      raw[RW * r] = w;                         // bf16 (hi, lo) pairs: no further split
    }
  };
  auto issue_any = [&](int t) {
    if (t < n_tiles) issue(t);
    else issue_z(t - n_tiles);
  };

  // transpose 8 rows x LC columns into LDS: column-major with blocks contiguous
  auto transpose = [&](int tile) {
    const bool ztile = tile >= n_tiles;
    if (SPLIT && !ztile) {
      // fp32 rows: row rr holds columns 4w .. 4w + 3 in raw[RW * rr + w]
#pragma unroll
      for (int e = 0; e < LC; ++e) {
        u32x4_t col, col_lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t h, l;
          split_bf16x2(__uint_as_float(raw[RW * (2 * r) + (e >> 2)][e & 3]),
                       __uint_as_float(raw[RW * (2 * r + 1) + (e >> 2)][e & 3]), h, l);
          col[r] = h;
          col_lo[r] = l;
        }
        const int rr = LC * cg + e;
        *reinterpret_cast<u32x4_t*>(xt + rr * XP + 8 * swz(rr, rg)) = col;
        *reinterpret_cast<u32x4_t*>(xt_lo + rr * XP + 8 * swz(rr, rg)) = col_lo;
      }
    } else {
      // bf16 rows: word e/2 of a row holds columns e & ~1 (low half) and e | 1.  The split
      // kernel keeps its bf16 (normaliser) rows in raw[RW * rr] and an all-zero low part.
#pragma unroll
      for (int e = 0; e < LC; ++e) {
        u32x4_t col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t w0 = raw[RW * (2 * r)][e >> 1], w1 = raw[RW * (2 * r + 1)][e >> 1];
          col[r] = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
        }
        const int rr = LC * cg + e;
        *reinterpret_cast<u32x4_t*>(xt + rr * XP + 8 * swz(rr, rg)) = col;
        if constexpr (SPLIT) *reinterpret_cast<u32x4_t*>(xt_lo + rr * XP + 8 * swz(rr, rg)) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  // Outputs through buffer resources: every lane issues the same stores on every path (rows
  // past M and z columns past D get an out-of-range offset and are dropped; a z tile of the
  // split kernel adds an empty store), so that the wait for the next tile's loads, which were
  // issued before these stores, never has to include them.
  const Rsrc ry = make_rsrc(y, (uint32_t)M * P * 2u);
  const Rsrc ryl = make_rsrc(SPLIT ? y_lo : y, (uint32_t)M * P * 2u);
  const Rsrc rzt = make_rsrc(p.zt + (int64_t)bh * M * D, (uint32_t)M * D * 4u);
  auto compute_store = [&](int tile) {
    const bool ztile = tile >= n_tiles;
    const int zbase = (tile - n_tiles) * (PB / 2);
    auto column_group = [&](int cgp) {
      // the lane's row and chunk indices through an empty asm: the operand offsets below are
      // the same for every tile, and hoisted out of the tile loop they would hold ~30 registers
      int prv = pr, lgv = lg;
      asm volatile("" : "+v"(prv), "+v"(lgv));
      f32x4_t accs[2][ITW];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int a = 0; a < ITW; ++a) accs[pt][a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (SPLIT) {
        // two accumulators (pt = 0, 1), both chunks' operands read first, then three rounds
        // of independent MFMAs (hi*hi, lo*hi, hi*lo)
#pragma unroll
        for (int bc = 0; bc < NBC; ++bc) {
          u32x4_t ah[2], al[2];
#pragma unroll
          for (int pt = 0; pt < 2; ++pt) {
            const int r = 32 * cgp + 8 * (prv >> 2) + 4 * pt + (prv & 3);
            const int ofs = r * XP + 8 * swz(r, 4 * bc + lgv);
            ah[pt] = *reinterpret_cast<const u32x4_t*>(xt + ofs);
            al[pt] = *reinterpret_cast<const u32x4_t*>(xt_lo + ofs);
          }
#pragma unroll
          for (int a = 0; a < ITW; ++a)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) accs[pt][a] = mfma_bf16(ah[pt], bfrag[a][bc], accs[pt][a]);
#pragma unroll
          for (int a = 0; a < ITW; ++a)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) accs[pt][a] = mfma_bf16(al[pt], bfrag[a][bc], accs[pt][a]);
#pragma unroll
          for (int a = 0; a < ITW; ++a)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) accs[pt][a] = mfma_bf16(ah[pt], bfrag_lo[a][bc], accs[pt][a]);
        }
      } else {
#pragma unroll
        for (int bc = 0; bc < NBC; ++bc)
#pragma unroll
          for (int pt = 0; pt < 2; ++pt) {
            const int r = 32 * cgp + 8 * (prv >> 2) + 4 * pt + (prv & 3);
            const int ofs = r * XP + 8 * swz(r, 4 * bc + lgv);
            const u32x4_t afrag = *reinterpret_cast<const u32x4_t*>(xt + ofs);
#pragma unroll
            for (int a = 0; a < ITW; ++a) accs[pt][a] = mfma_bf16(afrag, bfrag[a][bc], accs[pt][a]);
            if constexpr (WLO) {
#pragma unroll
              for (int a = 0; a < ITW; ++a) accs[pt][a] = mfma_bf16(afrag, bfrag_lo[a][bc], accs[pt][a]);
            }
            // with 128 registers of M_c fragments, keep each operand read next to its MFMAs
            if constexpr (NBC * ITW >= 32) __builtin_amdgcn_sched_barrier(0);
          }
      }
      const int q = 32 * cgp + 8 * lg;         // first of this lane's 8 tile columns
#pragma unroll
      for (int a = 0; a < ITW; ++a) {
        const int i = 16 * (it0 + a) + pr;     // i >= M: nothing to store
        const f32x4_t c0 = accs[0][a], c1 = accs[1][a];
        if (!ztile) {
          const uint32_t o = i < M ? (uint32_t)(i * P + tile * PB + q) * 2u : kOutOfRange;
          if constexpr (SPLIT) {
            const float v[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            uint32_t h[4], l[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_bf16x2(v[2 * j], v[2 * j + 1], h[j], l[j]);
            buf_st16(ry, o, u32x4_t{h[0], h[1], h[2], h[3]});
            // the low plane non-temporally: the high plane, which the next readout reads at the
            // training accuracy, then stays in the infinity cache (train forward 0.485 -> 0.469 ms)
            buf_st16<2>(ryl, o, u32x4_t{l[0], l[1], l[2], l[3]});
          } else {
            buf_st16(ry, o, u32x4_t{pack_bf16x2(c0[0], c0[1]), pack_bf16x2(c0[2], c0[3]),
                                    pack_bf16x2(c1[0], c1[1]), pack_bf16x2(c1[2], c1[3])});
          }
        } else {
          // columns 2c, 2c+1 are hi, lo of z index zbase + c: four consecutive z~ values
          const int zi = zbase + q / 2;
          const uint32_t o = (i < M && zi < D) ? (uint32_t)(i * D + zi) * 4u : kOutOfRange;
          buf_st16(rzt, o,
                   u32x4_t{__float_as_uint(c0[0] + c0[1]), __float_as_uint(c0[2] + c0[3]),
                           __float_as_uint(c1[0] + c1[1]), __float_as_uint(c1[2] + c1[3])});
          if constexpr (SPLIT) buf_st16(ryl, kOutOfRange, u32x4_t{0u, 0u, 0u, 0u});
        }
      }
    };
    if constexpr (NBC >= 2) {
      // every wave takes all column groups (for NBC >= 2 every wave has rows of its own,
      // WPW = 1): a fixed number of stores, so the wait for the next tile's loads can count them
#pragma unroll
      for (int cgp = 0; cgp < NCG; ++cgp) {
        column_group(cgp);
        __builtin_amdgcn_sched_barrier(0);     // no overlap of groups: their registers add up
      }
    } else {
#pragma unroll 1
      for (int cgp = wp; cgp < NCG; cgp += WPW) column_group(cgp);
    }
  };

  // Per tile: transpose (waits for its loads), barrier, loads of the next tile, MFMAs and
  // stores, barrier.  The next tile's loads are in flight during the MFMAs and stores.  After
  // the first tile's loads the same number of stores as a tile's (all dropped: out of range)
  // is issued, so that on both paths into the loop the stores issued after the loads are
  // counted and the transpose waits for its loads alone.
  int tile = blockIdx.x;
  if (tile >= last) return;
  issue_any(tile);
  if constexpr (NBC >= 2) {
#pragma unroll
    for (int j = 0; j < NCG * ITW; ++j) {
      buf_st16(ry, kOutOfRange, u32x4_t{0u, 0u, 0u, 0u});
      if constexpr (SPLIT) buf_st16(ryl, kOutOfRange, u32x4_t{0u, 0u, 0u, 0u});
    }
  }
  while (true) {
    transpose(tile);
    __syncthreads();
    if (tile + p.n_wg_x < last) issue_any(tile + p.n_wg_x);
    compute_store(tile);
    __syncthreads();
    tile += p.n_wg_x;
    if (tile >= last) break;
  }
}

template <int NBC, int ITW, bool SPLIT, int NW, bool WLO = false>
static hipError_t launch_t(const MixMfmaParams& p, int row_groups, int bh, hipStream_t s) {
  constexpr int MPAD = 32 * NBC, PB = mix_tile_cols(NBC, SPLIT, NW), XP = MPAD;
  const size_t lds = (size_t)PB * XP * 2 * (SPLIT ? 2 : 1);
  auto kern = mix_mfma_kernel<NBC, ITW, SPLIT, NW, WLO>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.n_wg_x, row_groups, bh), dim3(NW * 64), lds, s, p);
  return hipGetLastError();
}

// Launch with the shape mix_shape(M, split, wlo) (the host sized the W fragments with the same
// shape).  wlo: the bf16 kernel with W as hi + lo (mcf_lo required).
hipError_t launch_mix_mfma(MixMfmaParams p, int bh, bool split, bool wlo, hipStream_t stream) {
  const int M = p.M;
  if (M < 1 || M > 256) return hipErrorInvalidValue;
  if (split ? (!p.xf || !p.mcf_lo || !p.y_lo || p.xsplits < 1) : (!p.x || p.zsplits != 1))
    return hipErrorInvalidValue;
  if (split && wlo) return hipErrorInvalidValue;
  if (wlo && !p.mcf_lo) return hipErrorInvalidValue;
  const MixShape sh = mix_shape(M, split, wlo);
  const int NBC = sh.nbc, ITW = sh.itw, row_groups = sh.row_groups, NW = sh.nw;
  p.wave_rows = sh.wave_rows;
  if (NBC >= 2 && sh.wave_rows != NW) return hipErrorInvalidValue;   // the kernel assumes WPW = 1
  const int pb = mix_tile_cols(NBC, split, NW);
  const int n_tiles = p.frag / pb;
  if (p.frag % pb != 0) return hipErrorInvalidValue;
  const int n_all = n_tiles + (2 * p.D + pb - 1) / pb;     // summary tiles + normaliser tiles
  // about two 4-wave (or one 8-wave) workgroups per CU across all heads, each striding over
  // many column tiles
  const int target = NW == 8 ? 256 : 512;
  int want = (target + bh * row_groups - 1) / (bh * row_groups);
  if (want > n_all) want = n_all;
  if (want < 1) want = 1;
  // several row groups: a multiple of 8 workgroups per row group puts the row groups of one
  // column tile on the same XCD (workgroups are dealt to the 8 XCDs round robin), so the
  // tile they all load is fetched from HBM once into that XCD's L2
  if (row_groups > 1 && want > 8) want &= ~7;
  p.n_wg_x = want;
#define MHLA_MIX_CASE(N, I, S, W, L) \
  if (NBC == N && ITW == I && split == S && NW == W && wlo == L) \
    return launch_t<N, I, S, W, L>(p, row_groups, bh, stream);
  MHLA_MIX_CASE(1, 1, false, 4, false) MHLA_MIX_CASE(2, 1, false, 4, false) MHLA_MIX_CASE(4, 2, false, 4, false)
  MHLA_MIX_CASE(8, 4, false, 4, false) MHLA_MIX_CASE(1, 1, true, 4, false) MHLA_MIX_CASE(2, 1, true, 4, false)
  MHLA_MIX_CASE(4, 1, true, 4, false) MHLA_MIX_CASE(8, 2, true, 8, false)
  MHLA_MIX_CASE(1, 1, false, 4, true) MHLA_MIX_CASE(2, 1, false, 4, true) MHLA_MIX_CASE(4, 2, false, 4, true)
  MHLA_MIX_CASE(8, 2, false, 8, true)
#undef MHLA_MIX_CASE
  return hipErrorInvalidValue;
}

}  // namespace mhla
