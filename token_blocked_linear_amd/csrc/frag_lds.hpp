// LDS staging of d x d summaries in fragment layout, shared by the readout and the backward
// kernels.  A summary T (rows k = contraction index, columns = output index) is stored as
// MFMA A-operand fragments: element (kc, ct, lane, e) holds T[32kc + 8(lane/16) + e][16ct + lane%16]
// at flat index ((kc * NCT + ct) * 64 + lane) * 8 + e.  In LDS, bit 2 of a fragment's lane index
// is flipped when bit 3 is set (lds_pos), so that the permuted operand reads below cover every
// bank once per 8 lanes.  Output channels are taken 32 at a time as two MFMA tiles h = 0, 1
// whose A row m is output 8*(m/4) + 4h + m%4 of the group (a_offsets), so that lane (t, g) ends
// with the 8 consecutive outputs 8g .. 8g+7 of its column t.
#pragma once

#include "mhla_device.hpp"

namespace mhla {

template <bool SPLIT>
__device__ inline void store_frag8(uint16_t* s_hi, uint16_t* s_lo, int pos, const float (&a)[8]) {
  if (SPLIT) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16x2(a[2 * i], a[2 * i + 1], h[i], l[i]);
    st16(s_hi + pos, u32x4_t{h[0], h[1], h[2], h[3]});
    st16(s_lo + pos, u32x4_t{l[0], l[1], l[2], l[3]});
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


// Normaliser fragments from z~ (fp32 in LDS): rows 4g = hi, 4g + 1 = lo, other rows zero.
template <int D>
__device__ inline void build_zfrag(const float* s_zt, uint16_t* s_z, int tid) {
  constexpr int NKC = Dims<D>::NKC;
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
}

// A-operand LDS offsets: A row pr of tile ct is channel 32*(ct/2) + 8*(pr/4) + 4*(ct%2) + pr%4
// (d >= 32).  It sits in fragment ct & ~1 (or the next one for pr >= 8) at lane
// 16*lg + 8*b + 4*(ct%2) + pr%4, b = (pr/4)%2, which the LDS swizzle moves to
// 16*lg + 8*b + 4*((ct%2) ^ b) + pr%4.  Only these two lane-dependent bases exist.
struct AOffsets {
  int even, odd;
};
__device__ inline AOffsets a_offsets(int lane) {
  const int pr = lane & 15, lg = lane >> 4, b3 = (pr >> 2) & 1;
  return {((pr >> 3) * 64 + 16 * lg + 8 * b3 + 4 * (0 ^ b3) + (pr & 3)) * 8,
          ((pr >> 3) * 64 + 16 * lg + 8 * b3 + 4 * (1 ^ b3) + (pr & 3)) * 8};
}

}  // namespace mhla
