// Streaming decode of chunkwise-causal MHLA: one new token per (batch, head) and call.
//
// "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head", Method -> Key
// design 2 (the token-expanded identity q~^T S~_i = sum_t m_{i,b(t)} (q~^T K~_t) V_t^T) and Key
// design 4 (compatible with streaming / stateful inference).  With the causal reading of the
// causal readouts, token t of block i (t / n_b; with a CLS token 0 for t = 0, else 1 + (t - 1) / n_b) reads
//   o_t = q~_t^T (S~<_i + m_ii R_t) / q~_t^T (z~<_i + m_ii r_t),   S~<_i = sum_{b<i} m_ib S_b,
// R_t = sum of k~ v^T over block i's tokens up to t (r_t: of k~).  The state is fp32.
//
// The d output channels of a head are cut into slices of C = 2^log2_c channels, one workgroup
// each (d / C workgroups per head), so that a small batch still spreads over the chip: a slice
// holds the d x C columns of every d x d matrix (the completed blocks' S_b, S~<_i, R) and its own
// copy of the d-vectors (z_b, z~<_i, r), which every slice updates identically.  Slice layout,
// floats: hS [M][d*C], hz [M][d], St [d*C], zt [d], R [d*C], r [d]; slices of a head follow each
// other, heads follow each other.
//
// Thread tid owns the float4s e = tid + 256 j of the slice's matrices (feature f = 4 e / C,
// channels 4 e % C .. + 3; C * d >= 1024) and, for tid < d, feature tid of the vectors -- the same
// elements on every call,
// so the state needs no synchronisation beyond the order of the calls.  At the first token of a
// block (i > 0) the thread stores R as S_{i-1}, forms its elements of S~<_i from row i of M_c and
// clears R; then it adds k~_f v_c to R and sums q~_f (S~< + m_ii R) over its features.  The
// partial sums of a channel meet through lane shuffles and LDS in a fixed order.
#include <type_traits>

#include "mhla_device.hpp"

namespace mhla {

template <typename T>
__device__ inline float load_elem(const void* base, int64_t i) {
  if constexpr (sizeof(T) == 2) return bf16lo_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  else return reinterpret_cast<const float*>(base)[i];
}

template <typename TIn, typename TOut, int D, int PHI>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeParams p) {
  static_assert(D >= 32 && D <= 128, "head sizes 32 .. 128 (causal plans)");
  __shared__ float s_q[D], s_k[D], s_v[D], s_den[4];
  __shared__ float4 s_part[kThreads];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int lc = p.log2_c, C = 1 << lc, S = D >> lc;         // C * D >= 1024
  const int DC = D * C, per = DC / (4 * kThreads);            // float4s of a matrix per thread
  const int bh = (int)(blockIdx.x / S), sl = (int)(blockIdx.x % S), h = bh % p.H;
  const int M = p.M;
  const int64_t slot = ((int64_t)bh * S + sl) * ((int64_t)(M + 2) * (DC + D));
  float* hS = p.state + slot;            // [M][DC]
  float* hz = hS + (int64_t)M * DC;      // [M][D]
  float* St = hz + (int64_t)M * D;       // [DC]
  float* zt = St + DC;                   // [D]
  float* R = zt + D;                     // [DC]
  float* r = R + DC;                     // [D]
  float4* hS4 = reinterpret_cast<float4*>(hS);
  float4* St4 = reinterpret_cast<float4*>(St);
  float4* R4 = reinterpret_cast<float4*>(R);
  const int DC4 = DC / 4;

  // block i of position t and t's place in it (with a CLS token: block 0 is position 0 alone)
  const int64_t tg = p.t - p.cls;
  const int i = tg < 0 ? 0 : (int)(tg / p.nb) + p.cls, pos = tg < 0 ? 0 : (int)(tg % p.nb);
  const float* mrow = p.mc ? p.mc + (int64_t)h * p.mc_head_stride + (int64_t)i * M : nullptr;
  const float mii = mrow ? mrow[i] : 1.0f;

  // the thread's R and S~< (and r, z~<) do not depend on the token: their loads go out with
  // the token's, before the barrier
  constexpr int MAXPER = D * D / (4 * kThreads);
  float4 rr[MAXPER], ss[MAXPER];
#pragma unroll
  for (int j = 0; j < MAXPER; ++j)
    if (j < per) {
      rr[j] = R4[tid + kThreads * j];
      ss[j] = St4[tid + kThreads * j];
    }
  float rv = 0.f, zv = 0.f;
  if (tid < D) {
    rv = r[tid];
    zv = zt[tid];
    const int64_t x = (int64_t)bh * D + tid;
    s_q[tid] = phi_map<PHI>(load_elem<TIn>(p.q, x));
    s_k[tid] = phi_map<PHI>(load_elem<TIn>(p.k, x));
    if (tid < C) s_v[tid] = load_elem<TIn>(p.v, (int64_t)bh * D + sl * C + tid);
  }

  if (pos == 0 && i > 0) {
    // block i-1 is complete: keep it, mix the completed blocks with row i of M_c, restart R, r
    const float m = mrow[i - 1];
#pragma unroll
    for (int j = 0; j < MAXPER; ++j)
      if (j < per) {
        const int e = tid + kThreads * j;
        const float4 done = rr[j];
        hS4[(int64_t)(i - 1) * DC4 + e] = done;
        // four interleaved partial sums (b mod 4), so that four loads are in flight
        float4 a[4] = {make_float4(m * done.x, m * done.y, m * done.z, m * done.w), make_float4(0.f, 0.f, 0.f, 0.f),
                       make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
        int b = 0;
        for (; b + 4 <= i - 1; b += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float mb = mrow[b + u];
            const float4 x = hS4[(int64_t)(b + u) * DC4 + e];
            a[u].x = fmaf(mb, x.x, a[u].x);
            a[u].y = fmaf(mb, x.y, a[u].y);
            a[u].z = fmaf(mb, x.z, a[u].z);
            a[u].w = fmaf(mb, x.w, a[u].w);
          }
        }
        for (; b < i - 1; ++b) {
          const float mb = mrow[b];
          const float4 x = hS4[(int64_t)b * DC4 + e];
          a[0].x = fmaf(mb, x.x, a[0].x);
          a[0].y = fmaf(mb, x.y, a[0].y);
          a[0].z = fmaf(mb, x.z, a[0].z);
          a[0].w = fmaf(mb, x.w, a[0].w);
        }
        const float4 sum = make_float4((a[0].x + a[1].x) + (a[2].x + a[3].x), (a[0].y + a[1].y) + (a[2].y + a[3].y),
                                       (a[0].z + a[1].z) + (a[2].z + a[3].z), (a[0].w + a[1].w) + (a[2].w + a[3].w));
        St4[e] = sum;
        ss[j] = sum;
        rr[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    if (tid < D) {
      hz[(int64_t)(i - 1) * D + tid] = rv;
      float a = m * rv;
      for (int b = 0; b < i - 1; ++b) a = fmaf(mrow[b], hz[(int64_t)b * D + tid], a);
      zt[tid] = a;
      zv = a;
      rv = 0.f;
    }
  }
  __syncthreads();   // s_q, s_k, s_v

  // R += k~ v^T (token t sees itself), then the thread's part of q~^T (S~< + m_ii R) for its
  // four channels c4 .. c4 + 3 of feature f
  const int lc4 = lc - 2, C4 = C >> 2;
  const int c4 = (tid & (C4 - 1)) * 4, f0 = tid >> lc4, fstep = kThreads >> lc4;
  const float v0 = s_v[c4], v1 = s_v[c4 + 1], v2 = s_v[c4 + 2], v3 = s_v[c4 + 3];
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < MAXPER; ++j)
    if (j < per) {
      const int f = f0 + fstep * j;
      const float kf = s_k[f], qf = s_q[f];
      float4 rn = rr[j];
      const float4 st = ss[j];
      rn.x = fmaf(kf, v0, rn.x);
      rn.y = fmaf(kf, v1, rn.y);
      rn.z = fmaf(kf, v2, rn.z);
      rn.w = fmaf(kf, v3, rn.w);
      R4[tid + kThreads * j] = rn;
      num.x = fmaf(qf, fmaf(mii, rn.x, st.x), num.x);
      num.y = fmaf(qf, fmaf(mii, rn.y, st.y), num.y);
      num.z = fmaf(qf, fmaf(mii, rn.z, st.z), num.z);
      num.w = fmaf(qf, fmaf(mii, rn.w, st.w), num.w);
    }
  float den = 0.f;
  if (tid < D) {
    const float rn = rv + s_k[tid];
    r[tid] = rn;
    den = s_q[tid] * fmaf(mii, rn, zv);
  }
  // lanes of one channel group within a wave (lane = group mod C/4), then the waves
  for (int m = 32; m >= C4; m >>= 1) {
    num.x += __shfl_xor(num.x, m);
    num.y += __shfl_xor(num.y, m);
    num.z += __shfl_xor(num.z, m);
    num.w += __shfl_xor(num.w, m);
  }
  for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m);
  const int cw = C4 < 64 ? 64 : C4;
  if (lane < C4) s_part[tid] = num;
  if (lane == 0) s_den[wave] = den;
  __syncthreads();
  if (tid < C) {
    const float* part = reinterpret_cast<const float*>(s_part);
    float n = 0.f;
    for (int q = 0; q < kThreads / cw; ++q) n += part[4 * ((tid >> 2) + cw * q) + (tid & 3)];  // fixed order
    const float dsum = (s_den[0] + s_den[1]) + (s_den[2] + s_den[3]);
    const float o = p.normalized ? n / dsum : n;
    const int64_t x = (int64_t)bh * D + sl * C + tid;
    if constexpr (sizeof(TOut) == 2) reinterpret_cast<uint16_t*>(p.o)[x] = (uint16_t)f32_to_bf16_bits(o);
    else reinterpret_cast<float*>(p.o)[x] = o;
  }
}

// The state that decode_step_kernel leaves after positions 0 .. n-1, written at once from a
// chunkwise causal forward over them.  With i = Mp - 1 the block of position n - 1: the completed
// blocks b < i are kept (hS[b], hz[b]), S~<_i and z~<_i are row i of the strictly lower mixing,
// and R, r are block i's sums over its positions up to n - 1 (its whole summary in the prefix:
// the prefix's last block ends at n - 1).  Element (f, c) of a slice's matrix is feature f,
// channel sl C + c, at f C + c; the summaries are read from their fragment layout (feature f:
// chunk f / 32, lane group (f % 32) / 8, element f % 8; channel ch: tile ch / 16, lane ch % 16).
__global__ __launch_bounds__(kThreads) void prefill_state_kernel(PrefillStateParams p, int D) {
  const int C = 1 << p.log2_c, S = D >> p.log2_c, DC = D * C, NCT = D / 16, Mp = p.Mp;
  const int64_t per_slice = (int64_t)(Mp + 1) * (DC + D);   // hS[0 .. Mp-2], St, R; hz[..], zt, r
  const int64_t total = (int64_t)p.BH * S * per_slice;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t bs = idx / per_slice;
    int64_t w = idx - bs * per_slice;
    const int bh = (int)(bs / S), sl = (int)(bs % S);
    float* slot = p.state + bs * ((int64_t)(p.M + 2) * (DC + D));
    float* hS = slot;
    float* hz = hS + (int64_t)p.M * DC;
    float* St = hz + (int64_t)p.M * D;
    float* zt = St + DC;
    float* R = zt + D;
    float* r = R + DC;
    const int64_t last = (int64_t)bh * Mp + (Mp - 1);   // the prefix's row of block Mp - 1
    if (w < (int64_t)(Mp + 1) * DC) {
      const int m = (int)(w / DC), e = (int)(w % DC);     // m < Mp - 1: hS[m]; Mp - 1: St; Mp: R
      const int f = e / C, ch = sl * C + e % C;
      const int pos = (((f >> 5) * NCT + (ch >> 4)) * 64 + 16 * ((f & 31) >> 3) + (ch & 15)) * 8 + (f & 7);
      float x = 0.f;
      if (m == Mp - 1) {                                  // S~<_i: hi + lo of the mixing
        if (p.st_hi) {
          x = __uint_as_float((uint32_t)p.st_hi[last * p.frag + pos] << 16);
          if (p.st_lo) x += __uint_as_float((uint32_t)p.st_lo[last * p.frag + pos] << 16);
        }
        St[e] = x;
      } else {                                            // S_b: the sum of its slice partials
        const int b = m < Mp - 1 ? m : Mp - 1;
        const int64_t row = (int64_t)bh * Mp + b;
        for (int s = 0; s < p.splits; ++s) x += p.part[(row * p.splits + s) * p.frag + pos];
        if (m < Mp - 1) hS[(int64_t)m * DC + e] = x;
        else R[e] = x;
      }
    } else {
      w -= (int64_t)(Mp + 1) * DC;
      const int m = (int)(w / D), f = (int)(w % D);
      float x = 0.f;
      if (m == Mp - 1) {
        if (p.zt) x = p.zt[last * D + f];
        zt[f] = x;
      } else {
        const int b = m < Mp - 1 ? m : Mp - 1;
        const int64_t row = (int64_t)bh * Mp + b;
        for (int s = 0; s < p.splits; ++s) x += p.pz[(row * p.splits + s) * D + f];
        if (m < Mp - 1) hz[(int64_t)m * D + f] = x;
        else r[f] = x;
      }
    }
  }
}

// zeroes `n` floats (a plain fill: no memset node, so a captured graph replays it correctly)
__global__ __launch_bounds__(kThreads) void decode_zero_kernel(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) x[i] = 0.f;
}

template <typename TIn, typename TOut, int PHI>
static hipError_t decode_d(const DecodeParams& p, int d, hipStream_t s) {
  const dim3 grid((unsigned)p.BH * (unsigned)(d >> p.log2_c));
  switch (d) {
    case 32: hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, 32, PHI>), grid, dim3(kThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, 64, PHI>), grid, dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL((decode_step_kernel<TIn, TOut, 128, PHI>), grid, dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeParams& p, int d, bool in_fp32, bool out_fp32, int phi, hipStream_t s) {
  // C = 2^log2_c channels per workgroup: at least 8, at most d, and C * d >= 4 * 256
  if (p.log2_c < 3 || (1 << p.log2_c) > d || (d << p.log2_c) < 4 * kThreads) return hipErrorInvalidValue;
  auto go = [&](auto phi_c) {
    constexpr int PHI = decltype(phi_c)::value;
    if (in_fp32) return out_fp32 ? decode_d<float, float, PHI>(p, d, s) : decode_d<float, uint16_t, PHI>(p, d, s);
    return out_fp32 ? decode_d<uint16_t, float, PHI>(p, d, s) : decode_d<uint16_t, uint16_t, PHI>(p, d, s);
  };
  switch (phi) {
    case kPhiElu1: return go(std::integral_constant<int, kPhiElu1>{});
    case kPhiRelu: return go(std::integral_constant<int, kPhiRelu>{});
    case kPhiExp: return go(std::integral_constant<int, kPhiExp>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_state(const PrefillStateParams& p, int d, hipStream_t s) {
  if (p.log2_c < 3 || (1 << p.log2_c) > d || p.Mp < 1 || p.Mp > p.M) return hipErrorInvalidValue;
  const int64_t total = (int64_t)p.BH * (d >> p.log2_c) * (int64_t)(p.Mp + 1) * ((int64_t)d * (1 << p.log2_c) + d);
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(prefill_state_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, d);
  return hipGetLastError();
}

hipError_t launch_decode_zero(float* x, int64_t n, hipStream_t s) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(decode_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, n);
  return hipGetLastError();
}

}  // namespace mhla
