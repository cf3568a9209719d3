// Host side of the C ABI declared in include/mhla.h: descriptor validation, the plan
// (geometry, kernel variants, token slicing, workspace layout), launches of the summary,
// mixing and readout kernels on the caller's stream, and optional per-kernel HIP events.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "mhla.h"
#include "mhla_device.hpp"

namespace mhla {
hipError_t launch_summary(const SummaryParams& p, int d, bool in_fp32, bool split_k, bool split_v,
                          bool want_u, bool out_bf16, int phi, int n_units, hipStream_t stream);
hipError_t launch_summary_tokw(const SummaryParams& p, int d, bool in_fp32, bool v_fp32, int phi, int n_units,
                               hipStream_t stream);
hipError_t launch_mix(const MixParams& p, int d, int frag, int bh, bool split, hipStream_t stream);
hipError_t launch_mix_mfma(MixMfmaParams p, int bh, bool split, bool wlo, hipStream_t stream);
hipError_t launch_readout(const ReadoutParams& p, int d, bool in_fp32, bool out_fp32, int mode,
                          bool split, int fuse, bool q_stream, int phi, int n_wg, hipStream_t stream);
hipError_t launch_bwd_tiles(const BwdParams& p, int d, bool in_fp32, bool out_fp32, int mode, int phi,
                            bool key_side, int n_units, hipStream_t stream);
hipError_t launch_dmc(const DmcParams& p, float* dmc, hipStream_t stream);
hipError_t launch_mala_stage(const MalaStageParams& p, int d, int bh, hipStream_t stream);
hipError_t launch_decode_step(const DecodeParams& p, int d, bool in_fp32, bool out_fp32, int phi, hipStream_t s);
hipError_t launch_decode_zero(float* x, int64_t n, hipStream_t s);
hipError_t launch_causal(const CausalParams& p, int d, bool in_fp32, bool out_fp32, int phi, int n_units,
                         hipStream_t stream);
hipError_t launch_slice_prefix(float* ps, float* pz, int64_t rows, int splits, int frag, int d, hipStream_t stream);
hipError_t launch_frag_to_rowmajor(const uint16_t* hi, const uint16_t* lo, const float* part, int splits,
                                   int64_t rows, int d, int frag, float* out, hipStream_t stream);
hipError_t launch_sum_splits(const float* part, int splits, int64_t rows, int d, float* out, hipStream_t stream);
hipError_t launch_prefill_state(const PrefillStateParams& p, int d, hipStream_t s);
}  // namespace mhla

namespace {

constexpr int kMaxKernels = 4;

// Mixing step placement: a separate kernel, or the readout's prologue (few blocks).
enum { kFuseNone = 0, kFuseBf16 = 1, kFusePartials = 2 };
#ifndef MHLA_FUSE_MAX_BLOCKS
#define MHLA_FUSE_MAX_BLOCKS 16
#endif
constexpr int kFuseMaxBlocks = MHLA_FUSE_MAX_BLOCKS;
#ifndef MHLA_MIX_IN_PLACE
#define MHLA_MIX_IN_PLACE 1
#endif
constexpr bool kMixInPlace = MHLA_MIX_IN_PLACE != 0;
#ifndef MHLA_MIX_MC_SPLIT
#define MHLA_MIX_MC_SPLIT 1
#endif
constexpr bool kMixMcSplit = MHLA_MIX_MC_SPLIT != 0;

// Timing: one event before a call's first kernel and one after each of its kernels.
constexpr int kMaxTimedKernels = 7;
struct TimedLaunch {
  hipEvent_t ev[kMaxTimedKernels + 1];
};
struct PassTimer {
  std::vector<TimedLaunch> calls;
  size_t used = 0;
};

// The backward's kernels in launch order (the dM_c entry covers its two kernels and is empty
// when no dM_c is requested).
constexpr int kBwdKernels = 7;
const char* const kBwdNames[kBwdKernels] = {"bwd_summary", "bwd_mix",     "bwd_dq", "bwd_dsummary",
                                            "bwd_dmix",    "bwd_keyside", "bwd_dmc"};

}  // namespace

struct mhla_plan {
  mhla_desc desc;
  int d;
  int64_t B, H, BH, N, M, n_b;
  mhla::Geom geom;
  bool in_fp32, out_fp32, mala, split, split_v;
  bool rd_split;   // the readout's own operands split (= split, except at MHLA_ACCURACY_TRAIN)
  bool mix_mfma;   // bf16 summary stack (mixed on MFMA or in the readout prologue)
  bool mix_split;  // mixing kernel on MFMA with split operands over fp32 partials
  bool mix_wlo;    // the bf16 mixing kernel takes M_c as bf16 hi + lo
  bool causal;     // chunkwise-causal readout (1D)
  bool causal_split;  // the bf16-input causal kernel's own products on split operands (= split,
                      // except in a decode prefill's plan, which keeps the decode plan's)
  bool mix_kernel; // a mixing kernel of its own is launched
  bool mix_in_place; // the mixing kernel overwrites the bf16 summary stack with the mixed one
  bool q_stream;     // the readout loads the queries with the non-temporal policy
  int fuse;        // kFuse*: where the mixing step runs
  int n_kernels;
  const char* kernel_names[kMaxKernels];
  int mode;
  int frag;
  int32_t sum_splits, sum_tok;
  int32_t rd_splits, rd_tok;
  // workspace layout (byte offsets)
  size_t off_sb, off_ps, off_pz, off_pu, off_st_hi, off_st_lo, off_zt, off_mcf, off_mcf_lo, ws_bytes;
  mhla::MixShape mix;   // MFMA mixing launch shape (mix_mfma or mix_split)
  int mcf_heads;
  // timing
  bool timing;
  PassTimer fwd_timer, bwd_timer;
};

namespace {

// Start a timed call on `s`: take the next event set (created on first use) and record the
// start event.
bool timer_begin(PassTimer& t, hipStream_t s, TimedLaunch*& tl) {
  if (t.used == t.calls.size()) {
    TimedLaunch c;
    for (int i = 0; i <= kMaxTimedKernels; ++i)
      if (hipEventCreate(&c.ev[i]) != hipSuccess) return false;
    t.calls.push_back(c);
  }
  tl = &t.calls[t.used++];
  return hipEventRecord(tl->ev[0], s) == hipSuccess;
}

// Summed milliseconds of kernel `index` over the timed calls (waits for the last one).
mhla_status timer_read(const PassTimer& t, int index, int n_kernels, double* total_ms, int64_t* launches) {
  double sum = 0.0;
  if (t.used > 0) {
    if (hipEventSynchronize(t.calls[t.used - 1].ev[n_kernels]) != hipSuccess) return MHLA_ERR_HIP;
    for (size_t i = 0; i < t.used; ++i) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, t.calls[i].ev[index], t.calls[i].ev[index + 1]) != hipSuccess)
        return MHLA_ERR_HIP;
      sum += ms;
    }
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int64_t)t.used;
  return MHLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mhla_status build_plan(const mhla_desc* din, mhla_plan* P) {
  // the earlier layout ended before `flags`: accepted with flags = 0
  mhla_desc dcopy = {};
  if (din->struct_size == sizeof(mhla_desc)) {
    dcopy = *din;
  } else if (din->struct_size == offsetof(mhla_desc, flags)) {
    std::memcpy(&dcopy, din, offsetof(mhla_desc, flags));
    dcopy.struct_size = sizeof(mhla_desc);
  } else {
    return MHLA_ERR_INVALID_ARG;
  }
  const mhla_desc* d = &dcopy;
  if ((d->flags & ~(MHLA_FLAG_RAGGED_BLOCKS | MHLA_FLAG_CLS_TOKEN)) != 0 || d->reserved != 0)
    return MHLA_ERR_INVALID_ARG;
  const bool ragged = (d->flags & MHLA_FLAG_RAGGED_BLOCKS) != 0;
  const int64_t cls = (d->flags & MHLA_FLAG_CLS_TOKEN) ? 1 : 0;
  if (d->in_dtype != MHLA_DTYPE_BF16 && d->in_dtype != MHLA_DTYPE_FP32) return MHLA_ERR_UNSUPPORTED;
  if (d->out_dtype != MHLA_DTYPE_BF16 && d->out_dtype != MHLA_DTYPE_FP32) return MHLA_ERR_UNSUPPORTED;
  if (d->phi != MHLA_PHI_ELU1 && d->phi != MHLA_PHI_RELU && d->phi != MHLA_PHI_EXP)
    return MHLA_ERR_UNSUPPORTED;
  if (d->readout < MHLA_READOUT_NORMALIZED || d->readout > MHLA_READOUT_CAUSAL_UNNORMALIZED)
    return MHLA_ERR_UNSUPPORTED;
  if (d->accuracy < MHLA_ACCURACY_AUTO || d->accuracy > MHLA_ACCURACY_TRAIN) return MHLA_ERR_UNSUPPORTED;
  if (d->mc_per_head != 0 && d->mc_per_head != 1) return MHLA_ERR_INVALID_ARG;
  if (!(d->head_dim == 16 || d->head_dim == 32 || d->head_dim == 64 || d->head_dim == 128))
    return MHLA_ERR_UNSUPPORTED;
  if (d->ndim < 1 || d->ndim > 3) return MHLA_ERR_SHAPE;
  if (d->batch < 1 || d->heads < 1) return MHLA_ERR_SHAPE;
  if (d->batch > 65535 || d->heads > 65535) return MHLA_ERR_SHAPE;   // before their product

  // Extents below 2^31 each; the token and block counts are built one axis at a time and
  // bounded after every factor, so no product can overflow (each factor and each partial
  // product stays below 2^31).
  constexpr int64_t kLim = (int64_t)1 << 31;
  int64_t grid[3] = {1, 1, 1}, block[3] = {1, 1, 1};
  const int pad = 3 - d->ndim;
  int64_t nblk[3] = {1, 1, 1};
  int64_t n_grid = 1, n_blk = 1, nb = 1;
  for (int a = 0; a < d->ndim; ++a) {
    if (d->grid[a] < 1 || d->block[a] < 1) return MHLA_ERR_SHAPE;
    if (d->grid[a] >= kLim) return MHLA_ERR_SHAPE;
    if (d->grid[a] % d->block[a] != 0 && !ragged) return MHLA_ERR_SHAPE;
    grid[pad + a] = d->grid[a];
    block[pad + a] = std::min(d->block[a], d->grid[a]);   // a block never exceeds the grid
    nblk[pad + a] = (grid[pad + a] + block[pad + a] - 1) / block[pad + a];
    n_grid *= grid[pad + a];
    if (n_grid >= kLim) return MHLA_ERR_SHAPE;
    n_blk *= nblk[pad + a];
    if (n_blk > 65535) return MHLA_ERR_SHAPE;
    nb *= block[pad + a];                                 // <= n_grid: bounded with it
  }
  const int64_t N = cls + n_grid;                          // tokens per head
  if (N >= kLim) return MHLA_ERR_SHAPE;
  const int64_t M = cls + n_blk;
  const int64_t BH = d->batch * d->heads;                  // < 2^32: no overflow
  if (BH > 65535 || M > 65535) return MHLA_ERR_SHAPE;
  if (d->readout == MHLA_READOUT_MALA && M != 1) return MHLA_ERR_UNSUPPORTED;
  const bool causal = d->readout == MHLA_READOUT_CAUSAL_NORMALIZED || d->readout == MHLA_READOUT_CAUSAL_UNNORMALIZED;
  if (causal && (d->ndim != 1 || d->head_dim < 32)) return MHLA_ERR_UNSUPPORTED;   // 1D sequences, d >= 32
  // element offsets are 64-bit; guard the total size against overflow
  if (BH > ((int64_t)1 << 62) / (N * d->head_dim * 4)) return MHLA_ERR_SHAPE;
  // the kernels address one head of Q, K, V (and one head's summary stack) through buffer
  // resources with 31-bit byte ranges
  if (N * d->head_dim * 4 >= ((int64_t)1 << 31)) return MHLA_ERR_SHAPE;

  P->desc = *d;
  P->d = (int)d->head_dim;
  P->B = d->batch;
  P->H = d->heads;
  P->BH = BH;
  P->N = N;
  P->M = M;
  P->n_b = nb;
  mhla::Geom& g = P->geom;
  g.G1 = (int32_t)grid[1];
  g.G2 = (int32_t)grid[2];
  g.B0 = (int32_t)block[0];
  g.B1 = (int32_t)block[1];
  g.B2 = (int32_t)block[2];
  g.NB1 = (int32_t)nblk[1];
  g.NB2 = (int32_t)nblk[2];
  g.G0 = (int32_t)grid[0];
  g.cls = (int32_t)cls;
  g.fB2 = mhla::make_fastdiv((uint32_t)block[2]);
  g.fB1 = mhla::make_fastdiv((uint32_t)block[1]);
  g.n_b = (int32_t)nb;
  g.N = (int32_t)N;
  g.M = (int32_t)M;

  P->in_fp32 = d->in_dtype == MHLA_DTYPE_FP32;
  P->out_fp32 = d->out_dtype == MHLA_DTYPE_FP32;
  P->mala = d->readout == MHLA_READOUT_MALA;
  P->causal = causal;
  P->mode = d->readout;
  // `split` sets the precision of the summaries and the mixing (of the earlier blocks, for the
  // causal readout), and of the bf16-input causal kernel's own products; the fp32-input causal
  // kernel keeps its running state and in-sub-chunk scores split whatever this says.
  if (d->accuracy == MHLA_ACCURACY_SPLIT || d->accuracy == MHLA_ACCURACY_TRAIN)
    P->split = true;
  else if (d->accuracy == MHLA_ACCURACY_BF16)
    P->split = false;
  else
    P->split = P->mala || P->in_fp32 || d->phi != MHLA_PHI_ELU1;
  P->split_v = P->split && P->in_fp32;
  P->causal_split = P->split;

  const int dk = P->d < 32 ? 32 : P->d;
  P->frag = (dk / 32) * (P->d / 16) * 512;

  // Token slicing: enough workgroups to fill 256 CUs several times over, slices >= 256 tokens.
  {
    const int64_t units = BH * M;
    int64_t s = 1;
    if (units < 1024) {
      s = (1024 + units - 1) / units;
      const int64_t max_s = (nb + 255) / 256;
      if (s > max_s) s = max_s;
      if (s < 1) s = 1;
    }
    int64_t tok = (nb + s - 1) / s;
    tok = (tok + 31) / 32 * 32;
    s = (nb + tok - 1) / tok;
    P->sum_splits = (int32_t)s;
    P->sum_tok = (int32_t)tok;
  }
  {
    int64_t s = (nb + 255) / 256;
    int64_t tok = (nb + s - 1) / s;
    tok = (tok + 15) / 16 * 16;
    s = (nb + tok - 1) / tok;
    P->rd_splits = (int32_t)s;
    P->rd_tok = (int32_t)tok;
  }
  if (causal) {   // the summary's token slices are the causal readout's units
    int64_t s = (nb + 255) / 256;
    int64_t tok = (nb + s - 1) / s;
    tok = (tok + 31) / 32 * 32;
    s = (nb + tok - 1) / tok;
    P->sum_splits = P->rd_splits = (int32_t)s;
    P->sum_tok = P->rd_tok = (int32_t)tok;
  }

  // Summary output: a bf16 stack when one token slice covers a block with bf16 operands (the
  // bf16 accuracy level); otherwise fp32 partials per token slice.
  P->mix_mfma = !P->split && !P->mala && !P->in_fp32 && P->sum_splits == 1 && M <= 256;
  // Mixing step: in the readout's prologue for MALA (the centring) and for few blocks; else a
  // kernel of its own: MFMA over the bf16 stack, MFMA with split operands over fp32 partials
  // (M <= 256), VALU over fp32 partials beyond.
  if (P->mala) P->fuse = kFusePartials;
  else if (M <= kFuseMaxBlocks && !causal) P->fuse = P->mix_mfma ? kFuseBf16 : kFusePartials;
  else P->fuse = kFuseNone;
  // causal: a mixing kernel (strictly lower M_c) unless there is one block
  const bool mix_kernel = P->fuse == kFuseNone && !(causal && M == 1);
  P->mix_split = mix_kernel && !P->mix_mfma && M <= 256;
  P->mix_kernel = mix_kernel;
  // MHLA_ACCURACY_TRAIN: split summaries and mixing (what mhla_backward_saved reads), and a
  // readout of the mixed stack's high part with the operands MHLA_ACCURACY_AUTO would choose
  P->rd_split = P->split;
  if (d->accuracy == MHLA_ACCURACY_TRAIN && mix_kernel && !causal && !P->mala && !P->in_fp32 &&
      d->phi == MHLA_PHI_ELU1)
    P->rd_split = false;
  P->n_kernels = 0;
  P->kernel_names[P->n_kernels++] = "summary";
  if (mix_kernel) P->kernel_names[P->n_kernels++] = "mix";
  if (causal) {
    if (P->sum_splits > 1) P->kernel_names[P->n_kernels++] = "scan";
    P->kernel_names[P->n_kernels++] = "causal";
  } else {
    P->kernel_names[P->n_kernels++] = mix_kernel ? "readout" : "mix+readout";
  }

  // Workspace layout.
  const size_t f = (size_t)P->frag, dd = (size_t)P->d;
  const size_t slots = (size_t)BH * M * P->sum_splits;
  size_t off = 0;
  P->off_sb = off;   off = align256(off + (P->mix_mfma ? (size_t)BH * M * f * 2 : 0));
  P->off_ps = off;   off = align256(off + (P->mix_mfma ? 0 : slots * f * 4));
  P->off_pz = off;   off = align256(off + slots * dd * 4);
  P->off_pu = off;   off = align256(off + (P->mala ? slots * dd * 4 : 0));
  // The MFMA mixing of the bf16 stack overwrites the stack in place: for M <= 256 one workgroup
  // covers every row of a column tile and has the whole tile in LDS before its first store, so
  // the mixed stack needs no space of its own (and the stack traffic of a step touches half as
  // many bytes, which then stay in the infinity cache between the three kernels).
  // The bf16 stack's mixing takes M_c as hi + lo: one bf16 M_c perturbs each weight by up to 2^-8
  // relative, the largest rounding of the bf16 path (M_c enters the fused prologue in fp32).
  P->mix_wlo = kMixMcSplit && mix_kernel && P->mix_mfma;
  P->mix_in_place =
      kMixInPlace && mix_kernel && P->mix_mfma && mhla::mix_shape((int)M, false, P->mix_wlo).row_groups == 1;
  if (P->mix_in_place) {
    P->off_st_hi = P->off_sb;
  } else {
    P->off_st_hi = off;
    off = align256(off + (mix_kernel ? (size_t)BH * M * f * 2 : 0));
  }
  // Queries larger than half the 256 MiB infinity cache are streamed past it (nt), so that they
  // do not evict the mixed stack the readout is reading; smaller ones keep the default policy.
  P->q_stream = mix_kernel && P->mix_mfma && !causal && BH * N * d->head_dim * 2 > ((int64_t)128 << 20);
  P->off_st_lo = off;
  off = align256(off + (mix_kernel && (P->split || P->mix_split) ? (size_t)BH * M * f * 2 : 0));
  P->off_zt = off;   off = align256(off + (mix_kernel ? (size_t)BH * M * dd * 4 : 0));
  // bf16 M_c operand fragments (and their low parts) for the MFMA mixing kernel
  P->mcf_heads = d->mc_per_head ? (int)d->heads : 1;
  P->mix = mhla::mix_shape((int)M, P->mix_split, P->mix_wlo);
  const size_t mcf_bytes = (size_t)P->mcf_heads * P->mix.nitp * P->mix.nbc * 512 * 2;
  P->off_mcf = off;
  off = align256(off + (mix_kernel && (P->mix_mfma || P->mix_split) ? mcf_bytes : 0));
  P->off_mcf_lo = off;
  off = align256(off + (P->mix_split || P->mix_wlo ? mcf_bytes : 0));
  P->ws_bytes = off;
  if (BH * M * P->rd_splits >= ((int64_t)1 << 31)) return MHLA_ERR_SHAPE;

  P->timing = false;
  return MHLA_OK;
}

}  // namespace

extern "C" {

mhla_status mhla_create(const mhla_desc* desc, mhla_handle* out) {
  if (!desc || !out) return MHLA_ERR_INVALID_ARG;
  *out = nullptr;
  try {
    mhla_plan* P = new (std::nothrow) mhla_plan();
    if (!P) return MHLA_ERR_INTERNAL;
    const mhla_status s = build_plan(desc, P);
    if (s != MHLA_OK) {
      delete P;
      return s;
    }
    if (std::getenv("MHLA_LOG"))
      std::fprintf(stderr,
                   "mhla: N=%lld M=%lld n_b=%lld d=%d split=%d summary_splits=%d readout_splits=%d "
                   "workspace=%zu\n",
                   (long long)P->N, (long long)P->M, (long long)P->n_b, P->d, (int)P->split,
                   P->sum_splits, P->rd_splits, P->ws_bytes);
    *out = P;
    return MHLA_OK;
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

mhla_status mhla_workspace_size(mhla_handle h, size_t* bytes) {
  if (!h || !bytes) return MHLA_ERR_INVALID_ARG;
  *bytes = h->ws_bytes;
  return MHLA_OK;
}

mhla_status mhla_plan_get_info(mhla_handle h, mhla_plan_info* info) {
  if (!h || !info || info->struct_size != sizeof(mhla_plan_info)) return MHLA_ERR_INVALID_ARG;
  info->n_tokens = h->N;
  info->n_blocks = h->M;
  info->block_tokens = h->n_b;
  info->workspace_bytes = (int64_t)h->ws_bytes;
  info->summary_splits = h->sum_splits;
  info->readout_splits = h->rd_splits;
  info->n_kernels = h->n_kernels;
  info->split_operands = h->split ? 1 : 0;
  return MHLA_OK;
}

}  // extern "C"

namespace {

// The forward's launches on stream s.  With `im`, the run stops after the mixing step (or after
// the summaries when im->St is NULL) and leaves those steps' results in im's fp32 layouts.
struct Intermediates {
  float* S;
  float* z;
  float* St;
  float* zt;
};
// With `pf` (a causal plan over a decode prefix), the decode state is written from the summaries
// and the mixing before the slice scan reuses the partials, and the run goes on to the readout.
struct PrefillHook {
  float* state;
  int64_t M;      // blocks of the decode plan
  int log2_c;     // its channel-slice width
};
mhla_status forward_run(mhla_handle h, const void* q, const void* k, const void* v, const float* mc, void* o,
                        void* workspace, hipStream_t s, const Intermediates* im, const PrefillHook* pf = nullptr) {
  char* ws = static_cast<char*>(workspace);
  float* ps = reinterpret_cast<float*>(ws + h->off_ps);
  float* pz = reinterpret_cast<float*>(ws + h->off_pz);
  float* pu = h->mala ? reinterpret_cast<float*>(ws + h->off_pu) : nullptr;
  uint16_t* st_hi = reinterpret_cast<uint16_t*>(ws + h->off_st_hi);
  uint16_t* st_lo = h->split ? reinterpret_cast<uint16_t*>(ws + h->off_st_lo) : nullptr;
  float* zt = reinterpret_cast<float*>(ws + h->off_zt);
  TimedLaunch* tl = nullptr;
  int ev_i = 0;
  // (the intermediates' launches are not a forward: the per-kernel timers skip them)
  if (!im && h->timing && !timer_begin(h->fwd_timer, s, tl)) return MHLA_ERR_HIP;
  auto mark = [&]() -> bool { return !tl || hipEventRecord(tl->ev[++ev_i], s) == hipSuccess; };

  const bool mix_kernel = h->mix_kernel;
  const int64_t mc_stride = h->desc.mc_per_head ? h->M * h->M : 0;

  mhla::SummaryParams sp = {};
  sp.k = k;
  sp.v = v;
  sp.sb = reinterpret_cast<uint16_t*>(ws + h->off_sb);
  sp.ps = ps;
  sp.pz = pz;
  sp.pu = pu;
  sp.g = h->geom;
  sp.splits = h->sum_splits;
  sp.tok_per_split = h->sum_tok;
  sp.mc = mc;
  sp.mc_head_stride = mc_stride;
  sp.mcf = (mix_kernel && (h->mix_mfma || h->mix_split)) ? reinterpret_cast<uint16_t*>(ws + h->off_mcf) : nullptr;
  sp.mcf_lo = (h->mix_split || h->mix_wlo) ? reinterpret_cast<uint16_t*>(ws + h->off_mcf_lo) : nullptr;
  sp.mcf_transposed = 0;
  sp.mcf_causal = h->causal ? 1 : 0;
  sp.mcf_heads = h->mcf_heads;
  sp.mcf_nitp = h->mix.nitp;
  sp.mcf_nbc = h->mix.nbc;
  hipError_t e = mhla::launch_summary(sp, h->d, h->in_fp32, h->split, h->split_v, h->mala,
                                      h->mix_mfma, (int)h->desc.phi, (int)(h->sum_splits * h->M * h->BH), s);
  if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
  if (im) {   // the block summaries, before a mixing in place overwrites them
    const int64_t rows = h->BH * h->M;
    e = h->mix_mfma ? mhla::launch_frag_to_rowmajor(sp.sb, nullptr, nullptr, 1, rows, h->d, h->frag, im->S, s)
                    : mhla::launch_frag_to_rowmajor(nullptr, nullptr, ps, h->sum_splits, rows, h->d, h->frag, im->S, s);
    if (e == hipSuccess) e = mhla::launch_sum_splits(pz, h->sum_splits, rows, h->d, im->z, s);
    if (e != hipSuccess) return MHLA_ERR_HIP;
    if (!im->St) return MHLA_OK;
  }

  if (mix_kernel) {
    if (h->mix_mfma || h->mix_split) {
      mhla::MixMfmaParams mm = {};
      mm.x = sp.sb;
      mm.xf = ps;
      mm.xsplits = h->sum_splits;
      mm.z = pz;
      mm.zsplits = h->mix_split ? h->sum_splits : 1;
      mm.mcf = reinterpret_cast<const uint16_t*>(ws + h->off_mcf);
      mm.mcf_lo = reinterpret_cast<const uint16_t*>(ws + h->off_mcf_lo);
      mm.mcf_per_head = h->desc.mc_per_head ? 1 : 0;
      mm.y = st_hi;
      mm.y_lo = reinterpret_cast<uint16_t*>(ws + h->off_st_lo);
      mm.zt = zt;
      mm.M = (int32_t)h->M;
      mm.H = (int32_t)h->H;
      mm.D = h->d;
      mm.frag = h->frag;
      e = mhla::launch_mix_mfma(mm, (int)h->BH, h->mix_split, h->mix_wlo, s);
    } else {
      mhla::MixParams mp;
      mp.ps = ps;
      mp.pz = pz;
      mp.pu = pu;
      mp.mc = mc;          // NULL only when M == 1: the kernel then uses the weight 1
      mp.mc_head_stride = mc_stride;
      mp.st_hi = st_hi;
      mp.st_lo = st_lo;
      mp.zt = zt;
      mp.M = (int32_t)h->M;
      mp.splits = h->sum_splits;
      mp.H = (int32_t)h->H;
      mp.N = (int32_t)h->N;
      mp.zsplits = h->sum_splits;
      mp.mc_transposed = 0;
      mp.causal = h->causal ? 1 : 0;
      e = mhla::launch_mix(mp, h->d, h->frag, (int)h->BH, h->split, s);
    }
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
  }
  if (im) {   // the mixed summaries (hi + lo when the mixing leaves low parts)
    const int64_t rows = h->BH * h->M;
    const bool lo = h->split || h->mix_split;
    e = mhla::launch_frag_to_rowmajor(st_hi, lo ? reinterpret_cast<const uint16_t*>(ws + h->off_st_lo) : nullptr,
                                      nullptr, 1, rows, h->d, h->frag, im->St, s);
    if (e == hipSuccess) e = hipMemcpyAsync(im->zt, zt, (size_t)rows * h->d * 4, hipMemcpyDeviceToDevice, s);
    return e == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
  }

  if (pf) {   // (split accuracy: fp32 partials, and a mixing with low parts when there is one)
    mhla::PrefillStateParams pp = {};
    pp.state = pf->state;
    pp.part = ps;
    pp.pz = pz;
    pp.st_hi = mix_kernel ? st_hi : nullptr;
    pp.st_lo = mix_kernel ? reinterpret_cast<const uint16_t*>(ws + h->off_st_lo) : nullptr;
    pp.zt = mix_kernel ? zt : nullptr;
    pp.splits = h->sum_splits;
    pp.BH = (int32_t)h->BH;
    pp.Mp = (int32_t)h->M;
    pp.M = (int32_t)pf->M;
    pp.frag = h->frag;
    pp.log2_c = pf->log2_c;
    e = mhla::launch_prefill_state(pp, h->d, s);
    if (e != hipSuccess) return MHLA_ERR_HIP;
  }

  if (h->causal) {
    const int64_t rows = h->BH * h->M;
    if (h->sum_splits > 1) {   // partials -> exclusive prefix over the block's token slices
      e = mhla::launch_slice_prefix(ps, pz, rows, h->sum_splits, h->frag, h->d, s);
      if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
    }
    mhla::CausalParams cp = {};
    cp.q = q;
    cp.k = k;
    cp.v = v;
    cp.o = o;
    cp.st_hi = mix_kernel ? st_hi : nullptr;
    cp.st_lo = mix_kernel && (h->split || h->mix_split) ? reinterpret_cast<const uint16_t*>(ws + h->off_st_lo)
                                                       : nullptr;   // bf16 mixing: no low parts
    cp.zt = mix_kernel ? zt : nullptr;
    cp.pre = h->sum_splits > 1 ? ps : nullptr;
    cp.prez = h->sum_splits > 1 ? pz : nullptr;
    cp.mc = mc;
    cp.mc_head_stride = mc_stride;
    cp.H = (int32_t)h->H;
    cp.g = h->geom;
    cp.splits = h->rd_splits;
    cp.tok_per_split = h->rd_tok;
    cp.BH = (int32_t)h->BH;
    cp.xcd_map = (h->BH % 8 == 0) ? 1 : 0;
    cp.normalized = h->mode == MHLA_READOUT_CAUSAL_NORMALIZED ? 1 : 0;
    cp.split = h->causal_split ? 1 : 0;
    e = mhla::launch_causal(cp, h->d, h->in_fp32, h->out_fp32, (int)h->desc.phi,
                            (int)(h->rd_splits * h->M * h->BH), s);
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
    return MHLA_OK;
  }

  mhla::ReadoutParams rp;
  rp.q = q;
  rp.o = o;
  rp.st_hi = st_hi;
  rp.st_lo = h->rd_split ? st_lo : nullptr;
  rp.zt = zt;
  rp.g = h->geom;
  rp.splits = h->rd_splits;
  rp.tok_per_split = h->rd_tok;
  rp.BH = (int32_t)h->BH;
  rp.xcd_map = (h->BH % 8 == 0) ? 1 : 0;
  rp.sb = sp.sb;
  rp.ps = ps;
  rp.pz = pz;
  rp.pu = pu;
  rp.mc = mc;
  rp.mc_head_stride = mc_stride;
  rp.H = (int32_t)h->H;
  rp.ssplits = h->sum_splits;
  e = mhla::launch_readout(rp, h->d, h->in_fp32, h->out_fp32, h->mode, h->rd_split, h->fuse, h->q_stream,
                           (int)h->desc.phi, (int)(h->rd_splits * h->M * h->BH), s);
  if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
  return MHLA_OK;
}

}  // namespace

extern "C" {

mhla_status mhla_forward(mhla_handle h, const void* q, const void* k, const void* v,
                         const float* mc, void* o, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!h || !q || !k || !v || !o) return MHLA_ERR_INVALID_ARG;
  if (!mc && h->M != 1) return MHLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return MHLA_ERR_INVALID_ARG;
  if (mc && !aligned(mc, 4)) return MHLA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v || (workspace && o == workspace)) return MHLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < h->ws_bytes) return MHLA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHLA_ERR_WORKSPACE;
  try {
    return forward_run(h, q, k, v, mc, o, workspace, reinterpret_cast<hipStream_t>(stream), nullptr);
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

mhla_status mhla_forward_intermediates(mhla_handle h, const void* k, const void* v, const float* mc, float* S,
                                       float* z, float* St, float* zt, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!h || !k || !v || !S || !z || (!St) != (!zt)) return MHLA_ERR_INVALID_ARG;
  if (!mc && h->M != 1) return MHLA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || (mc && !aligned(mc, 4))) return MHLA_ERR_INVALID_ARG;
  if (!aligned(S, 4) || !aligned(z, 4) || (St && (!aligned(St, 4) || !aligned(zt, 4)))) return MHLA_ERR_INVALID_ARG;
  if (St && !h->mix_kernel) return MHLA_ERR_UNSUPPORTED;   // mixed inside the readout: no mixed stack
  if (!workspace || workspace_bytes < h->ws_bytes) return MHLA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHLA_ERR_WORKSPACE;
  try {
    const Intermediates im = {S, z, St, zt};
    return forward_run(h, nullptr, k, v, mc, nullptr, workspace, reinterpret_cast<hipStream_t>(stream), &im);
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

namespace {

// Backward workspace: forward summaries recomputed at split precision, the backward's own
// summaries, g, and the per-(batch, head) dM_c partials.
struct BwdLayout {
  size_t ps, pz, st_hi, st_lo, zt, dps, dpzs, ds_hi, ds_lo, dz, tok_scale, tok_zw, dmcp;
  size_t pu, ub, du_part, du;                        // MALA: u partials, u / N, du partials, du
  size_t mcf_hi, mcf_lo, mcft_hi, mcft_lo, total;   // M_c and M_c^T operand fragments
  bool mfma_mix;                                     // M <= 256: mixing on MFMA
  mhla::MixShape mix;
  // dM_c: groups (H for a per-head M_c, else 1) x chunks of the (batch-head, position) steps
  int dmc_groups, dmc_group_bh, dmc_steps_per_bh, dmc_nchunks, dmc_steps_per_chunk;
};

// saved: the forward's summaries (and, unless MALA, its mixed summaries) come from the forward's
// workspace (mhla_backward_saved), so they take no room here.
BwdLayout bwd_layout(const mhla_plan* h, bool saved = false) {
  BwdLayout L;
  const size_t f = (size_t)h->frag, dd = (size_t)h->d;
  const size_t rows = (size_t)h->BH * h->M;
  const size_t slots = rows * h->sum_splits;
  const size_t own_sum = saved ? 0 : 1, own_mix = saved && !h->mala ? 0 : 1;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) { at = off; off = align256(off + bytes); };
  take(L.ps, own_sum * slots * f * 4);
  take(L.pz, own_sum * slots * dd * 4);
  take(L.st_hi, own_mix * rows * f * 2);
  take(L.st_lo, own_mix * rows * f * 2);
  take(L.zt, own_mix * rows * dd * 4);
  take(L.dps, slots * f * 4);
  take(L.dpzs, slots * dd * 4);
  take(L.ds_hi, rows * f * 2);
  take(L.ds_lo, rows * f * 2);
  take(L.dz, rows * dd * 4);
  take(L.tok_scale, (size_t)h->BH * h->N * 4);
  take(L.tok_zw, (size_t)h->BH * h->N * 4);
  const size_t mala_rows = h->mala ? rows : 0;
  take(L.pu, own_sum * mala_rows * h->sum_splits * dd * 4);
  take(L.ub, mala_rows * dd * 4);
  take(L.du_part, mala_rows * h->rd_splits * dd * 4);
  take(L.du, mala_rows * dd * 4);
  {
    L.dmc_groups = h->desc.mc_per_head ? (int)h->H : 1;
    L.dmc_group_bh = h->desc.mc_per_head ? (int)h->B : (int)h->BH;
    L.dmc_steps_per_bh = (h->frag + h->d + 63) / 64;   // 64-position steps (the last one padded)
    const int64_t total = (int64_t)L.dmc_group_bh * L.dmc_steps_per_bh;
    const int64_t tile = mhla::dmc_tile((int)h->M), t = (h->M + tile - 1) / tile;
    // one round of workgroups: two 8-wave workgroups per CU (128 x 128 tiles), four 4-wave ones
    // (64 x 64); each chunk then has as many steps as the work allows and the partials to
    // reduce are fewest
    const int64_t want = tile == 128 ? 512 : 1024;
    int64_t n = (want + t * t * L.dmc_groups - 1) / (t * t * L.dmc_groups);
    if (n > total) n = total;
    if (n < 1) n = 1;
    const int64_t spc = (total + n - 1) / n;
    L.dmc_steps_per_chunk = (int)spc;
    L.dmc_nchunks = (int)((total + spc - 1) / spc);
  }
  take(L.dmcp, h->mala ? 0 : (size_t)L.dmc_groups * L.dmc_nchunks * h->M * h->M * 4);
  L.mfma_mix = !h->mala && h->M <= 256;   // MALA (one block) has no mixing
  L.mix = mhla::mix_shape((int)h->M, true);
  const size_t fb = L.mfma_mix ? (size_t)h->mcf_heads * L.mix.nitp * L.mix.nbc * 512 * 2 : 0;
  take(L.mcf_hi, saved ? 0 : fb);   // the forward mixing's operands: only when it is recomputed
  take(L.mcf_lo, saved ? 0 : fb);
  take(L.mcft_hi, fb);
  take(L.mcft_lo, fb);
  L.total = off;
  return L;
}

mhla_status bwd_supported(const mhla_plan* h) {
  if (h->causal) return MHLA_ERR_UNSUPPORTED;   // no causal backward here
  if (h->d < 32) return MHLA_ERR_UNSUPPORTED;   // head sizes 32, 64, 128
  return MHLA_OK;
}

// The backward can take the forward's summaries when they are the fp32 partials it would compute
// (split operands) and, unless MALA (whose centring runs in the backward), its mixed summaries
// when the forward keeps a mixed stack (a mixing kernel of its own).
mhla_status bwd_saved_supported(const mhla_plan* h) {
  const mhla_status st = bwd_supported(h);
  if (st != MHLA_OK) return st;
  if (!h->split) return MHLA_ERR_UNSUPPORTED;
  if (!h->mala && !h->mix_kernel) return MHLA_ERR_UNSUPPORTED;
  return MHLA_OK;
}

}  // namespace

mhla_status mhla_backward_workspace_size(mhla_handle h, size_t* bytes) {
  if (!h || !bytes) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = bwd_supported(h);
  if (st != MHLA_OK) return st;
  *bytes = bwd_layout(h).total;
  return MHLA_OK;
}

// fwd: the forward's workspace (mhla_backward_saved) or NULL (recompute the forward's steps)
static mhla_status backward_impl(mhla_handle h, const void* q, const void* k, const void* v, const float* mc,
                                 const void* dout, void* dq, void* dk, void* dv, float* dmc, const char* fwd,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !q || !k || !v || !dout || !dq || !dk || !dv) return MHLA_ERR_INVALID_ARG;
  const bool saved = fwd != nullptr;
  const mhla_status st = saved ? bwd_saved_supported(h) : bwd_supported(h);
  if (st != MHLA_OK) return st;
  if (!mc && h->M != 1) return MHLA_ERR_INVALID_ARG;
  if (h->mala && dmc) return MHLA_ERR_INVALID_ARG;   // MALA has no M_c
  const void* ins[] = {q, k, v, dout};
  void* outs[] = {dq, dk, dv};
  for (const void* a : ins)
    if (!aligned(a, 16)) return MHLA_ERR_INVALID_ARG;
  for (void* a : outs) {
    if (!aligned(a, 16)) return MHLA_ERR_INVALID_ARG;
    for (const void* b : ins)
      if (a == b) return MHLA_ERR_INVALID_ARG;
    if (workspace && a == workspace) return MHLA_ERR_INVALID_ARG;
  }
  if (dq == dk || dq == dv || dk == dv) return MHLA_ERR_INVALID_ARG;
  if (mc && !aligned(mc, 4)) return MHLA_ERR_INVALID_ARG;
  if (dmc && !aligned(dmc, 4)) return MHLA_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(h, saved);
  if (!workspace || workspace_bytes < L.total) return MHLA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MHLA_ERR_WORKSPACE;
  try {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    auto U16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
    // the forward's summaries (fp32 slice partials) and mixed summaries (hi, lo, fp32 z~): from the
    // forward's workspace when saved (MALA: its C comes from the staging kernel below), else here
    char* fw = const_cast<char*>(fwd);
    float* ps = saved ? reinterpret_cast<float*>(fw + h->off_ps) : F(L.ps);
    float* pz = saved ? reinterpret_cast<float*>(fw + h->off_pz) : F(L.pz);
    float* pu = !h->mala ? nullptr : saved ? reinterpret_cast<float*>(fw + h->off_pu) : F(L.pu);
    const bool fwd_mix = saved && !h->mala;
    uint16_t* st_hi = fwd_mix ? reinterpret_cast<uint16_t*>(fw + h->off_st_hi) : U16(L.st_hi);
    uint16_t* st_lo = fwd_mix ? reinterpret_cast<uint16_t*>(fw + h->off_st_lo) : U16(L.st_lo);
    float* zt = fwd_mix ? reinterpret_cast<float*>(fw + h->off_zt) : F(L.zt);
    const int64_t mc_stride = h->desc.mc_per_head ? h->M * h->M : 0;
    const int phi = (int)h->desc.phi;
    const int units_sum = (int)(h->sum_splits * h->M * h->BH);
    const int units_rd = (int)(h->rd_splits * h->M * h->BH);
    TimedLaunch* tl = nullptr;
    int ev_i = 0;
    if (h->timing && !timer_begin(h->bwd_timer, s, tl)) return MHLA_ERR_HIP;
    auto mark = [&]() -> bool { return !tl || hipEventRecord(tl->ev[++ev_i], s) == hipSuccess; };

    // 1-2. the forward's summaries and mixed summaries at split precision
    mhla::SummaryParams sp = {};
    sp.k = k;
    sp.v = v;
    sp.ps = ps;
    sp.pz = pz;
    sp.g = h->geom;
    sp.splits = h->sum_splits;
    sp.tok_per_split = h->sum_tok;
    if (L.mfma_mix) {   // side job: M_c operand fragments (hi, lo) for the mixing kernel
      sp.mc = mc;
      sp.mc_head_stride = mc_stride;
      sp.mcf = U16(L.mcf_hi);
      sp.mcf_lo = U16(L.mcf_lo);
      sp.mcf_transposed = 0;
      sp.mcf_heads = h->mcf_heads;
      sp.mcf_nitp = L.mix.nitp;
      sp.mcf_nbc = L.mix.nbc;
    }
    if (h->mala) sp.pu = pu;
    hipError_t e = saved ? hipSuccess
                         : mhla::launch_summary(sp, h->d, h->in_fp32, true, h->in_fp32, h->mala, false, phi,
                                                units_sum, s);
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;
    // MALA: C = S - z u^T / N, z, u / N (stage 0); dS, dz = dz' - dS u / N, du (stage 1)
    auto mala_stage = [&](int stage) -> hipError_t {
      mhla::MalaStageParams mp = {};
      mp.ps = stage == 0 ? ps : F(L.dps);
      mp.pz = stage == 0 ? pz : F(L.dpzs);
      mp.pu = pu;
      mp.ub = F(L.ub);
      mp.du_part = F(L.du_part);
      mp.y_hi = stage == 0 ? st_hi : U16(L.ds_hi);
      mp.y_lo = stage == 0 ? st_lo : U16(L.ds_lo);
      mp.zo = stage == 0 ? zt : F(L.dz);
      mp.ub_out = F(L.ub);
      mp.du = F(L.du);
      mp.ss = h->sum_splits;
      mp.rs = h->rd_splits;
      mp.N = (int32_t)h->N;
      mp.stage = stage;
      return mhla::launch_mala_stage(mp, h->d, (int)h->BH, s);
    };
    // mixing with W = M_c (mc_transposed = 0) or M_c^T (1): S~ = M_c S, then dS = M_c^T dS~
    auto mix = [&](const float* xs, const float* zs, int zsplits, int transposed, uint16_t* y_hi,
                   uint16_t* y_lo, float* zo) -> hipError_t {
      if (L.mfma_mix) {
        mhla::MixMfmaParams mm = {};
        mm.xf = xs;
        mm.xsplits = h->sum_splits;
        mm.z = zs;
        mm.zsplits = zsplits;
        mm.mcf = U16(transposed ? L.mcft_hi : L.mcf_hi);
        mm.mcf_lo = U16(transposed ? L.mcft_lo : L.mcf_lo);
        mm.mcf_per_head = h->desc.mc_per_head ? 1 : 0;
        mm.y = y_hi;
        mm.y_lo = y_lo;
        mm.zt = zo;
        mm.M = (int32_t)h->M;
        mm.H = (int32_t)h->H;
        mm.D = h->d;
        mm.frag = h->frag;
        return mhla::launch_mix_mfma(mm, (int)h->BH, true, false, s);
      }
      mhla::MixParams mp = {};
      mp.ps = xs;
      mp.pz = zs;
      mp.mc = mc;
      mp.mc_head_stride = mc_stride;
      mp.st_hi = y_hi;
      mp.st_lo = y_lo;
      mp.zt = zo;
      mp.M = (int32_t)h->M;
      mp.splits = h->sum_splits;
      mp.H = (int32_t)h->H;
      mp.N = (int32_t)h->N;
      mp.zsplits = zsplits;
      mp.mc_transposed = transposed;
      return mhla::launch_mix(mp, h->d, h->frag, (int)h->BH, true, s);
    };
    e = h->mala ? mala_stage(0) : fwd_mix ? hipSuccess : mix(ps, pz, h->sum_splits, 0, st_hi, st_lo, zt);
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;

    // 3. query side: dq, g, dz~ partials
    mhla::BwdParams bp = {};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.dout = dout;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.st_hi = st_hi;
    bp.st_lo = st_lo;
    bp.zt = zt;
    bp.ds_hi = U16(L.ds_hi);
    bp.ds_lo = U16(L.ds_lo);
    bp.dz = F(L.dz);
    bp.tok_scale = F(L.tok_scale);
    bp.tok_zw = F(L.tok_zw);
    bp.du_part = h->mala ? F(L.du_part) : nullptr;
    bp.du = nullptr;                                    // set for the key side below
    bp.g = h->geom;
    bp.splits = h->rd_splits;
    bp.tok_per_split = h->rd_tok;
    bp.BH = (int32_t)h->BH;
    bp.xcd_map = (h->BH % 8 == 0) ? 1 : 0;
    if ((e = mhla::launch_bwd_tiles(bp, h->d, h->in_fp32, h->out_fp32, h->mode, phi, false, units_rd, s)) !=
            hipSuccess ||
        !mark())
      return MHLA_ERR_HIP;

    // 4. dS~ = sum_t (q~_t / den_t) dO_t^T and dz~ = sum_t q~_t gden_t: the summary kernel with
    //    K := Q scaled per token by 1/den, V := dO, normaliser weights -(dO . o)
    mhla::SummaryParams sq = sp;
    sq.k = q;
    sq.v = dout;
    sq.pu = nullptr;
    sq.ps = F(L.dps);
    sq.pz = F(L.dpzs);
    sq.kscale = F(L.tok_scale);
    sq.zw = F(L.tok_zw);
    if (L.mfma_mix) {   // side job: M_c^T operand fragments for the transposed mixing
      sq.mcf = U16(L.mcft_hi);
      sq.mcf_lo = U16(L.mcft_lo);
      sq.mcf_transposed = 1;
    }
    e = mhla::launch_summary_tokw(sq, h->d, h->in_fp32, h->out_fp32, phi, units_sum, s);
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;

    // 5. dS = M_c^T dS~, dz = M_c^T dz~
    e = h->mala ? mala_stage(1) : mix(F(L.dps), F(L.dpzs), h->sum_splits, 1, U16(L.ds_hi), U16(L.ds_lo), F(L.dz));
    if (e != hipSuccess || !mark()) return MHLA_ERR_HIP;

    // 6. key side: dk, dv
    bp.du = h->mala ? F(L.du) : nullptr;
    if ((e = mhla::launch_bwd_tiles(bp, h->d, h->in_fp32, h->out_fp32, h->mode, phi, true, units_rd, s)) !=
            hipSuccess ||
        !mark())
      return MHLA_ERR_HIP;

    // 7. dM_c
    if (dmc) {
      mhla::DmcParams dp = {};
      dp.dps = F(L.dps);
      dp.ps = ps;
      dp.dpz = F(L.dpzs);
      dp.pz = pz;
      dp.out = F(L.dmcp);
      dp.M = (int32_t)h->M;
      dp.frag = h->frag;
      dp.D = h->d;
      dp.ssplits = h->sum_splits;
      dp.zsplits_d = h->sum_splits;
      dp.H = (int32_t)h->H;
      dp.per_head = h->desc.mc_per_head ? 1 : 0;
      dp.group_bh = L.dmc_group_bh;
      dp.steps_per_bh = L.dmc_steps_per_bh;
      dp.nchunks = L.dmc_nchunks;
      dp.steps_per_chunk = L.dmc_steps_per_chunk;
      if ((e = mhla::launch_dmc(dp, dmc, s)) != hipSuccess) return MHLA_ERR_HIP;
    }
    if (!mark()) return MHLA_ERR_HIP;
    return MHLA_OK;
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

mhla_status mhla_backward(mhla_handle h, const void* q, const void* k, const void* v, const float* mc,
                          const void* dout, void* dq, void* dk, void* dv, float* dmc, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return backward_impl(h, q, k, v, mc, dout, dq, dk, dv, dmc, nullptr, workspace, workspace_bytes, stream);
}

mhla_status mhla_backward_saved_workspace_size(mhla_handle h, size_t* bytes) {
  if (!h || !bytes) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = bwd_saved_supported(h);
  if (st != MHLA_OK) return st;
  *bytes = bwd_layout(h, true).total;
  return MHLA_OK;
}

mhla_status mhla_backward_saved(mhla_handle h, const void* q, const void* k, const void* v, const float* mc,
                                const void* dout, void* dq, void* dk, void* dv, float* dmc,
                                const void* fwd_workspace, size_t fwd_workspace_bytes, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!h) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = bwd_saved_supported(h);
  if (st != MHLA_OK) return st;
  if (!fwd_workspace) return MHLA_ERR_INVALID_ARG;
  if (fwd_workspace_bytes < h->ws_bytes || !aligned(fwd_workspace, 256)) return MHLA_ERR_WORKSPACE;
  // the forward's workspace is read: no output and no part of this call's workspace may overlap it
  const char* f0 = static_cast<const char*>(fwd_workspace);
  const char* f1 = f0 + h->ws_bytes;
  for (const void* a : {(const void*)dq, (const void*)dk, (const void*)dv, (const void*)dmc})
    if (a && static_cast<const char*>(a) >= f0 && static_cast<const char*>(a) < f1) return MHLA_ERR_INVALID_ARG;
  if (workspace) {
    const char* w0 = static_cast<const char*>(workspace);
    const char* w1 = w0 + workspace_bytes;
    if (w0 < f1 && f0 < w1) return MHLA_ERR_INVALID_ARG;
  }
  return backward_impl(h, q, k, v, mc, dout, dq, dk, dv, dmc, f0, workspace, workspace_bytes, stream);
}

// ---- streaming decode --------------------------------------------------------------------
static mhla_status decode_supported(const mhla_plan* h) {
  if (!h->causal) return MHLA_ERR_UNSUPPORTED;
  return MHLA_OK;
}
// channels per decode workgroup, as log2: the head's d channels are cut into the fewest slices
// (powers of two, each of at least max(8, 1024 / d) channels) that give 512 workgroups over all
// (batch, head) pairs
static int decode_log2_c(const mhla_plan* h) {
  const int min_c = h->d >= 128 ? 8 : 1024 / h->d;
  int slices = 1;
  while (h->BH * slices < 512 && h->d / (slices * 2) >= min_c) slices *= 2;
  int lc = 0;
  while ((slices << lc) < h->d) ++lc;
  return lc;
}
static size_t decode_state_bytes(const mhla_plan* h) {
  const size_t slices = (size_t)h->d >> decode_log2_c(h);
  return (size_t)h->BH * (size_t)(h->M + 2) * ((size_t)h->d * h->d + slices * h->d) * 4;
}

mhla_status mhla_decode_state_size(mhla_handle h, size_t* bytes) {
  if (!h || !bytes) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = decode_supported(h);
  if (st != MHLA_OK) return st;
  *bytes = decode_state_bytes(h);
  return MHLA_OK;
}

mhla_status mhla_decode_reset(mhla_handle h, void* state, size_t state_bytes, void* stream) {
  if (!h || !state) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = decode_supported(h);
  if (st != MHLA_OK) return st;
  if (state_bytes < decode_state_bytes(h) || !aligned(state, 256)) return MHLA_ERR_WORKSPACE;
  const hipError_t e = mhla::launch_decode_zero(static_cast<float*>(state), (int64_t)(decode_state_bytes(h) / 4),
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
}

mhla_status mhla_decode_step(mhla_handle h, void* state, size_t state_bytes, int64_t t, const void* q,
                             const void* k, const void* v, const float* mc, void* o, void* stream) {
  if (!h || !state || !q || !k || !v || !o) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = decode_supported(h);
  if (st != MHLA_OK) return st;
  if (t < 0 || t >= h->N) return MHLA_ERR_INVALID_ARG;
  if (!mc && h->M != 1) return MHLA_ERR_INVALID_ARG;
  const size_t ein = h->in_fp32 ? 4 : 2, eout = h->out_fp32 ? 4 : 2;
  if (!aligned(q, ein) || !aligned(k, ein) || !aligned(v, ein) || !aligned(o, eout)) return MHLA_ERR_INVALID_ARG;
  if (mc && !aligned(mc, 4)) return MHLA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v || o == state) return MHLA_ERR_INVALID_ARG;
  if (state_bytes < decode_state_bytes(h) || !aligned(state, 256)) return MHLA_ERR_WORKSPACE;
  try {
    mhla::DecodeParams p = {};
    p.state = static_cast<float*>(state);
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.mc = mc;
    p.mc_head_stride = h->desc.mc_per_head ? h->M * h->M : 0;
    p.t = t;
    p.H = (int32_t)h->H;
    p.M = (int32_t)h->M;
    p.nb = (int32_t)h->n_b;
    p.BH = (int32_t)h->BH;
    p.normalized = h->mode == MHLA_READOUT_CAUSAL_NORMALIZED ? 1 : 0;
    p.log2_c = decode_log2_c(h);
    p.cls = h->geom.cls;
    const hipError_t e = mhla::launch_decode_step(p, h->d, h->in_fp32, h->out_fp32, (int)h->desc.phi,
                                                  reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? MHLA_OK : MHLA_ERR_HIP;
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

namespace {

// A prefill's own plan: positions 0 .. n-1 of h's sequence as a causal plan (the last block cut
// short where n ends inside it) whose summaries and mixing are at split accuracy, so that the
// state it leaves is fp32-exact as a decode step's, and whose in-slice products are at the decode
// plan's accuracy; its workspace, then a copy of the leading Mp x Mp part of M_c (per head if M_c
// is).
mhla_status prefill_plan(const mhla_plan* h, int64_t n, mhla_plan* sub, size_t* mc_off, size_t* total) {
  mhla_desc d = h->desc;
  d.grid[0] = n - h->geom.cls;
  d.flags |= MHLA_FLAG_RAGGED_BLOCKS;
  d.accuracy = MHLA_ACCURACY_SPLIT;
  const mhla_status st = build_plan(&d, sub);
  if (st != MHLA_OK) return st;
  sub->causal_split = h->split;   // the outputs at the decode plan's own accuracy
  const size_t heads = h->desc.mc_per_head ? (size_t)h->H : 1;
  *mc_off = sub->ws_bytes;
  *total = align256(sub->ws_bytes + heads * (size_t)sub->M * (size_t)sub->M * 4);
  return MHLA_OK;
}

bool prefill_supported(const mhla_plan* h, int64_t n) {
  // a prefix of at least one grid token (a prefix of the CLS token alone is one decode step)
  return h->causal && n - h->geom.cls >= 1 && n <= h->N;
}

}  // namespace

mhla_status mhla_decode_prefill_workspace_size(mhla_handle h, int64_t n, size_t* bytes) {
  if (!h || !bytes) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = decode_supported(h);
  if (st != MHLA_OK) return st;
  if (n < 1 || n > h->N) return MHLA_ERR_INVALID_ARG;
  if (!prefill_supported(h, n)) {
    *bytes = 0;
    return MHLA_OK;
  }
  try {
    mhla_plan sub;
    size_t mc_off = 0, total = 0;
    const mhla_status s2 = prefill_plan(h, n, &sub, &mc_off, &total);
    if (s2 != MHLA_OK) return s2;
    *bytes = total;
    return MHLA_OK;
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

mhla_status mhla_decode_prefill(mhla_handle h, void* state, size_t state_bytes, int64_t n, const void* q,
                                const void* k, const void* v, const float* mc, void* o, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!h || !state || !q || !k || !v || !o) return MHLA_ERR_INVALID_ARG;
  const mhla_status st = decode_supported(h);
  if (st != MHLA_OK) return st;
  if (n < 1 || n > h->N) return MHLA_ERR_INVALID_ARG;
  if (!mc && h->M != 1) return MHLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return MHLA_ERR_INVALID_ARG;
  if (mc && !aligned(mc, 4)) return MHLA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v || o == state || (workspace && (o == workspace || state == workspace)))
    return MHLA_ERR_INVALID_ARG;
  if (state_bytes < decode_state_bytes(h) || !aligned(state, 256)) return MHLA_ERR_WORKSPACE;
  try {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!prefill_supported(h, n)) {
      // the CLS token alone: one decode step on a cleared state
      const hipError_t e = mhla::launch_decode_zero(static_cast<float*>(state), (int64_t)(decode_state_bytes(h) / 4), s);
      if (e != hipSuccess) return MHLA_ERR_HIP;
      return mhla_decode_step(h, state, state_bytes, 0, q, k, v, mc, o, stream);
    }
    mhla_plan sub;
    size_t mc_off = 0, total = 0;
    const mhla_status s2 = prefill_plan(h, n, &sub, &mc_off, &total);
    if (s2 != MHLA_OK) return s2;
    if (!workspace || workspace_bytes < total) return MHLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MHLA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    // the prefix's M_c: the leading Mp x Mp block of every head's M x M
    float* mc_sub = nullptr;
    if (mc) {
      mc_sub = reinterpret_cast<float*>(ws + mc_off);
      const int64_t heads = h->desc.mc_per_head ? h->H : 1, Mp = sub.M, M = h->M;
      for (int64_t hh = 0; hh < heads; ++hh)
        if (hipMemcpy2DAsync(mc_sub + hh * Mp * Mp, (size_t)Mp * 4, mc + hh * M * M, (size_t)M * 4, (size_t)Mp * 4,
                             (size_t)Mp, hipMemcpyDeviceToDevice, s) != hipSuccess)
          return MHLA_ERR_HIP;
    }
    const PrefillHook hook = {static_cast<float*>(state), h->M, decode_log2_c(h)};
    return forward_run(&sub, q, k, v, mc_sub, o, workspace, s, nullptr, &hook);
  } catch (...) {
    return MHLA_ERR_INTERNAL;
  }
}

mhla_status mhla_destroy(mhla_handle h) {
  if (!h) return MHLA_OK;
  for (PassTimer* t : {&h->fwd_timer, &h->bwd_timer})
    for (auto& c : t->calls)
      for (int i = 0; i <= kMaxTimedKernels; ++i) (void)hipEventDestroy(c.ev[i]);
  delete h;
  return MHLA_OK;
}

const char* mhla_status_string(mhla_status s) {
  switch (s) {
    case MHLA_OK: return "success";
    case MHLA_ERR_INVALID_ARG: return "invalid argument";
    case MHLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MHLA_ERR_SHAPE: return "inconsistent or unsupported shape";
    case MHLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MHLA_ERR_HIP: return "HIP runtime or launch failure";
    case MHLA_ERR_INTERNAL: return "internal error";
    case MHLA_ERR_SCRATCH_LIMIT: return "workspace larger than the no-alloc entry point's scratch array";
    default: return "unknown status";
  }
}

mhla_status mhla_timing_enable(mhla_handle h, int enable) {
  if (!h) return MHLA_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return MHLA_OK;
}

mhla_status mhla_timing_read(mhla_handle h, int index, double* total_ms, int64_t* launches,
                             const char** name) {
  if (!h || index < 0 || index >= h->n_kernels) return MHLA_ERR_INVALID_ARG;
  if (name) *name = h->kernel_names[index];
  return timer_read(h->fwd_timer, index, h->n_kernels, total_ms, launches);
}

mhla_status mhla_backward_timing_read(mhla_handle h, int index, double* total_ms, int64_t* launches,
                                      const char** name) {
  if (!h || index < 0 || index >= kBwdKernels) return MHLA_ERR_INVALID_ARG;
  if (name) *name = kBwdNames[index];
  return timer_read(h->bwd_timer, index, kBwdKernels, total_ms, launches);
}

mhla_status mhla_timing_reset(mhla_handle h) {
  if (!h) return MHLA_ERR_INVALID_ARG;
  h->fwd_timer.used = 0;
  h->bwd_timer.used = 0;
  return MHLA_OK;
}

}  // extern "C"
