/*
 * mhla.h - C ABI of the MI355X (gfx950) forward of token-level multi-head linear attention.
 *
 * What is computed (page titles and sections):
 *   "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head"
 *     - Method, Overall framework: the N tokens are cut into M non-overlapping blocks (1D spans
 *       or tiles of a 2D/3D token grid); each block b has a local summary
 *       S_b = sum_{j in b} phi(K_j) V_j^T (d x d) and normaliser z_b = sum_{j in b} phi(K_j).
 *     - Key design 2 (multi-head mixing): row i of the coefficient matrix M_c (M x M) mixes
 *       the summaries for query block i: S~_i = sum_b m_ib S_b, z~_i = sum_b m_ib z_b; a query
 *       q in block i reads out o = phi(q)^T S~_i / phi(q)^T z~_i (flowchart).  The same section
 *       allows the normaliser to be dropped for long sequences (UNNORMALIZED readout).
 *   "Rectifying Magnitude Neglect in Linear Attention"
 *     - Method, Key design (MALA formula design): with one block (M = 1),
 *       Y_i = beta_i phi(Q_i) sum_j phi(K_j)^T V_j - gamma_i sum_j V_j,
 *       beta_i = 1 + 1/(phi(Q_i) sum_m phi(K_m)^T), gamma_i = phi(Q_i) sum_m phi(K_m)^T / N.
 *   phi is ELU+1 (alpha = 1): x + 1 for x > 0, exp(x) otherwise.  No 1/sqrt(d) scaling is applied.
 *
 * Conventions
 *   - Q, K, V, O are dense [B, H, N, d] row-major (d fastest), device memory, 16-byte aligned.
 *   - Tokens are in raster order over the token grid, last axis fastest.  Blocks are numbered
 *     in raster order over the block grid; block extents must divide the grid exactly.
 *   - M_c is float32 row-major, device memory: [M, M] shared by all heads, or [H, M, M] when
 *     mc_per_head = 1.  Row i belongs to query block i.  M_c may be NULL only when M == 1.
 *   - d (head_dim) is one of 16, 32, 64, 128 and is the same for keys and values.
 *
 * Ownership and concurrency
 *   - The caller owns every device buffer (Q, K, V, M_c, O, workspace).  The library owns only
 *     the host-side plan; it never allocates device memory.
 *   - Inputs are read-only.  O must not alias Q, K, V or the workspace (exact aliasing is
 *     rejected; partial overlap is undefined).
 *   - mhla_forward is asynchronous on the given HIP stream (NULL = default stream).  One
 *     (plan, workspace) pair may be in flight on one stream at a time.
 *   - mhla_forward, mhla_backward and the decode calls only launch kernels on `stream`: no
 *     allocation, memset or host synchronisation.  So they may be captured into a HIP graph,
 *     and each replay computes what the call would compute on the buffers' contents at replay
 *     time.  Per-kernel timing (mhla_timing_enable) adds event records to the captured work.
 *
 * Errors
 *   - Every call returns mhla_status; MHLA_OK is 0.  Arguments are validated before any
 *     launch; nothing is launched when a call fails validation.  A failed HIP launch returns
 *     MHLA_ERR_HIP.  NaN/Inf in the data propagate per IEEE and are not errors; there is no
 *     epsilon in any division.  The library never aborts and never throws across this ABI.
 */
#ifndef MHLA_H
#define MHLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MHLA_OK = 0,
  MHLA_ERR_INVALID_ARG = 1,   /* NULL pointer, bad struct_size, misaligned or aliased buffer   */
  MHLA_ERR_UNSUPPORTED = 2,   /* head_dim, dtype, feature map or mode not supported            */
  MHLA_ERR_SHAPE = 3,         /* grid/block extents inconsistent or not divisible              */
  MHLA_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than mhla_workspace_size            */
  MHLA_ERR_HIP = 5,           /* a HIP runtime call or kernel launch failed                    */
  MHLA_ERR_INTERNAL = 6,
  MHLA_ERR_SCRATCH_LIMIT = 7  /* mhla_forward_noalloc: the plan's workspace exceeds             */
                              /* MHLA_NOALLOC_SCRATCH_BYTES                                      */
} mhla_status;

typedef enum { MHLA_DTYPE_BF16 = 0, MHLA_DTYPE_FP32 = 1 } mhla_dtype;

/* Feature map phi applied to Q and K.  ELU+1 is the default; ReLU and exp are the other maps the
 * "Rectifying Magnitude Neglect in Linear Attention" notes find equivalent (Ablation).  Readings:
 * relu(x) = max(x, 0); exp(x) = e^x elementwise with no max subtraction.  With ReLU a query with no
 * positive feature has a zero normaliser: the IEEE result 0/0 = NaN is returned (no epsilon). */
typedef enum { MHLA_PHI_ELU1 = 0, MHLA_PHI_RELU = 1, MHLA_PHI_EXP = 2 } mhla_phi;

/* Chunkwise-causal modes ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
 * Multi-Head", Key design 4 names chunkwise-parallel training and streaming inference; the causal
 * form is a reading): the token-expanded sum of Key design 2 masked to keys t' <= t, i.e. query t
 * of block i reads sum_{b<i} m_ib S_b plus m_ii times its own block's prefix up to t; entries of
 * M_c above the diagonal are not read.  1D grids and d >= 32 only (else MHLA_ERR_UNSUPPORTED);
 * operand precision as the accuracy field says (see mhla_accuracy). */
typedef enum {
  MHLA_READOUT_NORMALIZED = 0,    /* o = phi(q)^T S~_i / phi(q)^T z~_i                         */
  MHLA_READOUT_UNNORMALIZED = 1,  /* o = phi(q)^T S~_i                                        */
  MHLA_READOUT_MALA = 2,          /* magnitude-aware readout; requires M == 1                  */
  MHLA_READOUT_CAUSAL_NORMALIZED = 3,    /* causal, normalised                                 */
  MHLA_READOUT_CAUSAL_UNNORMALIZED = 4   /* causal, no normaliser                              */
} mhla_readout;

typedef enum {
  MHLA_ACCURACY_AUTO = 0,   /* bf16 operands for MHLA with ELU+1 and bf16 inputs; split for     */
                            /* MALA, fp32 inputs and the ReLU / exp maps (whose outputs sit      */
                            /* near the 2e-2 bar with single bf16 operands)                      */
  MHLA_ACCURACY_BF16 = 1,   /* single bf16 MFMA operands, fp32 accumulation                     */
  MHLA_ACCURACY_SPLIT = 2,  /* operands not exact in bf16 are split hi + lo (about fp32 accuracy)*/
  MHLA_ACCURACY_TRAIN = 3   /* summaries and mixing as SPLIT (mhla_backward_saved reads them);   */
                            /* the readout's operands as AUTO chooses them: with a mixing kernel */
                            /* of its own, bf16 inputs and ELU+1, the mixed stack's high part    */
                            /* and single bf16 operands; elsewhere as SPLIT                      */
} mhla_accuracy;              /* The causal readouts: the field sets the summaries, the mixing of */
                              /* the earlier blocks and, for bf16 inputs, the in-slice scores and  */
                              /* the start-state readout; the weights of V (P) are always split    */
                              /* (one bf16 rounding there grows with the keys in view past the     */
                              /* 2e-2 bar).  fp32 inputs keep the running state and scores split.  */

typedef struct {
  uint32_t struct_size;     /* = sizeof(mhla_desc)                                             */
  int32_t in_dtype;         /* mhla_dtype of Q, K, V                                           */
  int32_t out_dtype;        /* mhla_dtype of O                                                 */
  int32_t phi;              /* mhla_phi                                                        */
  int32_t readout;          /* mhla_readout                                                    */
  int32_t accuracy;         /* mhla_accuracy                                                   */
  int32_t ndim;             /* 1, 2 or 3                                                       */
  int32_t mc_per_head;      /* 0: M_c is [M, M]; 1: M_c is [H, M, M]                           */
  int64_t grid[3];          /* token grid extents, first ndim used; N = product                */
  int64_t block[3];         /* block extents, first ndim used; each divides grid exactly       */
                            /* (unless MHLA_FLAG_RAGGED_BLOCKS)                                */
  int64_t batch;            /* B >= 1                                                          */
  int64_t heads;            /* H >= 1                                                          */
  int64_t head_dim;         /* d in {16, 32, 64, 128}                                          */
  int32_t flags;            /* MHLA_FLAG_* bits (0: every block whole, no CLS token)           */
  int32_t reserved;         /* must be 0                                                       */
} mhla_desc;

/* Geometry flags ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head":
 * the rank bound of Key design 1 is stated for general block sizes n_b; DeiT carries a CLS token
 * beside its patch grid).  Readings:
 *   MHLA_FLAG_RAGGED_BLOCKS  the block extents need not divide the grid: blocks tile the grid from
 *                            its origin and the last block along an axis keeps what is left
 *                            (fewer tokens); blocks are numbered in raster order over the
 *                            rounded-up block grid.  A block extent above the grid's is clipped.
 *   MHLA_FLAG_CLS_TOKEN      one extra token precedes the grid (token 0 of every head, N = 1 +
 *                            product of the grid) and forms block 0 on its own; the grid's blocks
 *                            are 1 .. M-1, and M_c is M x M with M counting the CLS block.
 * A descriptor whose struct_size is that of the earlier layout (without flags and reserved) is
 * accepted with flags = 0. */
enum { MHLA_FLAG_RAGGED_BLOCKS = 1, MHLA_FLAG_CLS_TOKEN = 2 };

typedef struct mhla_plan* mhla_handle;

/* Facts about a plan, for callers that size buffers or account bytes and FLOPs. */
typedef struct {
  uint32_t struct_size;     /* caller sets = sizeof(mhla_plan_info)                            */
  int64_t n_tokens;         /* N                                                               */
  int64_t n_blocks;         /* M                                                               */
  int64_t block_tokens;     /* n_b = N / M; with ragged blocks or a CLS token, the tokens of a  */
                            /* whole block (the most any block holds)                          */
  int64_t workspace_bytes;  /* same as mhla_workspace_size                                     */
  int32_t summary_splits;   /* token slices per block in the summary kernel                    */
  int32_t readout_splits;   /* token slices per block in the readout kernel                    */
  int32_t n_kernels;        /* kernels launched per mhla_forward: 3 (summary, mix, readout),   */
                            /* or 2 (summary, mix+readout) when the mixing step runs in the    */
                            /* readout's prologue: MALA readout, or at most 16 blocks; causal: */
                            /* summary, mix (M > 1), scan (blocks over 256 tokens), causal     */
  int32_t split_operands;   /* 1 if hi/lo operand splitting is in use                          */
} mhla_plan_info;

/* Validate a descriptor and build a host-side plan.  No device memory is allocated.
 * Errors: INVALID_ARG (NULL, struct_size), UNSUPPORTED (dtype, phi, readout, d, MALA with
 * M > 1), SHAPE (ndim, non-positive or non-dividing extents, sizes beyond 2^31 tokens). */
mhla_status mhla_create(const mhla_desc* desc, mhla_handle* out);

/* Device workspace the caller must pass to mhla_forward, in bytes (256-byte aligned start). */
mhla_status mhla_workspace_size(mhla_handle h, size_t* bytes);

/* Run the forward on `stream` (a hipStream_t, NULL = default stream).
 * q, k, v: device [B,H,N,d] of in_dtype.  o: device [B,H,N,d] of out_dtype.
 * mc: device float32 [M,M] or [H,M,M]; NULL allowed iff M == 1.
 * workspace: device, >= mhla_workspace_size bytes, 256-byte aligned; its contents on entry are
 * ignored and on return are unspecified.  Asynchronous: returns after the launches. */
mhla_status mhla_forward(mhla_handle h, const void* q, const void* k, const void* v,
                         const float* mc, void* o, void* workspace, size_t workspace_bytes,
                         void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it): mhla_forward with its workspace in a
 * fixed device array of MHLA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on (from the first call on that device until the process ends) instead of a caller buffer.
 * The array holds the workspace of every plan whose mhla_workspace_size is at most that size --
 * the 65536-token, 16-head, d = 128 sequence in 256 blocks needs 132 MiB; larger plans get
 * MHLA_ERR_SCRATCH_LIMIT and nothing is launched.  Arguments, validation and results are those
 * of mhla_forward.  The call allocates nothing; its first call on a device (the current device)
 * looks up that device's copy of the array.  Every call on a device shares that device's array:
 * calls that overlap on one device (on different streams, or from several threads) race and
 * give undefined results; calls in one stream's order are safe. */
#define MHLA_NOALLOC_SCRATCH_BYTES (160u << 20)
mhla_status mhla_forward_noalloc(mhla_handle h, const void* q, const void* k, const void* v,
                                 const float* mc, void* o, void* stream);

/* The forward's first two steps on their own, for inspecting them: the block summaries
 * S_b = sum_{j in b} phi(k_j) v_j^T, z_b = sum_{j in b} phi(k_j) ("MHLA: Restoring Expressivity of
 * Linear Attention via Token-Level Multi-Head", Overall framework) and the mixed summaries
 * S~_i = sum_b m_ib S_b, z~_i = sum_b m_ib z_b (Key design 2; for the causal readouts b < i, the
 * strictly lower part of M_c).  The plan's own summary and mixing kernels run at the plan's
 * precision on `workspace` (as for mhla_forward); their results are then written out in fp32.
 *   k, v, mc   as for mhla_forward (q is not read; nothing is written to an output tensor)
 *   S          device fp32 [B*H][M][d][d], S[bh][b][f][c] = feature f of phi(k), channel c of v
 *   z          device fp32 [B*H][M][d]
 *   St, zt     device fp32, the same shapes, for the mixed summaries; both NULL to stop after the
 *              summaries.  Non-NULL with a plan whose mixing runs inside its readout (at most 16
 *              blocks, MALA; mhla_plan_info.n_kernels == 2) or with one block in a causal plan,
 *              which keep no mixed stack: MHLA_ERR_UNSUPPORTED.
 * Values are those the forward computes and then reads: bf16 where the plan's stacks are bf16
 * (the summary of a one-slice block under bf16 operands, the mixed stack's high part), else the
 * sum of fp32 slice partials or of the hi and lo parts.  The buffers belong to the caller and must
 * not overlap the workspace.  Errors: INVALID_ARG (NULL k, v, S or z; only one of St, zt; mc NULL
 * with M > 1; misaligned pointers), WORKSPACE, UNSUPPORTED, HIP.  Asynchronous on `stream`. */
mhla_status mhla_forward_intermediates(mhla_handle h, const void* k, const void* v, const float* mc, float* S,
                                       float* z, float* St, float* zt, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Backward pass: gradients of L = sum(dout * O) with respect to Q, K, V and M_c, for the
 * normalised, unnormalised and MALA readouts (chain rule of the forward steps; M_c is trained end
 * to end per "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
 * Method -> Key design 3; MALA's beta and gamma per "Rectifying Magnitude Neglect in Linear
 * Attention", Method -> Key design, differentiated through the centred form
 * Y = u/N + beta q~^T (S - z u^T / N)).
 *   q, k, v      device, as for mhla_forward (plan's in_dtype)
 *   mc           device fp32 M_c as for mhla_forward (NULL iff M == 1)
 *   dout         device [B, H, N, d], the plan's out_dtype: dL/dO
 *   dq, dk, dv   device [B, H, N, d], the plan's out_dtype: written (not accumulated)
 *   dmc          device fp32 with M_c's shape, written; for a shared [M, M] M_c the sum over
 *                batch and heads, for a per-head [H, M, M] one the sum over batch; NULL skips it.
 *                MALA has no M_c: dmc must be NULL (else MHLA_ERR_INVALID_ARG)
 * The forward's summaries are recomputed (nothing from mhla_forward is reused; mhla_backward_saved
 * reads them from the forward's workspace instead); every product
 * uses hi/lo bf16 operand splits.  Not supported (MHLA_ERR_UNSUPPORTED): the causal readouts,
 * head size 16.  Outputs must not alias the inputs, each other or the workspace.  The workspace
 * (256-byte aligned) size comes from mhla_backward_workspace_size and differs from the
 * forward's.  Every sum runs in a fixed order: repeated calls give identical bits.
 * Asynchronous on `stream`, like mhla_forward. */
mhla_status mhla_backward_workspace_size(mhla_handle h, size_t* bytes);
mhla_status mhla_backward(mhla_handle h, const void* q, const void* k, const void* v, const float* mc,
                          const void* dout, void* dq, void* dk, void* dv, float* dmc, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Backward pass from the forward's saved state, for training: the same gradients as mhla_backward
 * (the same kernels on the same values: identical bits), without recomputing the forward's block
 * summaries S_b, z_b (and, except for MALA, its mixed summaries S~_i, z~_i), which are read from
 * the workspace of the plan's last mhla_forward call instead ("MHLA: Restoring Expressivity of
 * Linear Attention via Token-Level Multi-Head", Overall framework and Key design 2 give the
 * steps; Key design 3 trains M_c end to end).
 *   q, k, v, mc, dout, dq, dk, dv, dmc   as for mhla_backward; q, k, v and mc must be those of
 *                 that forward call, whose results are only as valid as this requirement
 *   fwd_workspace the workspace of that mhla_forward call on this plan, unchanged since (device,
 *                 256-byte aligned, at least mhla_workspace_size bytes, given as fwd_workspace_bytes);
 *                 only read
 *   workspace     device, mhla_backward_saved_workspace_size bytes (smaller than the recomputing
 *                 backward's), 256-byte aligned, not overlapping fwd_workspace
 * Supported where the forward keeps these summaries at the backward's precision: plans whose
 * summaries are split (MHLA_ACCURACY_SPLIT or MHLA_ACCURACY_TRAIN, or the automatic choice for
 * MALA, fp32 inputs and the ReLU and exp maps; mhla_plan_info.split_operands == 1) and which either mix in a kernel of their
 * own (more than 16 blocks: mhla_plan_info.n_kernels == 3) or read out MALA.  Else, and for
 * everything mhla_backward rejects, MHLA_ERR_UNSUPPORTED.  Errors as mhla_backward, plus
 * INVALID_ARG (fwd_workspace NULL, or overlapping an output or the workspace) and WORKSPACE
 * (fwd_workspace too small or misaligned).  Asynchronous on `stream`. */
mhla_status mhla_backward_saved_workspace_size(mhla_handle h, size_t* bytes);
mhla_status mhla_backward_saved(mhla_handle h, const void* q, const void* k, const void* v, const float* mc,
                                const void* dout, void* dq, void* dk, void* dv, float* dmc,
                                const void* fwd_workspace, size_t fwd_workspace_bytes, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Streaming decode: one new token per (batch, head) per call, for a causal plan ("MHLA: Restoring
 * Expressivity of Linear Attention via Token-Level Multi-Head", Method -> Key design 4: MHLA is
 * compatible with streaming / stateful inference; the causal reading of the causal readout modes
 * applies).  The plan (readout MHLA_READOUT_CAUSAL_*, a 1D grid, blocks of n_b tokens, ragged
 * blocks and a CLS token allowed) fixes the capacity: positions 0 .. N-1 (N counting a CLS token),
 * M blocks.  Token t lies in block i = t / n_b (with a CLS token: block 0 for t = 0, else
 * 1 + (t - 1) / n_b) and reads
 *     o_t = q~_t^T (S~<_i + m_ii R_t) / q~_t^T (z~<_i + m_ii r_t)    (no division: unnormalised)
 * with S~<_i = sum_{b<i} m_ib S_b over the completed blocks and R_t, r_t the sums of k~ v^T and k~
 * over block i's tokens up to t -- the same values as the causal forward's output t.
 *   state   device, mhla_decode_state_size bytes, 256-byte aligned, owned by the caller: per
 *           (batch, head) the completed blocks' S_b and z_b, S~<_i and z~<_i of the current block
 *           and the running R, r, all fp32, in a layout private to the library (the head's
 *           channels are cut into slices that each keep a copy of the d-vectors: about
 *           4 (M + 2)(d^2 + d s) bytes per (batch, head), s <= min(d / 8, d^2 / 1024) slices chosen
 *           from B * H).
 *           mhla_decode_reset clears it (position 0).
 *   t       the position of this call's token; calls on one state must come with t = 0, 1, 2, ...
 *           in order (t outside [0, N): MHLA_ERR_INVALID_ARG).  At the first token of a block the
 *           call also stores the finished block's summary and forms S~<_i from row i of M_c.
 *   q, k, v device [B, H, 1, d] of the plan's in_dtype; o: device [B, H, 1, d] of its out_dtype
 *   mc      device fp32 M_c as for mhla_forward (NULL iff M == 1).  Every call reads m_ii of its
 *           block; the first call of block i also reads row i below the diagonal.  So a caller
 *           that changes M_c between calls gets the causal readout of the M_c current at each
 *           block's start only if it changes M_c at block starts.
 * Arithmetic in fp32 (no MFMA: a d x d matrix-vector product per head).  Asynchronous on
 * `stream`; calls on one state must not overlap.  Not supported (MHLA_ERR_UNSUPPORTED): readouts
 * other than the causal ones. */
mhla_status mhla_decode_state_size(mhla_handle h, size_t* bytes);
mhla_status mhla_decode_reset(mhla_handle h, void* state, size_t state_bytes, void* stream);
mhla_status mhla_decode_step(mhla_handle h, void* state, size_t state_bytes, int64_t t, const void* q,
                             const void* k, const void* v, const float* mc, void* o, void* stream);

/* Prefill of the streaming decode: positions 0 .. n-1 (a prompt) of every (batch, head) in one call,
 * through the chunkwise causal forward, leaving in `state` what n calls of mhla_decode_step at
 * t = 0 .. n-1 would leave (the fp32 block summaries, the mixing of the completed blocks and the
 * last block's running sums), so that decoding continues at t = n.  The state's earlier contents
 * do not matter (no mhla_decode_reset is needed).
 *   n           1 <= n <= N (N counting a CLS token)
 *   q, k, v     device [B, H, n, d] of the plan's in_dtype (the prompt's positions)
 *   mc          as for mhla_decode_step (the plan's M x M, or H x M x M)
 *   o           device [B, H, n, d] of the plan's out_dtype: the outputs at positions 0 .. n-1
 *   workspace   device, mhla_decode_prefill_workspace_size(h, n) bytes, 256-byte aligned, its
 *               contents on entry irrelevant (0 bytes when n is a CLS token alone: one decode step)
 * The prefix's summaries and mixing run at split accuracy whatever the plan's accuracy field
 * (fp32-exact, as the decode state keeps them); its in-slice products follow the field, as in the
 * causal forward.  Outputs must not alias the inputs, the state or the workspace.
 * Errors: INVALID_ARG (NULL pointers, n out of range, mc NULL with M > 1, misalignment, aliasing),
 * UNSUPPORTED (not a causal plan), WORKSPACE (state or workspace too small or misaligned), HIP.
 * Asynchronous on `stream`. */
mhla_status mhla_decode_prefill_workspace_size(mhla_handle h, int64_t n, size_t* bytes);
mhla_status mhla_decode_prefill(mhla_handle h, void* state, size_t state_bytes, int64_t n, const void* q,
                                const void* k, const void* v, const float* mc, void* o, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Release a plan.  NULL is accepted. */
mhla_status mhla_destroy(mhla_handle h);

/* Static, human-readable text for a status code. */
const char* mhla_status_string(mhla_status s);

/* Fill `info` for a plan (info->struct_size must be set by the caller). */
mhla_status mhla_plan_get_info(mhla_handle h, mhla_plan_info* info);

/* Per-kernel timing.  While enabled, every mhla_forward records HIP events around each of its
 * kernels on the caller's stream (the plan owns the events).  mhla_timing_read synchronises on
 * the last recorded event, returns for kernel `index` (0 <= index < n_kernels) the summed
 * milliseconds and the number of timed launches, and leaves the counters untouched;
 * mhla_timing_reset clears them.  `name` receives a static string naming the kernel. */
mhla_status mhla_timing_enable(mhla_handle h, int enable);
mhla_status mhla_timing_read(mhla_handle h, int index, double* total_ms, int64_t* launches,
                             const char** name);
mhla_status mhla_timing_reset(mhla_handle h);

/* Per-kernel timing of mhla_backward, under the same switch and reset as the forward's: seven
 * entries in launch order, index 0..6 = "bwd_summary" (S, z recomputed), "bwd_mix" (S~, z~),
 * "bwd_dq" (dQ, g, dz~), "bwd_dsummary" (dS~), "bwd_dmix" (dS, dz), "bwd_keyside" (dK, dV),
 * "bwd_dmc" (dM_c: two kernels; empty when dmc is NULL). */
mhla_status mhla_backward_timing_read(mhla_handle h, int index, double* total_ms, int64_t* launches,
                                      const char** name);

#ifdef __cplusplus
}
#endif

#endif /* MHLA_H */
