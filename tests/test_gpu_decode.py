"""GPU parity of the streaming decode (mhla_decode_step): feeding a sequence one token per call
gives the chunkwise-causal readout of the whole sequence.

The reference is the fp64 oracle's causal readout (query t reads every t' <= t with weight
m_{b(t), b(t')}), run on the same seeded inputs; the bar is the causal readout's elementwise one,
|o_t - ref_t| <= tol * max(RMS(ref), |ref_t|), with tol 2e-2 for bf16 inputs and 1e-4 for fp32
inputs.  The decode state is fp32 throughout.  The cases cover every channel-slice width the
library picks (8 .. d channels per workgroup, from the number of (batch, head) pairs), and plans
with a CLS token (position 0, a block of its own).  Each case also checks the decoded sequence against
the library's own chunkwise causal forward on the same inputs, to the same bar.
"""
import numpy as np
import pytest

import synth
from gpu_util import announce, oracle_full, record, rel_err, run_hip, to_device
import token_blocked_linear_amd as T

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-4


def W(name, dtype, b, h, d, n, nb, seed, mc="softmax_gauss", readout="causal", phi="elu1", cls=False):
    return synth.Workload(name, dtype, b, h, d, (n,), (nb,), seed, mc, readout, phi, ragged=n % nb != 0, cls=cls)


CASES = [
    # 5 blocks, the last one 88 tokens
    W("dec_d64_ragged", "bf16", 2, 2, 64, 600, 128, 601),
    W("dec_d32_fp32_unnorm_relu", "fp32", 1, 3, 32, 500, 96, 602, "softmax_l1", "causal_unnormalized", "relu"),
    W("dec_d128_exp", "bf16", 1, 2, 128, 700, 200, 603, "locality", phi="exp"),
    W("dec_d128_fp32", "fp32", 1, 1, 128, 384, 64, 604),
    # one block: M = 1 and no M_c
    W("dec_one_block", "bf16", 2, 2, 64, 300, 300, 605, "none"),
    # blocks of one token (M = N): every call closes a block
    W("dec_unit_blocks", "fp32", 1, 2, 32, 96, 1, 606, "softmax_l1"),
    # 32 blocks of 128
    W("dec_m32_d128", "bf16", 1, 4, 128, 4096, 128, 607, "softmax_l1"),
    # more (batch, head) pairs: fewer, wider channel slices per head (64 channels; whole heads)
    W("dec_batch_d128_c64", "bf16", 16, 16, 128, 300, 64, 608),
    W("dec_batch_d64_c64", "bf16", 64, 8, 64, 200, 48, 609, "softmax_l1"),
    W("dec_batch_d128_c128", "fp32", 32, 16, 128, 130, 32, 610),
    # a CLS token: position 0 is block 0 on its own, then blocks of n_b (the last one short)
    W("dec_cls", "bf16", 2, 2, 64, 500, 128, 613, cls=True),
    W("dec_cls_fp32_unnorm", "fp32", 1, 3, 128, 300, 64, 614, readout="causal_unnormalized", cls=True),
]


def _inputs(w):
    q, k, v, mc, rng = synth.make_inputs(w)
    if w.phi == "relu":          # keep every query off ReLU's all-zero features
        q = np.abs(q)
    return q, k, v, mc, rng


def decode_sequence(w, q, k, v, mc, *, out_dtype="fp32", plan=None, state=None, t0=0, t1=None):
    """Steps tokens t0 .. t1-1 through mhla_decode_step; returns float64 [B, H, t1-t0, d]."""
    import torch
    mc_per_head = mc is not None and np.ndim(mc) == 3
    own = plan is None
    if own:
        plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                      in_dtype=w.dtype, out_dtype=out_dtype, readout=w.readout, phi=w.phi,
                      mc_per_head=mc_per_head, ragged=w.ragged, cls_token=w.cls)
        state = plan.alloc_decode_state()
    t1 = w.n_tokens if t1 is None else t1
    # token-major copies, so that one token of every (batch, head) is one contiguous [B, H, 1, d]
    seq = [to_device(np.ascontiguousarray(np.moveaxis(x[:, :, t0:t1], 2, 0)), w.dtype) for x in (q, k, v)]
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.empty((t1 - t0, w.batch, w.heads, 1, w.head_dim), dtype=odt, device="cuda:0")
    for t in range(t0, t1):
        i = t - t0
        plan.decode_step(state, t, *(x[i].unsqueeze(2) for x in seq), tmc, out[i])
    torch.cuda.synchronize()
    res = np.moveaxis(out[:, :, :, 0].float().cpu().numpy().astype(np.float64), 0, 2)
    if own:
        plan.close()
    return res


def causal_err(got, want):
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want) / np.maximum(rms, np.abs(want))))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_matches_causal_readout(w):
    announce(f"decode {w.name} shape={w.qkv_shape} block={w.block} blocks={w.n_blocks} {w.readout} "
             f"{w.phi} {w.dtype}")
    q, k, v, mc, _ = _inputs(w)
    got = decode_sequence(w, q, k, v, mc)
    want = oracle_full(w, q, k, v, mc)
    tol = FP32_TOL if w.dtype == "fp32" else BF16_TOL
    err = causal_err(got, want)
    chunk = run_hip(w, q, k, v, mc)
    err_chunk = causal_err(got, chunk)
    plain = rel_err(got, want)
    print(f"  err={err:.3e} (max|d|/RMS {plain:.3e}) vs chunkwise forward {err_chunk:.3e}")
    record("decode", w.name, r31=err, plain=plain, vs_chunkwise_r31=err_chunk, dtype=w.dtype, phi=w.phi,
           readout=w.readout)
    assert np.all(np.isfinite(got))
    assert err <= tol, (w.name, err)
    assert plain <= tol, (w.name, plain)         # the forward's own metric holds as well
    assert err_chunk <= tol, (w.name, err_chunk)


def test_decode_bf16_output_and_per_head_mc():
    w = W("dec_per_head_bf16_out", "bf16", 2, 3, 64, 520, 100, 611, "none")
    announce(w.name)
    q, k, v, _, rng = _inputs(w)
    mc = rng.uniform(0.0, 1.0, (w.heads, w.n_blocks, w.n_blocks))
    got = decode_sequence(w, q, k, v, mc, out_dtype="bf16")
    err = causal_err(got, oracle_full(w, q, k, v, mc))
    print(f"  err={err:.3e}")
    assert err <= BF16_TOL


def test_decode_reset_and_resume():
    """A reset state starts a new sequence; a state carries over between runs of calls, so that
    a sequence decoded in two parts equals the sequence decoded at once."""
    import torch
    w = W("dec_reset", "fp32", 1, 2, 64, 400, 96, 612)
    announce(w.name)
    q, k, v, mc, rng = _inputs(w)
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, readout=w.readout, phi=w.phi, ragged=w.ragged)
    state = plan.alloc_decode_state()
    # a first, unrelated sequence leaves the state dirty (parts of every block in it)
    junk = [rng.standard_normal(x.shape) for x in (q, k, v)]
    decode_sequence(w, *junk, mc, plan=plan, state=state, t1=250)
    plan.decode_reset(state)
    a = decode_sequence(w, q, k, v, mc, plan=plan, state=state, t1=150)
    b = decode_sequence(w, q, k, v, mc, plan=plan, state=state, t0=150)
    torch.cuda.synchronize()
    got = np.concatenate([a, b], axis=2)
    whole = decode_sequence(w, q, k, v, mc)
    plan.close()
    assert np.array_equal(got, whole)
    assert causal_err(got, oracle_full(w, q, k, v, mc)) <= FP32_TOL


PREFILL_CASES = [
    # (workload, prefix lengths): a position inside the first block, a block's end, the next
    # block's first position, mid-sequence, the whole sequence
    (W("pf_d64_ragged", "bf16", 2, 2, 64, 600, 128, 621), (1, 100, 128, 129, 300, 600)),
    # a CLS token: the CLS token alone (one decode step), then prefixes into the grid blocks
    (W("pf_cls", "bf16", 2, 2, 64, 500, 128, 622, cls=True), (1, 2, 129, 300)),
    (W("pf_d128_fp32", "fp32", 1, 1, 128, 384, 64, 623), (200,)),
    (W("pf_unit_blocks", "fp32", 1, 2, 32, 96, 1, 624, "softmax_l1"), (50,)),
    (W("pf_one_block", "bf16", 2, 2, 64, 300, 300, 625, "none"), (150,)),
    # blocks over 256 tokens: the prefix's summaries come in several token slices
    (W("pf_big_blocks", "bf16", 1, 2, 64, 1500, 600, 626), (1000,)),
    (W("pf_unnorm_relu", "fp32", 1, 3, 32, 500, 96, 627, "softmax_l1", "causal_unnormalized", "relu"), (250,)),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: c[0].name)
def test_decode_prefill_then_steps(case):
    """mhla_decode_prefill over positions 0 .. n-1, then mhla_decode_step from t = n: the whole
    sequence matches the causal oracle (both metrics) and the step-by-step decode, for a state
    left dirty by an unrelated sequence before the prefill."""
    import torch
    w, prefixes = case
    q, k, v, mc, rng = _inputs(w)
    want = oracle_full(w, q, k, v, mc)
    whole = decode_sequence(w, q, k, v, mc)
    tol = FP32_TOL if w.dtype == "fp32" else BF16_TOL
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype="fp32", readout=w.readout, phi=w.phi, ragged=w.ragged,
                  cls_token=w.cls)
    state = plan.alloc_decode_state()
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    for n in prefixes:
        announce(f"prefill {w.name} n={n} of {w.n_tokens} shape={w.qkv_shape} block={w.block} {w.readout}")
        junk = [rng.standard_normal(x.shape) for x in (q, k, v)]
        decode_sequence(w, *junk, mc, plan=plan, state=state, t1=min(w.n_tokens, 70))
        tq, tk, tv = (to_device(np.ascontiguousarray(x[:, :, :n]), w.dtype) for x in (q, k, v))
        o_pre = torch.empty((w.batch, w.heads, n, w.head_dim), dtype=torch.float32, device="cuda:0")
        ws = plan.alloc_prefill_workspace(n)
        plan.decode_prefill(state, tq, tk, tv, tmc, o_pre, ws)
        torch.cuda.synchronize()
        parts = [o_pre.cpu().numpy().astype(np.float64)]
        if n < w.n_tokens:
            parts.append(decode_sequence(w, q, k, v, mc, plan=plan, state=state, t0=n))
        got = np.concatenate(parts, axis=2)
        err, plain, err_steps = causal_err(got, want), rel_err(got, want), causal_err(got, whole)
        print(f"  n={n}: err={err:.3e} (max|d|/RMS {plain:.3e}) vs step-by-step decode {err_steps:.3e}")
        record("decode_prefill", f"{w.name}_n{n}", r31=err, plain=plain, vs_steps_r31=err_steps, dtype=w.dtype)
        assert np.all(np.isfinite(got))
        assert err <= tol and plain <= tol and err_steps <= tol, (w.name, n, err, plain, err_steps)
    plan.close()
