"""GPU parity at the largest sizes the library accepts.

mhla_create bounds one head's bytes (N * d * 4 < 2^31: the kernels address a head through buffer
resources with 31-bit byte ranges), the number of (batch, head) pairs and the number of blocks
(each <= 65535).  These cases sit at or next to those bounds:
  * the longest head at d = 128 (N = 2^31 / 512 - 1 = 4194303 tokens) in ragged blocks of 16384
    (256 blocks, the last one 16383 tokens): forward with bf16 and with fp32 inputs (byte offsets
    up to 2^31 - 16), and the causal readout.  M_c = I, so that a query's output is the attention
    over its own block only -- the oracle's pinned reduction of M_c = I to block-diagonal local
    attention -- and the reference at sampled queries is the oracle on that block alone (16384
    tokens instead of 4 million).  The mixing kernel still runs (with the identity).  Inputs:
    synth.standard_normal_parallel (seeded child streams, 16 threads), Q then K then V;
  * the most (batch, head) pairs, 65535, with a few tokens each, checked on sampled heads;
  * 2048 blocks (the VALU mixing kernel), checked in full;
  * streaming decode over 65535 (batch, head) pairs, checked on sampled heads.
Bars as everywhere: max|d| / RMS(o) <= 2e-2 for bf16 inputs, <= 1e-4 for fp32 inputs (RMS over
the sampled outputs for the longest head); the causal readout relative to max(RMS(o), |o_t|).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import announce, rel_err, run_hip

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-4
N_MAX_D128 = (1 << 31) // (128 * 4) - 1
NB = 16384


@pytest.fixture(scope="module")
def longest_head():
    shape = (1, 1, N_MAX_D128, 128)
    announce(f"generating inputs: shape={shape}")
    f32 = tuple(synth.standard_normal_parallel(shape, 510 + i, bf16=False) for i in range(3))
    b16 = tuple(synth.standard_normal_parallel(shape, 510 + i, bf16=True) for i in range(3))   # same draws
    announce("inputs ready")
    rng = np.random.default_rng(513)
    toks = sorted(set([0, 1, NB - 1, NB, N_MAX_D128 // 2, N_MAX_D128 - NB + 1, N_MAX_D128 - 2,
                       N_MAX_D128 - 1] + rng.choice(N_MAX_D128, 8, replace=False).tolist()))
    return {"fp32": f32, "bf16": b16}, toks


def _local_reference(q, k, v, toks, causal):
    """Outputs of the sampled queries from the oracle run on each query's own block (M_c = I)."""
    out = []
    for t in toks:
        b0 = (t // NB) * NB
        b1 = min(b0 + NB, N_MAX_D128)
        sl = slice(b0, b1)
        qb, kb, vb = q[:, :, sl], k[:, :, sl], v[:, :, sl]
        n = b1 - b0
        if causal:
            (r,) = oracle.forward_causal_sampled(qb, kb, vb, None, (n,), (n,), [(0, 0, [t - b0])])
        else:
            (r,) = oracle.forward_sampled(qb, kb, vb, None, (n,), (n,), [(0, 0, [t - b0])])
        out.append(r[0])
    return np.stack(out)


def _workload(dtype, readout="normalized"):
    return synth.Workload("max_head", dtype, 1, 1, 128, (N_MAX_D128,), (NB,), 0, "identity", readout,
                          ragged=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_longest_head_forward(longest_head, dtype):
    inputs, toks = longest_head
    q, k, v = inputs[dtype]
    w = _workload(dtype)
    mc = np.eye(w.n_blocks)
    announce(f"forward longest head, {dtype} inputs, {w.n_blocks} blocks")
    got = run_hip(w, q, k, v, mc)[0, 0, toks]
    ref = _local_reference(q, k, v, toks, causal=False)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) / rms
    print(f"  err={err:.3e} ({len(toks)} sampled queries)")
    assert np.all(np.isfinite(got))
    assert err <= (FP32_TOL if dtype == "fp32" else BF16_TOL)


def test_longest_head_causal(longest_head):
    inputs, toks = longest_head
    q, k, v = inputs["bf16"]
    w = _workload("bf16", "causal")
    mc = np.eye(w.n_blocks)
    announce(f"causal longest head, {w.n_blocks} blocks")
    got = run_hip(w, q, k, v, mc)[0, 0, toks]
    ref = _local_reference(q, k, v, toks, causal=True)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref) / np.maximum(rms, np.abs(ref))))
    print(f"  err={err:.3e} ({len(toks)} sampled queries)")
    assert err <= BF16_TOL


def test_most_heads():
    w = synth.Workload("max_heads", "bf16", 65535, 1, 32, (8,), (4,), 503, "softmax_l1")
    announce(f"{w.name} shape={w.qkv_shape}")
    q, k, v, mc, _ = synth.make_inputs(w)
    got = run_hip(w, q, k, v, mc)
    rng = np.random.default_rng(504)
    heads = [(0, 0), (65534, 0)] + [(int(b), 0) for b in rng.choice(65535, 62, replace=False)]
    want = oracle.forward(q, k, v, mc, w.grid, w.block, heads=heads)
    err = rel_err(np.stack([got[b, h] for b, h in heads]), want)
    print(f"  err={err:.3e} ({len(heads)} heads)")
    assert np.all(np.isfinite(got))
    assert err <= BF16_TOL


def test_decode_most_heads():
    """Streaming decode over the most (batch, head) pairs, 65535 (one workgroup per pair at
    d = 32), position by position through 3 blocks; sampled heads against the oracle's causal
    readout (elementwise bar relative to max(RMS(o), |o_t|))."""
    import torch
    import token_blocked_linear_amd as T
    from gpu_util import oracle_full, to_device
    w = synth.Workload("max_heads_decode", "bf16", 65535, 1, 32, (10,), (4,), 506, "softmax_gauss", "causal",
                       ragged=True)
    announce(f"{w.name} shape={w.qkv_shape} blocks={w.n_blocks}")
    q, k, v, mc, _ = synth.make_inputs(w)
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype="fp32", readout=w.readout, ragged=True)
    state = plan.alloc_decode_state()
    seq = [to_device(np.ascontiguousarray(np.moveaxis(x, 2, 0)), w.dtype) for x in (q, k, v)]
    tmc = torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    out = torch.empty((w.grid[0], w.batch, w.heads, 1, w.head_dim), dtype=torch.float32, device="cuda:0")
    for t in range(w.grid[0]):
        plan.decode_step(state, t, *(x[t].unsqueeze(2) for x in seq), tmc, out[t])
    torch.cuda.synchronize()
    got = np.moveaxis(out[:, :, :, 0].cpu().numpy().astype(np.float64), 0, 2)
    plan.close()
    rng = np.random.default_rng(507)
    heads = [(0, 0), (65534, 0)] + [(int(b), 0) for b in rng.choice(65535, 62, replace=False)]
    want = oracle_full(w, q, k, v, mc, heads=heads)
    g = np.stack([got[b, h] for b, h in heads])
    rms = float(np.sqrt(np.mean(want * want)))
    err = float(np.max(np.abs(g - want) / np.maximum(rms, np.abs(want))))
    print(f"  err={err:.3e} ({len(heads)} heads)")
    assert np.all(np.isfinite(got))
    assert err <= BF16_TOL


def test_two_thousand_blocks():
    w = synth.Workload("m2048", "bf16", 1, 2, 32, (32768,), (16,), 505, "softmax_gauss")
    announce(f"{w.name} blocks={w.n_blocks}")
    q, k, v, mc, _ = synth.make_inputs(w)
    got = run_hip(w, q, k, v, mc)
    err = rel_err(got, oracle.forward(q, k, v, mc, w.grid, w.block))
    print(f"  err={err:.3e}")
    assert err <= BF16_TOL
