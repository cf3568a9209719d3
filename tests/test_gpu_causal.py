"""GPU parity of the chunkwise-causal readout against the fp64 causal oracle.

Bar: |o_gpu - o_oracle| <= tol * max(RMS(o_oracle), |o_oracle|) elementwise, tol = 2e-2 for bf16
inputs and 1e-4 for fp32 inputs (the forward's tolerances); test_causal_small also holds every
case to the forward's plain metric max|o_gpu - o_oracle| / RMS(o_oracle) <= tol.  The forward's metric divides by RMS(o)
alone; a causal output spans a far wider range (the first token's output is v_0 itself, the later
ones average ever more values: max|o| / RMS(o) is 26 to 61 on these cases against about 5 for the
non-causal readout), so the same per-element precision of the split operands (about 1e-5 of |o_t|)
would read as 1e-4 of RMS.  Below the RMS the bar is the forward's; above it, relative to |o_t|.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import announce, oracle_full, record, rel_err, run_hip

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-4


def _tol(w):
    return FP32_TOL if w.dtype == "fp32" else BF16_TOL


def causal_err(got, want):
    """max |got - want| / max(RMS(want), |want|) over all elements."""
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want) / np.maximum(rms, np.abs(want))))


def W(name, dtype, b, h, d, n, nb, seed, mc="softmax_gauss", readout="causal", phi="elu1"):
    return synth.Workload(name, dtype, b, h, d, (n,), (nb,), seed, mc, readout, phi)


CASES = [
    W("c_m4", "bf16", 1, 2, 64, 1024, 256, 201),
    W("c_ragged_sub", "bf16", 2, 3, 64, 1000, 200, 202, "softmax_l1"),        # 200 = 3 x 64 + 8
    W("c_d32_m15", "bf16", 1, 2, 32, 960, 64, 203, "softmax_l1"),
    W("c_d128_m16", "bf16", 1, 2, 128, 2048, 128, 204),
    W("c_d128_ragged", "bf16", 1, 1, 128, 600, 200, 205),                    # 200 = 6 x 32 + 8
    W("c_m1_long", "bf16", 1, 2, 64, 3000, 3000, 206, "none"),               # 12 token slices
    W("c_m1_short", "bf16", 1, 1, 64, 100, 100, 207, "none"),
    W("c_one_token_blocks", "bf16", 1, 1, 64, 40, 1, 208, "softmax_l1"),
    W("c_m4_four_slices", "bf16", 1, 2, 64, 4096, 1024, 209),
    W("c_m300_valu", "bf16", 1, 1, 32, 4800, 16, 210),
    W("c_identity", "bf16", 1, 2, 64, 1024, 128, 211, "identity"),
    W("c_unnorm", "bf16", 1, 2, 64, 1000, 200, 212, "softmax_l1", "causal_unnormalized"),
    W("c_fp32", "fp32", 1, 2, 64, 512, 128, 213),
    W("c_fp32_d128_slices", "fp32", 1, 1, 128, 1200, 600, 214),
    W("c_fp32_d32_unnorm", "fp32", 1, 2, 32, 640, 64, 215, "softmax_l1", "causal_unnormalized"),
    W("c_relu", "bf16", 1, 2, 64, 1024, 256, 216, phi="relu"),
    W("c_exp", "bf16", 1, 2, 64, 1024, 256, 217, phi="exp"),
    W("c_exp_d128", "bf16", 1, 2, 128, 1024, 128, 218, phi="exp"),
    # many heads with fp32 inputs: the outputs with only a few keys in view (the first tokens)
    # carry the in-sub-chunk products' rounding without averaging
    W("c_fp32_heads_d64", "fp32", 8, 16, 64, 512, 128, 219),
    W("c_fp32_heads_d128", "fp32", 32, 16, 128, 128, 128, 220, "none"),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_causal_small(w):
    announce(f"causal {w.name} shape={w.qkv_shape} block={w.block} {w.readout} {w.phi} {w.dtype}")
    q, k, v, mc, _ = synth.make_inputs(w)
    if w.phi == "relu":
        q = np.abs(q)
    got = run_hip(w, q, k, v, mc)
    want = oracle_full(w, q, k, v, mc)
    err = causal_err(got, want)
    plain = rel_err(got, want)
    print(f"  err={err:.3e} (max|d|/RMS {plain:.3e})")
    record("causal", w.name, r31=err, plain=plain, max_o_over_rms=float(np.max(np.abs(want)) / np.sqrt(np.mean(want ** 2))),
           dtype=w.dtype, phi=w.phi, readout=w.readout)
    assert np.all(np.isfinite(got))
    assert err <= _tol(w), (w.name, err)
    assert plain <= _tol(w), (w.name, plain)     # the forward's own metric holds as well


@pytest.mark.parametrize("name", ["c_m4", "c_d128_m16", "c_m300_valu"])
def test_causal_split_accuracy_option(name):
    """bf16 inputs with ELU+1: the default takes single bf16 operands for the earlier blocks'
    summaries and mixing; MHLA_ACCURACY_SPLIT splits them too and must be tighter."""
    w = next(c for c in CASES if c.name == name)
    announce(f"causal {w.name} accuracy auto / split")
    q, k, v, mc, _ = synth.make_inputs(w)
    want = oracle_full(w, q, k, v, mc)
    e_auto = causal_err(run_hip(w, q, k, v, mc), want)
    e_split = causal_err(run_hip(w, q, k, v, mc, accuracy="split"), want)
    print(f"  auto={e_auto:.3e} split={e_split:.3e}")
    assert e_auto <= BF16_TOL and e_split <= 1e-3 and e_split < e_auto


def test_causal_per_head_mc_and_upper_triangle_unused():
    w = W("c_per_head", "bf16", 2, 3, 64, 768, 128, 221, "none")
    announce(w.name)
    q, k, v, _, rng = synth.make_inputs(w)
    mc = rng.uniform(0.0, 1.0, (w.heads, w.n_blocks, w.n_blocks)).astype(np.float32).astype(np.float64)
    got = run_hip(w, q, k, v, mc)
    want = oracle_full(w, q, k, v, mc)
    assert causal_err(got, want) <= BF16_TOL
    # entries above the diagonal are never read: changing them changes nothing (bit for bit)
    mc2 = mc + np.triu(np.ones_like(mc[0]), 1)[None]
    assert np.array_equal(run_hip(w, q, k, v, mc2), got)


def test_causal_bf16_output():
    w = W("c_bf16_out", "bf16", 1, 2, 64, 1024, 256, 231)
    announce(w.name)
    q, k, v, mc, _ = synth.make_inputs(w)
    got = run_hip(w, q, k, v, mc, out_dtype="bf16")
    want = oracle_full(w, q, k, v, mc)
    rms = np.sqrt(np.mean(want ** 2))
    excess = np.abs(got - want) - (BF16_TOL * np.maximum(rms, np.abs(want)) + 2.0 ** -8 * np.abs(want))
    assert excess.max() <= 0, excess.max()


def test_causal_deterministic():
    w = W("c_det", "bf16", 1, 2, 64, 2048, 256, 241)
    q, k, v, mc, _ = synth.make_inputs(w)
    a, b = run_hip(w, q, k, v, mc, repeat=2)
    assert np.array_equal(a, b)


def test_causal_long1d_full_size():
    """The long-sequence workload (1 x 16 heads, 65536 tokens, d = 128, 256 blocks of 256) with the
    causal readout: one head in full, every head at sampled queries (the plain masked sum)."""
    w = synth.WORKLOADS["long1d"].with_(readout="causal")
    announce(f"causal full {w.name} shape={w.qkv_shape}")
    q, k, v, mc, rng = synth.make_inputs(w)
    got = run_hip(w, q, k, v, mc)
    assert np.all(np.isfinite(got))
    want0 = oracle_full(w, q, k, v, mc, heads=[(0, 3)])[0]
    err0 = causal_err(got[0, 3], want0)
    toks = sorted(set([0, 1, 255, 256, 257, 4095, 32768, 65535] + list(rng.integers(0, w.n_tokens, 8))))
    samples = [(0, h, toks) for h in range(w.heads)]
    ws = oracle.forward_causal_sampled(q, k, v, mc, w.grid, w.block, samples)
    want_s = np.stack(ws)
    got_s = np.stack([got[0, h, toks] for h in range(w.heads)])
    err_s = causal_err(got_s, want_s)
    print(f"  head 3 err={err0:.3e} sampled err={err_s:.3e}")
    assert err0 <= BF16_TOL and err_s <= BF16_TOL
