"""GPU parity of the backward pass (dQ, dK, dV, dM_c; MALA: dQ, dK, dV) against the fp64 oracle.

The gradients are of L = sum(dO * O) for a seeded standard-normal dO.  Bar, for every gradient
tensor separately, as max|g_gpu - g_oracle| / RMS(g_oracle):
  * bf16 inputs: 2e-2, the forward's bar;
  * fp32 inputs: 5e-4.  Every product of the backward runs on split bf16 operands (hi + lo),
    about 3 * 2^-18 = 1.1e-5 relative error per product against fp32's 6e-8.  The gradients are
    sums of opposite-signed terms (dq~ = S~ g + z~ gden, dk~ = dS v + dz): on these inputs the
    sum of the terms' magnitudes reaches about 25x the RMS of the result (the exp map is the
    worst), and dK goes through two such contractions in a row, so 2 * 25 * 1.1e-5 = 5.5e-4.
    The forward's 1e-4 assumes a quotient of positive sums, which has no such cancellation.
"""
import numpy as np
import pytest

import synth
from gpu_util import announce, oracle_backward, record, rel_err, run_hip_backward

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 5e-4
NAMES = ("dq", "dk", "dv", "dmc")


def _tol(w):
    return FP32_TOL if w.dtype == "fp32" else BF16_TOL


def _inputs(w, out_dtype="fp32", positive_q=False):
    q, k, v, mc, rng = synth.make_inputs(w)
    if positive_q:   # ReLU: keep every query's features off the all-zero case
        q = np.abs(q)
    do = synth.make_grad_output(w, rng, out_dtype)
    return q, k, v, mc, do


def _check(w, got, want, tol, heads=None):
    if got[3] is None:            # dM_c not requested (or no M_c: a single block)
        want = tuple(want[:3]) + (None,)
    errs = {}
    for name, g, r in zip(NAMES, got, want):
        if r is None:
            assert g is None
            continue
        if heads is not None and name != "dmc":
            g = np.stack([g[b, h] for b, h in heads])
        assert np.all(np.isfinite(g)), name
        errs[name] = rel_err(g, r)
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    record("backward", w.name, dtype=w.dtype, readout=w.readout, phi=w.phi, tol=tol, **errs)
    for n, e in errs.items():
        assert e <= tol, (w.name, n, e)


CASES = [
    synth.Workload("bw_2d", "bf16", 2, 2, 64, (32, 32), (8, 8), 101, "softmax_l1"),
    synth.Workload("bw_ragged1d", "bf16", 2, 3, 64, (1000,), (200,), 102, "softmax_l1"),
    synth.Workload("bw_odd2d_d32", "bf16", 2, 2, 32, (30, 42), (5, 7), 103, "softmax_l1"),
    synth.Workload("bw_odd3d_d128", "bf16", 1, 2, 128, (6, 10, 12), (3, 5, 4), 104, "softmax_l1"),
    synth.Workload("bw_unnorm", "bf16", 2, 2, 64, (32, 32), (8, 8), 105, "softmax_l1", "unnormalized"),
    synth.Workload("bw_m1_long", "bf16", 1, 3, 64, (3001,), (3001,), 106, "none"),
    synth.Workload("bw_one_token_blocks", "bf16", 1, 1, 64, (40,), (1,), 107, "softmax_l1"),
    synth.Workload("bw_identity", "bf16", 1, 2, 64, (48, 48), (16, 24), 108, "identity"),
    synth.Workload("bw_ones", "bf16", 1, 2, 64, (48, 48), (16, 24), 109, "ones"),
    synth.Workload("bw_m100", "bf16", 1, 2, 64, (1000,), (10,), 110, "softmax_l1"),
    synth.Workload("bw_m200_d128", "bf16", 1, 2, 128, (3200,), (16,), 111, "softmax_gauss"),
    synth.Workload("bw_m144_d32", "bf16", 2, 1, 32, (48, 48), (4, 4), 112, "locality"),
    synth.Workload("bw_two_slices", "bf16", 1, 1, 64, (16384,), (512,), 116, "softmax_gauss"),
    synth.Workload("bw_m256_d32", "bf16", 1, 2, 32, (4096,), (16,), 117, "softmax_gauss"),
    synth.Workload("bw_m300_valu_mix", "bf16", 1, 1, 32, (4800,), (16,), 118, "softmax_gauss"),
    synth.Workload("bw_fp32_2d", "fp32", 2, 2, 64, (24, 24), (8, 12), 113, "softmax_l1"),
    synth.Workload("bw_fp32_d128", "fp32", 1, 2, 128, (900,), (300,), 114, "softmax_gauss"),
    synth.Workload("bw_fp32_unnorm_d32", "fp32", 1, 2, 32, (20, 20), (5, 4), 115, "softmax_l1", "unnormalized"),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_small(w):
    announce(f"backward {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} {w.readout}")
    q, k, v, mc, do = _inputs(w)
    got = run_hip_backward(w, q, k, v, mc, do)
    _check(w, got, oracle_backward(w, q, k, v, mc, do), _tol(w))


MAP_CASES = [
    synth.Workload("bw_relu_2d", "bf16", 2, 2, 64, (32, 32), (8, 8), 121, "softmax_l1", phi="relu"),
    synth.Workload("bw_exp_2d", "bf16", 2, 2, 64, (32, 32), (8, 8), 122, "softmax_l1", phi="exp"),
    synth.Workload("bw_relu_d128", "bf16", 1, 2, 128, (6, 10, 12), (3, 5, 4), 123, "softmax_l1", phi="relu"),
    synth.Workload("bw_exp_d32_unnorm", "bf16", 1, 2, 32, (1000,), (200,), 124, "softmax_l1", "unnormalized",
                   phi="exp"),
    synth.Workload("bw_relu_fp32", "fp32", 1, 2, 64, (24, 24), (8, 12), 125, "softmax_l1", phi="relu"),
    synth.Workload("bw_exp_fp32", "fp32", 1, 2, 64, (24, 24), (8, 12), 126, "softmax_l1", phi="exp"),
]


@pytest.mark.parametrize("w", MAP_CASES, ids=lambda w: w.name)
def test_backward_feature_maps(w):
    announce(f"backward {w.name} phi={w.phi} shape={w.qkv_shape} {w.readout}")
    q, k, v, mc, do = _inputs(w, positive_q=w.phi == "relu")
    got = run_hip_backward(w, q, k, v, mc, do)
    _check(w, got, oracle_backward(w, q, k, v, mc, do), _tol(w))


def test_backward_per_head_mc():
    w = synth.Workload("bw_per_head", "bf16", 2, 3, 64, (32, 32), (8, 16), 131, "none")
    announce(w.name)
    q, k, v, _, rng = synth.make_inputs(w)
    mc = rng.uniform(0.0, 1.0, (w.heads, w.n_blocks, w.n_blocks)).astype(np.float32).astype(np.float64)
    do = synth.make_grad_output(w, rng)
    got = run_hip_backward(w, q, k, v, mc, do)
    assert got[3].shape == mc.shape
    _check(w, got, oracle_backward(w, q, k, v, mc, do), BF16_TOL)


def _check_bf16_gradients(w, got, want, heads=None):
    """dQ, dK, dV in bf16: within the bar plus each output's own rounding (2^-8 relative at
    most); dM_c stays fp32 and takes the plain bar."""
    errs = {}
    for name, g, r in zip(NAMES[:3], got[:3], want[:3]):
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
        assert np.all(np.isfinite(g)), name
        rms = np.sqrt(np.mean(r ** 2))
        excess = np.abs(g - r) - (BF16_TOL * rms + 2.0 ** -8 * np.abs(r))
        errs[name] = rel_err(g, r)
        assert excess.max() <= 0, (w.name, name, excess.max())
    if got[3] is not None and want[3] is not None:
        errs["dmc"] = rel_err(got[3], want[3])
        assert errs["dmc"] <= BF16_TOL, (w.name, errs["dmc"])
    print("  bf16 gradients " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    record("backward_bf16_gradients", w.name, phi=w.phi, readout=w.readout, **errs)


@pytest.mark.parametrize("phi", ["elu1", "exp"])
def test_backward_bf16_gradients(phi):
    w = synth.Workload("bw_bf16_out", "bf16", 2, 2, 64, (1000,), (200,), 141, "softmax_l1", phi=phi)
    announce(f"{w.name} {phi}")
    q, k, v, mc, do = _inputs(w, out_dtype="bf16")
    got = run_hip_backward(w, q, k, v, mc, do, out_dtype="bf16")
    _check_bf16_gradients(w, got, oracle_backward(w, q, k, v, mc, do))


# bf16 dO takes the LDS-streamed token-weighted summary for dS~: head sizes 32 and 128, odd 2D
# and 3D blocks (partial stages, gathered token weights), the unnormalised readout, ReLU, and
# many small blocks
BF16_GRAD_CASES = [
    synth.Workload("bwg_odd2d_d32", "bf16", 2, 2, 32, (30, 42), (5, 7), 181, "softmax_l1"),
    synth.Workload("bwg_odd3d_d128", "bf16", 1, 2, 128, (6, 10, 12), (3, 5, 4), 182, "softmax_l1"),
    synth.Workload("bwg_unnorm_2d", "bf16", 2, 2, 64, (32, 32), (8, 8), 183, "softmax_l1", "unnormalized"),
    synth.Workload("bwg_relu_d128", "bf16", 1, 2, 128, (6, 10, 12), (3, 5, 4), 184, "softmax_l1", phi="relu"),
    synth.Workload("bwg_m200_d128", "bf16", 1, 2, 128, (3200,), (16,), 185, "softmax_gauss"),
    synth.Workload("bwg_ragged_cls", "bf16", 1, 2, 64, (30, 34), (4, 4), 186, "softmax_gauss", ragged=True,
                   cls=True),
]


@pytest.mark.parametrize("w", BF16_GRAD_CASES, ids=lambda w: w.name)
def test_backward_bf16_gradients_shapes(w):
    announce(f"backward bf16 gradients {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} {w.readout}")
    q, k, v, mc, do = _inputs(w, out_dtype="bf16", positive_q=w.phi == "relu")
    got = run_hip_backward(w, q, k, v, mc, do, out_dtype="bf16")
    _check_bf16_gradients(w, got, oracle_backward(w, q, k, v, mc, do))


def test_backward_without_dmc_and_deterministic():
    w = synth.Workload("bw_nodmc", "bf16", 2, 2, 64, (32, 32), (8, 8), 151, "softmax_l1")
    announce(w.name)
    q, k, v, mc, do = _inputs(w)
    a = run_hip_backward(w, q, k, v, mc, do, want_dmc=False)
    assert a[3] is None
    runs = run_hip_backward(w, q, k, v, mc, do, repeat=3)
    for r in runs:
        for x, y in zip(r[:3], a[:3]):
            assert np.array_equal(x, y)            # same kernels, fixed summation order
        assert np.array_equal(r[3], runs[0][3])
    _check(w, a, oracle_backward(w, q, k, v, mc, do)[:3] + (None,), BF16_TOL)


def test_backward_two_plans_in_a_row_smaller_second():
    """A larger then a smaller problem through fresh plans and workspaces: nothing carries
    over between calls."""
    for w in (synth.Workload("bw_big", "bf16", 2, 2, 64, (64, 64), (16, 16), 161, "softmax_l1"),
              synth.Workload("bw_small", "bf16", 1, 1, 64, (16, 16), (8, 8), 162, "softmax_l1")):
        announce(w.name)
        q, k, v, mc, do = _inputs(w)
        _check(w, run_hip_backward(w, q, k, v, mc, do), oracle_backward(w, q, k, v, mc, do), BF16_TOL)


# ------------------------------------------------------------------------------------------
# full sizes of the image and video workloads (every head), and the long sequence (sampled
# heads for dQ, dK, dV; dM_c through a property that holds at any size)
# ------------------------------------------------------------------------------------------

# ------------------------------------------------------------------------------------------
# MALA (one block): the centred chain rule against the oracle's linear-form chain rule
# (oracle.mala_backward); no M_c, so no dM_c
# ------------------------------------------------------------------------------------------

MALA_CASES = [
    synth.Workload("bw_mala_2d", "bf16", 2, 2, 64, (32, 32), (32, 32), 171, "none", "mala"),
    synth.Workload("bw_mala_ragged1d", "bf16", 2, 3, 64, (1000,), (1000,), 172, "none", "mala"),
    synth.Workload("bw_mala_d32", "bf16", 1, 2, 32, (30, 42), (30, 42), 173, "none", "mala"),
    synth.Workload("bw_mala_d128", "bf16", 1, 2, 128, (6, 10, 12), (6, 10, 12), 174, "none", "mala"),
    synth.Workload("bw_mala_long", "bf16", 1, 2, 64, (20000,), (20000,), 175, "none", "mala"),
    synth.Workload("bw_mala_tiny", "bf16", 1, 1, 64, (5,), (5,), 176, "none", "mala"),
    synth.Workload("bw_mala_fp32", "fp32", 2, 2, 64, (24, 24), (24, 24), 177, "none", "mala"),
    synth.Workload("bw_mala_fp32_d128", "fp32", 1, 2, 128, (900,), (900,), 178, "none", "mala"),
    synth.Workload("bw_mala_relu", "bf16", 1, 2, 64, (32, 32), (32, 32), 179, "none", "mala", phi="relu"),
    synth.Workload("bw_mala_exp", "bf16", 1, 2, 64, (32, 32), (32, 32), 180, "none", "mala", phi="exp"),
    synth.Workload("bw_mala_exp_fp32_d32", "fp32", 1, 2, 32, (20, 20), (20, 20), 181, "none", "mala",
                   phi="exp"),
]


@pytest.mark.parametrize("w", MALA_CASES, ids=lambda w: w.name)
def test_backward_mala(w):
    announce(f"backward {w.name} phi={w.phi} shape={w.qkv_shape} mala")
    q, k, v, mc, do = _inputs(w, positive_q=w.phi == "relu")
    assert mc is None
    got = run_hip_backward(w, q, k, v, mc, do)
    assert got[3] is None
    _check(w, got, oracle_backward(w, q, k, v, mc, do), _tol(w))


def test_backward_mala_full_image_and_bf16_gradients():
    """The full MALA image workload (every head), with fp32 and with bf16 gradients (the plain
    bar plus each bf16 output's own rounding, as for the MHLA case); repeated calls are
    bit-identical."""
    w = synth.WORKLOADS["image_mala"]
    announce(f"backward full image_mala shape={w.qkv_shape}")
    q, k, v, mc, do = _inputs(w)
    runs = run_hip_backward(w, q, k, v, mc, do, repeat=2)
    for x, y in zip(runs[0][:3], runs[1][:3]):
        assert np.array_equal(x, y)
    want = oracle_backward(w, q, k, v, mc, do)
    _check(w, runs[0], want, BF16_TOL)
    do16 = synth.round_to_bf16(do)
    got = run_hip_backward(w, q, k, v, mc, do16, out_dtype="bf16")
    want = oracle_backward(w, q, k, v, mc, do16)
    for name, g, r in zip(NAMES[:3], got[:3], want[:3]):
        rms = np.sqrt(np.mean(r ** 2))
        excess = np.abs(g - r) - (BF16_TOL * rms + 2.0 ** -8 * np.abs(r))
        print(f"  bf16 {name} max|d|/rms={rel_err(g, r):.2e}")
        assert excess.max() <= 0, (name, excess.max())


@pytest.mark.parametrize("name", ["image", "video3d"])
def test_backward_full(name):
    w = synth.WORKLOADS[name]
    announce(f"backward full {name} shape={w.qkv_shape} blocks={w.n_blocks}")
    q, k, v, mc, do = _inputs(w)
    got = run_hip_backward(w, q, k, v, mc, do)
    _check(w, got, oracle_backward(w, q, k, v, mc, do), BF16_TOL)


@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_backward_long1d_sampled(out_dtype):
    """The long-sequence workload at full size, with fp32 gradients and with bf16 gradients (as
    the benchmark runs it): heads 0 and 15 against the oracle, dM_c through its invariance."""
    w = synth.WORKLOADS["long1d"]
    announce(f"backward full long1d shape={w.qkv_shape} blocks={w.n_blocks} gradients {out_dtype}")
    q, k, v, mc, do = _inputs(w, out_dtype=out_dtype)
    got = run_hip_backward(w, q, k, v, mc, do, out_dtype=out_dtype)
    heads = [(0, 0), (0, w.heads - 1)]
    want = oracle_backward(w, q, k, v, mc, do, heads=heads)
    if out_dtype == "bf16":
        _check_bf16_gradients(w, got[:3] + (None,), want[:3] + (None,), heads=heads)
    else:
        _check(w, got[:3] + (None,), want[:3] + (None,), BF16_TOL, heads=heads)
    # O is invariant under scaling row i of M_c (S~_i and z~_i scale together), so
    # sum_b M_c[i, b] dM_c[i, b] = 0 for every row i.
    dmc = got[3]
    terms = mc * dmc
    scale = float(np.sqrt(np.mean(np.sum(np.abs(terms), axis=1) ** 2)))
    resid = np.abs(terms.sum(axis=1))
    print(f"  row-invariance residual max={resid.max() / scale:.2e}")
    assert np.all(np.isfinite(dmc))
    assert resid.max() <= BF16_TOL * scale
