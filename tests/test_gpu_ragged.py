"""GPU parity with ragged blocks (block extents that do not divide the grid) and a CLS token,
against the fp64 oracle's RaggedGrid geometry.

Readings (oracle RaggedGrid): blocks tile the grid from its origin, the last block along an axis
keeps what is left; blocks are numbered in raster order over the rounded-up block grid; a CLS
token is token 0 and block 0 on its own.  Bars as for whole blocks: forward max|d|/RMS(o) 2e-2
(bf16 inputs) and 1e-4 (fp32); backward 2e-2 and 5e-4 (the backward's derived bar); the causal
readout's elementwise bar relative to max(RMS(o), |o_t|).
"""
import numpy as np
import pytest

import synth
from gpu_util import announce, oracle_backward, oracle_full, rel_err, run_hip, run_hip_backward

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-4
BWD_FP32_TOL = 5e-4


def R(name, dtype, b, h, d, grid, block, seed, mc="softmax_gauss", readout="normalized", phi="elu1",
      ragged=True, cls=False):
    return synth.Workload(name, dtype, b, h, d, tuple(grid), tuple(block), seed, mc, readout, phi,
                          ragged=ragged, cls=cls)


def _inputs(w):
    q, k, v, mc, rng = synth.make_inputs(w)
    if w.phi == "relu":          # keep every query off ReLU's all-zero features
        q = np.abs(q)
    return q, k, v, mc, rng


FORWARD_CASES = [
    # DeiT-T at 224 px: 14 x 14 patches in 7 x 7 blocks and the CLS token (197 tokens, 5 blocks)
    R("deit_t_cls", "bf16", 64, 3, 64, (14, 14), (7, 7), 301, ragged=False, cls=True),
    R("deit_t_cls_fp32", "fp32", 8, 3, 64, (14, 14), (7, 7), 302, ragged=False, cls=True),
    # ragged 2D: 3 x 3 blocks of 16, 8, 8, 4 ... tokens
    R("r2d_10x10_b4", "bf16", 2, 2, 64, (10, 10), (4, 4), 303, "softmax_l1"),
    # last-axis extents 16 then 10 (one contiguous run of 8 and one not), d = 32
    R("r2d_30x42_d32", "bf16", 2, 2, 32, (30, 42), (8, 16), 304, "locality"),
    # 3D, last-axis extents 8 then 5, d = 128
    R("r3d_d128", "bf16", 1, 2, 128, (6, 10, 13), (4, 4, 8), 305, "softmax_l1"),
    # a block extent beyond the grid's is clipped to it
    R("r_clip", "bf16", 1, 2, 64, (5, 40), (8, 16), 306, "softmax_l1"),
    # 1D ragged with a CLS token: blocks of 1, 300, 300, 300, 100 tokens
    R("r1d_cls", "bf16", 2, 2, 64, (1000,), (300,), 307, cls=True),
    R("r1d_cls_unnorm", "bf16", 1, 2, 64, (1000,), (300,), 308, readout="unnormalized", cls=True),
    R("r2d_cls_fp32_d16", "fp32", 1, 2, 16, (9, 11), (4, 4), 309, cls=True),
    R("r2d_cls_fp32_unnorm", "fp32", 1, 2, 64, (9, 11), (4, 4), 310, readout="unnormalized", cls=True),
    # one grid token and the CLS token: two one-token blocks
    R("cls_one_token", "bf16", 1, 2, 64, (1,), (1,), 311, cls=True),
    # more blocks than the readout's fused prologue takes: the mixing kernel (MFMA, bf16 stack)
    R("r1d_m106_mix", "bf16", 1, 2, 64, (5000,), (48,), 312, cls=True),
    # ... on split operands over fp32 partials, and the VALU mixing beyond 256 blocks
    R("r1d_m106_fp32_mix", "fp32", 1, 1, 64, (5000,), (48,), 313, cls=True),
    R("r1d_m314_valu", "bf16", 1, 1, 32, (20000,), (64,), 314, cls=True),
    # several token slices per block with a ragged last block
    R("r1d_slices", "bf16", 1, 2, 64, (9000,), (4096,), 315),
]

MAP_CASES = [
    R("r2d_relu", "bf16", 2, 2, 64, (10, 10), (4, 4), 321, "softmax_l1", phi="relu"),
    R("r2d_exp_cls", "bf16", 2, 2, 64, (14, 14), (6, 6), 322, phi="exp", cls=True),
    R("r3d_exp_d128", "bf16", 1, 2, 128, (6, 10, 13), (4, 4, 8), 323, "softmax_l1", phi="exp"),
    R("r1d_relu_fp32_cls", "fp32", 1, 2, 64, (1000,), (300,), 324, phi="relu", cls=True),
]


@pytest.mark.parametrize("w", FORWARD_CASES + MAP_CASES, ids=lambda w: w.name)
def test_ragged_forward(w):
    announce(f"ragged forward {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} cls={w.cls} "
             f"blocks={w.n_blocks} {w.readout} {w.phi} {w.dtype}")
    q, k, v, mc, _ = _inputs(w)
    got = run_hip(w, q, k, v, mc)
    want = oracle_full(w, q, k, v, mc)
    err = rel_err(got, want)
    print(f"  err={err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= (FP32_TOL if w.dtype == "fp32" else BF16_TOL), (w.name, err)


def test_ragged_forward_bf16_accuracy_level_and_per_head_mc():
    """The bf16-operand level (bf16 summary stack, MFMA mixing) with a per-head M_c."""
    w = R("r_cls_per_head", "bf16", 2, 3, 64, (14, 14), (7, 7), 331, "none", ragged=False, cls=True)
    announce(w.name)
    q, k, v, _, rng = _inputs(w)
    mc = rng.uniform(0.0, 1.0, (w.heads, w.n_blocks, w.n_blocks)).astype(np.float32).astype(np.float64)
    for accuracy in ("bf16", "split"):
        got = run_hip(w, q, k, v, mc, accuracy=accuracy)
        err = rel_err(got, oracle_full(w, q, k, v, mc))
        print(f"  {accuracy}: err={err:.3e}")
        assert err <= BF16_TOL, (accuracy, err)


def test_cls_token_reads_and_is_read_through_its_own_block():
    """The CLS block's row and column of M_c act on the CLS token alone: zeroing every other
    entry of its row leaves the CLS output equal to v_0 (its own value, the sole key it sees),
    and the grid tokens' outputs do not change when the CLS row changes."""
    w = R("r_cls_row", "fp32", 1, 1, 64, (14, 14), (7, 7), 332, ragged=False, cls=True)
    announce(w.name)
    q, k, v, mc, _ = _inputs(w)
    a = run_hip(w, q, k, v, mc)
    mc2 = mc.copy()
    mc2[0, :] = 0.0
    mc2[0, 0] = 0.5
    b = run_hip(w, q, k, v, mc2)
    np.testing.assert_allclose(b[0, 0, 0], v[0, 0, 0], rtol=1e-5, atol=1e-5)
    assert np.array_equal(a[0, 0, 1:], b[0, 0, 1:])


CAUSAL_CASES = [
    R("c_r1d_cls", "bf16", 1, 2, 64, (1000,), (256,), 341, readout="causal", cls=True),
    R("c_r1d_ragged", "bf16", 2, 2, 128, (1100,), (300,), 342, "softmax_l1", readout="causal"),
    R("c_r1d_cls_unnorm_fp32", "fp32", 1, 2, 32, (700,), (128,), 343, readout="causal_unnormalized", cls=True),
    R("c_r1d_cls_m40", "bf16", 1, 1, 64, (2000,), (51,), 344, readout="causal", cls=True),
]


@pytest.mark.parametrize("w", CAUSAL_CASES, ids=lambda w: w.name)
def test_ragged_causal(w):
    announce(f"ragged causal {w.name} shape={w.qkv_shape} block={w.block} cls={w.cls} {w.readout} {w.dtype}")
    q, k, v, mc, _ = _inputs(w)
    got = run_hip(w, q, k, v, mc)
    want = oracle_full(w, q, k, v, mc)
    rms = float(np.sqrt(np.mean(want * want)))
    err = float(np.max(np.abs(got - want) / np.maximum(rms, np.abs(want))))
    print(f"  err={err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= (FP32_TOL if w.dtype == "fp32" else BF16_TOL), (w.name, err)


BACKWARD_CASES = [
    R("b_deit_cls", "bf16", 4, 3, 64, (14, 14), (7, 7), 351, ragged=False, cls=True),
    R("b_r2d", "bf16", 2, 2, 64, (10, 10), (4, 4), 352, "softmax_l1"),
    # last axis 18 in blocks of 8: runs of 8, 8, 2 tokens in rows that start off a multiple of 4
    R("b_r2d_g18", "bf16", 1, 2, 64, (6, 18), (3, 8), 353, "softmax_l1"),
    R("b_r3d_d128", "bf16", 1, 2, 128, (6, 10, 13), (4, 4, 8), 354, "softmax_l1"),
    R("b_r1d_cls_exp", "bf16", 1, 2, 32, (1000,), (300,), 355, phi="exp", cls=True),
    R("b_r1d_cls_m106", "bf16", 1, 1, 64, (5000,), (48,), 356, cls=True),
    R("b_fp32_cls", "fp32", 1, 2, 64, (9, 11), (4, 4), 357, cls=True),
    R("b_fp32_unnorm_cls", "fp32", 1, 2, 64, (9, 11), (4, 4), 358, readout="unnormalized", cls=True),
]


@pytest.mark.parametrize("w", BACKWARD_CASES, ids=lambda w: w.name)
def test_ragged_backward(w):
    announce(f"ragged backward {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} cls={w.cls} "
             f"{w.readout} {w.phi} {w.dtype}")
    q, k, v, mc, rng = _inputs(w)
    do = synth.make_grad_output(w, rng)
    got = run_hip_backward(w, q, k, v, mc, do)
    want = oracle_backward(w, q, k, v, mc, do)
    tol = BWD_FP32_TOL if w.dtype == "fp32" else BF16_TOL
    errs = {n: rel_err(g, r) for n, g, r in zip(("dq", "dk", "dv", "dmc"), got, want)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, g in zip(("dq", "dk", "dv", "dmc"), got):
        assert np.all(np.isfinite(g)), n
    for n, e in errs.items():
        assert e <= tol, (w.name, n, e)
