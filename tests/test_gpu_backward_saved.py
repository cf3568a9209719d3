"""GPU tests of mhla_backward_saved: the backward that reads the forward's block summaries (and,
except for MALA, its mixed summaries) from the workspace of the plan's last forward call instead
of recomputing them ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
Multi-Head", Overall framework and Key design 2 for the steps; Key design 3 for training M_c).

Both backwards run the same kernels on the same values, so the saved one must reproduce the
recomputing one bit for bit; the recomputing one is held to the oracle in test_gpu_backward.py,
and here the gradients are checked against the oracle as well, with that file's bars.  The
forward that saves its state runs with split summaries and mixing (MHLA_ACCURACY_SPLIT, or
MHLA_ACCURACY_TRAIN, whose readout takes the mixed stack's high part with single operands); its
output is checked against the oracle with the forward's bar.
"""
import numpy as np
import pytest

import synth
from gpu_util import announce, oracle_backward, oracle_full, record, rel_err, to_device
import token_blocked_linear_amd as T

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 5e-4
FWD_TOL = {"bf16": 2e-2, "fp32": 1e-4}
NAMES = ("dq", "dk", "dv", "dmc")


def run_saved_and_recompute(w, q, k, v, mc, do, *, out_dtype="fp32", accuracy="split", heads=None):
    """Forward on a split plan, then the saved backward from its workspace and the recomputing
    backward; returns (o, saved gradients, recomputed gradients) as float64 numpy."""
    import torch
    mc_per_head = mc is not None and np.ndim(mc) == 3
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=out_dtype, readout=w.readout, accuracy=accuracy, phi=w.phi,
                  mc_per_head=mc_per_head, ragged=w.ragged, cls_token=w.cls)
    assert plan.info.split_operands == 1
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tdo = to_device(do, out_dtype)
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    fws = plan.alloc_workspace()
    o = torch.empty_like(tdo)
    plan.forward(tq, tk, tv, tmc, o, fws)
    grads = []
    for saved in (True, False):
        ws = plan.alloc_backward_saved_workspace() if saved else plan.alloc_backward_workspace()
        dq, dk, dv = (torch.empty_like(tdo) for _ in range(3))
        dmc = torch.full(tuple(np.shape(mc)), float("nan"), device="cuda:0") if mc is not None else None
        plan.backward(tq, tk, tv, tmc, tdo, dq, dk, dv, dmc, ws, fwd_workspace=fws if saved else None)
        torch.cuda.synchronize()
        grads.append(tuple(None if t is None else t.float().cpu().numpy().astype(np.float64)
                           for t in (dq, dk, dv, dmc)))
    torch.cuda.synchronize()
    out = o.float().cpu().numpy().astype(np.float64)
    plan.close()
    return out, grads[0], grads[1]


def check(w, o, saved, recomputed, q, k, v, mc, do, *, bwd_tol, heads=None):
    for name, a, b in zip(NAMES, saved, recomputed):
        if a is None:
            assert b is None
            continue
        assert np.array_equal(a, b), (w.name, name, float(np.max(np.abs(a - b))))
    fo = oracle_full(w, q, k, v, mc, heads=heads)
    og = o if heads is None else np.stack([o[b, h] for b, h in heads])
    fwd_err = rel_err(og, fo)
    assert fwd_err <= FWD_TOL[w.dtype], (w.name, "o", fwd_err)
    want = oracle_backward(w, q, k, v, mc, do, heads=heads)
    errs = {}
    for name, g, r in zip(NAMES, saved, want):
        if r is None or g is None or (heads is not None and name == "dmc"):
            continue
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
        errs[name] = rel_err(g, r)
    print(f"  o={fwd_err:.2e} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + " (saved == recomputed)")
    record("backward_saved", w.name, o=fwd_err, **errs)
    for n, e in errs.items():
        assert e <= bwd_tol, (w.name, n, e)


CASES = [
    synth.Workload("bws_1d_m64", "bf16", 2, 2, 64, (4096,), (64,), 201, "softmax_l1"),
    synth.Workload("bws_2d_d128", "bf16", 1, 2, 128, (48, 48), (8, 8), 202, "softmax_gauss"),
    synth.Workload("bws_odd2d_d32", "bf16", 2, 2, 32, (30, 42), (5, 7), 203, "locality"),
    synth.Workload("bws_m300_valu", "bf16", 1, 1, 32, (4800,), (16,), 204, "softmax_gauss"),
    synth.Workload("bws_two_slices", "bf16", 1, 1, 64, (16384,), (512,), 205, "softmax_gauss"),
    synth.Workload("bws_unnorm", "bf16", 2, 2, 64, (32, 32), (4, 4), 206, "softmax_l1", "unnormalized"),
    synth.Workload("bws_relu_auto", "bf16", 1, 2, 64, (48, 48), (8, 8), 207, "softmax_l1", phi="relu"),
    synth.Workload("bws_fp32_auto", "fp32", 1, 2, 64, (24, 24), (4, 4), 208, "softmax_l1"),
    synth.Workload("bws_ragged_cls", "bf16", 1, 2, 64, (30, 34), (4, 4), 209, "softmax_gauss", ragged=True,
                   cls=True),
    synth.Workload("bws_mala", "bf16", 2, 2, 64, (32, 32), (32, 32), 210, "none", "mala"),
    synth.Workload("bws_mala_fp32", "fp32", 1, 2, 128, (900,), (900,), 211, "none", "mala"),
    # MHLA_ACCURACY_TRAIN: the readout at the bf16 level from the split mixed stack's high part
    synth.Workload("bws_1d_m64_train", "bf16", 2, 2, 64, (4096,), (64,), 213, "softmax_l1"),
    synth.Workload("bws_2d_d128_train", "bf16", 1, 2, 128, (48, 48), (8, 8), 214, "softmax_gauss"),
    synth.Workload("bws_m300_valu_train", "bf16", 1, 1, 32, (4800,), (16,), 215, "softmax_gauss"),
    synth.Workload("bws_relu_train", "bf16", 1, 2, 64, (48, 48), (8, 8), 216, "softmax_l1", phi="relu"),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_saved_matches_recompute(w):
    announce(f"backward saved {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} {w.readout} {w.phi}")
    q, k, v, mc, rng = synth.make_inputs(w)
    if w.phi == "relu":
        q = np.abs(q)
    do = synth.make_grad_output(w, rng)
    accuracy = ("auto" if w.name.endswith("_auto") or w.readout == "mala" else
                "train" if w.name.endswith("_train") else "split")
    o, saved, recomputed = run_saved_and_recompute(w, q, k, v, mc, do, accuracy=accuracy)
    check(w, o, saved, recomputed, q, k, v, mc, do, bwd_tol=FP32_TOL if w.dtype == "fp32" else BF16_TOL)


def test_backward_saved_per_head_mc_and_bf16_gradients():
    """A per-head M_c, and bf16 dO / gradients (bit-identical to the recomputing backward)."""
    w = synth.Workload("bws_per_head_bf16", "bf16", 2, 3, 64, (32, 64), (4, 8), 212, "none")
    announce(w.name)
    q, k, v, _, rng = synth.make_inputs(w)
    mc = rng.uniform(0.0, 1.0, (w.heads, w.n_blocks, w.n_blocks)).astype(np.float32).astype(np.float64)
    do = synth.make_grad_output(w, rng, "bf16")
    o, saved, recomputed = run_saved_and_recompute(w, q, k, v, mc, do, out_dtype="bf16")
    for name, a, b in zip(NAMES, saved, recomputed):
        assert np.array_equal(a, b), name
    want = oracle_backward(w, q, k, v, mc, do)
    for name, g, r in zip(NAMES[:3], saved[:3], want[:3]):
        rms = np.sqrt(np.mean(r ** 2))
        excess = np.abs(g - r) - (BF16_TOL * rms + 2.0 ** -8 * np.abs(r))
        assert excess.max() <= 0, (name, excess.max())
    assert rel_err(saved[3], want[3]) <= BF16_TOL


def test_backward_saved_long1d_full_size():
    """The long-sequence workload at full size with bf16 gradients, as the training leg of the
    benchmark runs it (MHLA_ACCURACY_TRAIN): the saved backward equals the recomputing one bit for
    bit over every head, and the forward's output and the gradients of heads 0 and 15 match the
    oracle."""
    w = synth.WORKLOADS["long1d"]
    announce(f"backward saved long1d shape={w.qkv_shape}")
    q, k, v, mc, rng = synth.make_inputs(w)
    do = synth.make_grad_output(w, rng, "bf16")
    o, saved, recomputed = run_saved_and_recompute(w, q, k, v, mc, do, out_dtype="bf16", accuracy="train")
    for name, a, b in zip(NAMES, saved, recomputed):
        assert np.array_equal(a, b), name
    heads = [(0, 0), (0, w.heads - 1)]
    fo = oracle_full(w, q, k, v, mc, heads=heads)
    fwd_err = rel_err(np.stack([o[b, h] for b, h in heads]), fo)
    assert fwd_err <= FWD_TOL["bf16"], fwd_err
    want = oracle_backward(w, q, k, v, mc, do, heads=heads)
    errs = {}
    for name, g, r in zip(NAMES[:3], saved[:3], want[:3]):
        g = np.stack([g[b, h] for b, h in heads])
        rms = np.sqrt(np.mean(r ** 2))
        excess = np.abs(g - r) - (BF16_TOL * rms + 2.0 ** -8 * np.abs(r))
        errs[name] = rel_err(g, r)
        assert excess.max() <= 0, (name, excess.max())
    print(f"  o={fwd_err:.2e} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + " (saved == recomputed)")
    record("backward_saved", "long1d", o=fwd_err, **errs)


def test_backward_saved_video3d_full_size():
    """The video workload at full size (32 heads, 64 blocks of 4 x 8 x 8 tokens) through the
    training step at MHLA_ACCURACY_TRAIN: bit-identical gradients to the recomputing backward,
    and the forward's output and every gradient against the oracle."""
    w = synth.WORKLOADS["video3d"]
    announce(f"backward saved video3d shape={w.qkv_shape}")
    q, k, v, mc, rng = synth.make_inputs(w)
    do = synth.make_grad_output(w, rng)
    o, saved, recomputed = run_saved_and_recompute(w, q, k, v, mc, do, accuracy="train")
    check(w, o, saved, recomputed, q, k, v, mc, do, bwd_tol=BF16_TOL)
