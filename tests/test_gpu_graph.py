"""The library's calls under HIP graph capture.

The forward, the causal forward, the backward and the backward from saved state launch kernels only: no allocation, no
memset, no host synchronisation. A graph captured once (torch.cuda.graph around the call, on
torch's capture stream) must therefore reproduce the eager call. Each test replays the graph
several times. Before each replay it copies fresh inputs into the captured buffers, eagerly and
followed by a synchronisation. Every replay must equal an eager call on the same inputs bit for
bit, since every kernel reduces in a fixed order.
"""
import numpy as np
import pytest

import synth
from gpu_util import announce, to_device
import token_blocked_linear_amd as T

pytestmark = pytest.mark.gpu


def _plan(w, **kw):
    return T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype="fp32", readout=w.readout, phi=w.phi, **kw)


@pytest.mark.parametrize("w", [
    synth.Workload("g_image_small", "bf16", 2, 4, 64, (32, 64), (16, 16), 801, "softmax_l1"),
    synth.Workload("g_mix_kernel", "bf16", 1, 2, 64, (4096,), (64,), 802, "softmax_gauss"),
    synth.Workload("g_causal", "bf16", 1, 2, 128, (2048,), (256,), 803, "softmax_gauss", "causal"),
    synth.Workload("g_mala", "fp32", 1, 2, 64, (32, 32), (32, 32), 804, "none", "mala"),
], ids=lambda w: w.name)
def test_forward_graph_replays_equal_eager(w):
    import torch
    announce(f"graph forward {w.name} shape={w.qkv_shape} {w.readout}")
    plan = _plan(w)
    ws = plan.alloc_workspace()
    rng = np.random.default_rng(w.seed)
    q, k, v, mc, _ = synth.make_inputs(w)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tmc = None if mc is None else torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    o = torch.empty(w.qkv_shape, dtype=torch.float32, device="cuda:0")
    plan.forward(tq, tk, tv, tmc, o, ws)          # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(tq, tk, tv, tmc, o, ws)
    torch.cuda.synchronize()
    o_eager = torch.empty_like(o)
    for rep in range(3):
        fresh = [rng.standard_normal(w.qkv_shape).astype(np.float32) for _ in range(3)]
        for dst, x in zip((tq, tk, tv), fresh):
            dst.copy_(to_device(x, w.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        plan.forward(tq, tk, tv, tmc, o_eager, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), (w.name, rep)
        assert bool(torch.isfinite(o).all())
    plan.close()


def test_backward_graph_replays_equal_eager():
    import torch
    w = synth.Workload("g_backward", "bf16", 1, 2, 64, (64, 64), (16, 16), 805, "softmax_l1")
    announce(f"graph backward {w.name} shape={w.qkv_shape}")
    plan = _plan(w)
    ws = plan.alloc_backward_workspace()
    rng = np.random.default_rng(w.seed)
    q, k, v, mc, _ = synth.make_inputs(w)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tdo = to_device(synth.make_grad_output(w, rng), "fp32")
    tmc = torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    outs = [torch.empty_like(tdo) for _ in range(3)] + [torch.empty_like(tmc)]
    plan.backward(tq, tk, tv, tmc, tdo, *outs, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.backward(tq, tk, tv, tmc, tdo, *outs, ws)
    torch.cuda.synchronize()
    eager = [torch.empty_like(x) for x in outs]
    for rep in range(3):
        tdo.copy_(to_device(rng.standard_normal(w.qkv_shape), "fp32"))
        tq.copy_(to_device(rng.standard_normal(w.qkv_shape).astype(np.float32), w.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        plan.backward(tq, tk, tv, tmc, tdo, *eager, ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dmc"), outs, eager):
            assert torch.equal(a, b), (name, rep)
    plan.close()


def test_training_step_graph_replays_equal_eager():
    """The training step, captured as one graph: the forward at MHLA_ACCURACY_TRAIN, then the
    backward from its saved state.  Every replay equals the eager pair on the same inputs."""
    import torch
    w = synth.Workload("g_train", "bf16", 1, 2, 64, (4096,), (64,), 806, "softmax_gauss")
    announce(f"graph training step {w.name} shape={w.qkv_shape}")
    plan = _plan(w, accuracy="train")
    fws, bws = plan.alloc_workspace(), plan.alloc_backward_saved_workspace()
    rng = np.random.default_rng(w.seed)
    q, k, v, mc, _ = synth.make_inputs(w)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tdo = to_device(synth.make_grad_output(w, rng), "fp32")
    tmc = torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    o = torch.empty_like(tdo)
    outs = [torch.empty_like(tdo) for _ in range(3)] + [torch.empty_like(tmc)]

    def step(o_, grads):
        plan.forward(tq, tk, tv, tmc, o_, fws)
        plan.backward(tq, tk, tv, tmc, tdo, *grads, bws, fwd_workspace=fws)

    step(o, outs)                                  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(o, outs)
    torch.cuda.synchronize()
    o_eager = torch.empty_like(o)
    eager = [torch.empty_like(x) for x in outs]
    for rep in range(3):
        tdo.copy_(to_device(rng.standard_normal(w.qkv_shape), "fp32"))
        for dst in (tq, tk, tv):
            dst.copy_(to_device(rng.standard_normal(w.qkv_shape).astype(np.float32), w.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(o_eager, eager)
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), ("o", rep)
        for name, a, b in zip(("dq", "dk", "dv", "dmc"), outs, eager):
            assert torch.equal(a, b), (name, rep)
    plan.close()
