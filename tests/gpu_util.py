"""Helpers for GPU parity tests: upload seeded inputs, run the HIP library through its C ABI,
compare with the fp64 oracle."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

import oracle
import synth
import token_blocked_linear_amd as T


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        bits = synth.bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")


def run_hip(w: synth.Workload, q, k, v, mc, *, out_dtype="fp32", accuracy="auto", repeat=1):
    """One (or `repeat`) forward(s) through the C ABI; returns float64 numpy outputs."""
    import torch
    mc_per_head = mc is not None and np.ndim(mc) == 3
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=out_dtype, readout=w.readout, accuracy=accuracy, phi=w.phi,
                  mc_per_head=mc_per_head, ragged=w.ragged, cls_token=w.cls)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    ws = plan.alloc_workspace()
    outs = []
    for _ in range(repeat):
        o = torch.empty(w.qkv_shape, dtype=odt, device="cuda:0")
        plan.forward(tq, tk, tv, tmc, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    res = [o.float().cpu().numpy().astype(np.float64) for o in outs]
    plan.close()
    return res if repeat > 1 else res[0]


def rel_err(got, want):
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want))) / rms


def record(kind: str, case: str, **values) -> None:
    """Append one JSON line {kind, case, values...} to the file named by PARITY_METRICS_OUT (when
    set), so that a run's measured parity figures can be tabulated; numbers are rounded to 4
    significant digits."""
    path = os.environ.get("PARITY_METRICS_OUT")
    if not path:
        return
    vals = {k: (float(f"{v:.4g}") if isinstance(v, float) else v) for k, v in values.items()}
    with open(path, "a") as f:
        f.write(json.dumps({"kind": kind, "case": case, **vals}) + "\n")


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def oracle_geometry(w):
    """(grid, block) as the oracle takes them: a RaggedGrid for ragged blocks or a CLS token."""
    if w.ragged or w.cls:
        return oracle.RaggedGrid(w.grid, w.block, cls=w.cls), None
    return w.grid, w.block


def oracle_full(w, q, k, v, mc, heads=None):
    grid, block = oracle_geometry(w)
    if w.readout.startswith("causal"):
        mode = "unnormalized" if w.readout == "causal_unnormalized" else "normalized"
        return oracle.forward_causal(q, k, v, mc, grid, block, mode=mode, heads=heads, phi=w.phi)
    return oracle.forward(q, k, v, mc, grid, block, mode=w.readout, heads=heads, phi=w.phi)


def run_hip_backward(w: synth.Workload, q, k, v, mc, do, *, out_dtype="fp32", want_dmc=True, repeat=1):
    """Backward through the C ABI; returns float64 numpy (dq, dk, dv, dmc or None), or a list of
    such tuples for ``repeat`` > 1 (same inputs, fresh outputs every call)."""
    import torch
    mc_per_head = mc is not None and np.ndim(mc) == 3
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=out_dtype, readout=w.readout, phi=w.phi,
                  mc_per_head=mc_per_head, ragged=w.ragged, cls_token=w.cls)
    tq, tk, tv = (to_device(x, w.dtype) for x in (q, k, v))
    tdo = to_device(do, out_dtype)
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    ws = plan.alloc_backward_workspace()
    res = []
    for _ in range(repeat):
        dq, dk, dv = (torch.empty_like(tdo) for _ in range(3))
        dmc = torch.full(tuple(np.shape(mc)), float("nan"), device="cuda:0") if (want_dmc and mc is not None) else None
        plan.backward(tq, tk, tv, tmc, tdo, dq, dk, dv, dmc, ws)
        res.append((dq, dk, dv, dmc))
    torch.cuda.synchronize()
    out = [tuple(None if t is None else t.float().cpu().numpy().astype(np.float64) for t in r) for r in res]
    plan.close()
    return out if repeat > 1 else out[0]


def oracle_backward(w, q, k, v, mc, do, heads=None):
    grid, block = oracle_geometry(w)
    return oracle.backward(q, k, v, mc, grid, block, do, mode=w.readout, heads=heads, phi=w.phi)
