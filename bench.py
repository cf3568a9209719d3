"""Benchmark of the MHLA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long1d]

Defaults: 20 warm-up and 100 timed steps.

A step is one full forward (summary -> mixing -> readout) over one batch of seeded synthetic
input already resident in HBM.  Every workload of the metric's N = 4096 .. 65536 range (image,
image_mala, video3d, long1d) is timed; the headline `value` is long1d, the largest of them.
Per workload:
  - W untimed steps, then exactly K back-to-back steps between torch.cuda.synchronize() calls,
    with no per-kernel events: tokens/s = K * B * N / elapsed (the `value` of the headline);
  - a second pass of K steps with the library's HIP events around each kernel on the launch
    stream: per-kernel mean launch times, and from them each kernel's algorithmic bytes (or
    FLOPs) per launch over its mean duration;
  - a cold-cache pass: the median of single forwards with a 512 MiB scratch write in between.
`roofline` is the headline's dominant kernel, from the second pass.  The fp64 CPU oracle is
timed on a bounded sample of the headline workload (`cpu_baseline`).  One JSON line is printed.

`roofline.traffic` is the dominant kernel's measured HBM bytes per launch (FETCH_SIZE plus
WRITE_SIZE hardware counters, each scaled by what the counter reads for a plain copy of known
size), taken from profiles/traffic.md when that record was made from the current kernel sources
(same digest of the csrc/ files and the header), else null.

Beside the spec peaks (8 TB/s, 2.5 PFLOP/s bf16) the line carries rates measured in the same
run (`measured`): a 1 GiB non-temporal streaming read, a 1 GiB write and a 1 GiB copy through
the probe kernels of libmhla_peak.so, torch's 1 GiB device copy, a dense 8192^3 bf16 GEMM
through torch and a register-only loop of bf16 MFMAs.

`causal` times the chunkwise-causal forward on the long1d inputs.
`decode` times the streaming decode (mhla_decode_step, one position per call) of the long
sequence's heads (B = 1, 16 heads, d = 128, blocks of 256) over all 65536 positions, and of a
batch of 32 such sequences over 4096 positions: tokens/s by the wall clock (host launches
included) and the mean kernel time from HIP events against the algorithmic bytes.
`decode_prefill` times mhla_decode_prefill of the long sequence's 65536 positions in one call (the
prompt a decode would start from), by HIP events.
`backward` times mhla_backward (dQ, dK, dV, dM_c; gradients in the output dtype) on the long1d
inputs, K steps after W warm-ups, with per-kernel durations from the library's events.
`training` times a training step that keeps the forward's state: the forward at MHLA_ACCURACY_TRAIN
(split summaries and mixed summaries, what the backward recomputes), then mhla_backward_saved
from its workspace; `recompute_step_ms` beside it is the default forward plus mhla_backward.

    python bench.py --copy-calibration   # a plain 1 GiB device copy, for counter calibration
    python bench.py --digest             # digest of the kernel sources
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3
RANGE_WORKLOADS = ["image", "image_mala", "video3d", "long1d"]   # the N = 4096 .. 65536 configs
HEADLINE = "long1d"      # the largest single-GPU configuration of the metric: the `value`
# workloads whose bf16 output meets the plain 2e-2 bar by itself (asserted in the parity tests);
# the others are also timed with fp32 output, which meets it
BF16_OUT_PLAIN_BAR = {"long1d", "video3d", "image_mala", "deit_t"}


SOURCE_DIRS = ["token_blocked_linear_amd/csrc", "include"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.md")
TRAFFIC_TAG = "traffic-json: "


DIGEST_EXCLUDE = {"peak_probe.hip"}   # the measured-peak probe: not part of the MHLA path


def source_digest() -> str:
    """sha256 over the kernel and boundary sources (file names and contents, sorted)."""
    import hashlib
    h = hashlib.sha256()
    for d in SOURCE_DIRS:
        full = os.path.join(ROOT, d)
        for name in sorted(os.listdir(full)):
            if name.endswith((".hip", ".hpp", ".cpp", ".h")) and name not in DIGEST_EXCLUDE:
                h.update(name.encode())
                with open(os.path.join(full, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str, out_dtype: str):
    """Calibrated HBM bytes per launch from profiles/traffic.md, or None when absent or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = source_digest()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith(TRAFFIC_TAG):
                continue
            r = json.loads(line[len(TRAFFIC_TAG):])
            if (r.get("workload"), r.get("kernel"), r.get("out_dtype")) == (workload, kernel, out_dtype):
                return r["hbm_bytes_per_launch"] if r.get("source_digest") == digest else None
    return None


def measured_gemm_TFLOPs(n: int = 8192, reps: int = 10) -> float:
    """Dense bf16 GEMM rate measured now (torch.matmul of two contiguous n x n bf16 matrices,
    fp32 accumulation in the library): the practical MFMA ceiling, reported beside the spec peak."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.float32, generator=g).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device="cuda:0", dtype=torch.float32, generator=g).to(torch.bfloat16).contiguous()
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / t / 1e12


def measured_mfma_TFLOPs(blocks: int = 1024, iters: int = 1024, reps: int = 3):
    """Dense bf16 MFMA rate of a register-only loop (libmhla_peak.so): 1024 workgroups of 4 waves,
    each wave 8 * iters v_mfma_f32_16x16x32_bf16 (16384 flops each); best of `reps` timed launches
    after one warm-up.  None when the probe library is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "token_blocked_linear_amd", "libmhla_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mhla_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    flops = blocks * 4 * 8 * iters * 16384
    best = None
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.mhla_peak_mfma_bf16(blocks, iters, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        e1.synchronize()
        if st != 0:
            raise RuntimeError(f"mhla_peak_mfma_bf16: hip error {st}")
        if r > 0:
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
    return flops / best / 1e12


def measured_stream_GBps(n_bytes: int = 1 << 30, reps: int = 10):
    """Streaming rates of the probe kernels (libmhla_peak.so) over 1 GiB, best of `reps` after a
    warm-up: {"read": non-temporal loads, "write": default stores, "copy": read + write bytes}.
    None when the probe library is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "token_blocked_linear_amd", "libmhla_peak.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mhla_peak_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                     ctypes.c_void_p, ctypes.c_void_p]
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.empty(n_bytes // (64 << 10) * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for kind, name, moved in ((0, "read", n_bytes), (1, "write", n_bytes), (2, "copy", 2 * n_bytes)):
        best = None
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.mhla_peak_stream(kind, src.data_ptr(), dst.data_ptr(), n_bytes, sink.data_ptr(),
                                      stream.cuda_stream)
            e1.record(stream)
            e1.synchronize()
            if st != 0:
                raise RuntimeError(f"mhla_peak_stream: hip error {st}")
            if r > 0:
                t = e0.elapsed_time(e1) * 1e-3
                best = t if best is None else min(best, t)
        out[name] = round(moved / best / 1e9, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def measured_copy_GBps(n_bytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy bandwidth (read + write bytes / time) measured now: the practical
    HBM ceiling the kernels are also reported against."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n_bytes / t / 1e9


def copy_calibration(n_bytes: int = 1 << 30, reps: int = 10):
    """A plain device copy of known size: counters read on it calibrate FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "launches": reps}),
          flush=True)


def kernel_accounting(w: synth.Workload, out_bytes: int, split: bool = False):
    """Algorithmic bytes and FLOPs per launch of each kernel (summaries are not algorithmic).
    The mixing kernel contracts on MFMA (a bf16 stack, or fp32 partials as split operands up
    to 256 blocks); `split` with more blocks runs it on the VALU."""
    BH, N, d, M = w.batch * w.heads, w.n_tokens, w.head_dim, w.n_blocks
    in_b = 2 if w.dtype == "bf16" else 4
    tok = BH * N
    acc = {
        "summary": dict(bytes=tok * 2 * d * in_b, flops=tok * (2 * d * d + d), bound="hbm"),
        "readout": dict(bytes=tok * d * (in_b + out_bytes), flops=tok * (2 * d * d + 2 * d), bound="hbm"),
    }
    mix_bound = "alu" if split and (M > 256 or w.readout == "mala") else "mfma"
    if w.readout == "mala":
        acc["mix"] = dict(bytes=0, flops=BH * 2 * d * d, bound=mix_bound)
    else:
        acc["mix"] = dict(bytes=M * M * 4, flops=BH * 2 * M * M * (d * d + d), bound=mix_bound)
    # mixing step run in the readout's prologue: its inputs are summaries (not algorithmic),
    # so the fused kernel carries the readout's bytes plus M_c
    acc["mix+readout"] = dict(bytes=acc["readout"]["bytes"] + acc["mix"]["bytes"],
                              flops=acc["readout"]["flops"] + acc["mix"]["flops"], bound="hbm")
    # causal readout: Q, K, V read and O written; the state readout and update (2 d^2 each) plus
    # the in-sub-chunk term (scores and P V against up to SUB keys, SUB = 32 at d = 128, else 64)
    sub = 32 if d >= 128 else 64
    acc["causal"] = dict(bytes=tok * d * (3 * in_b + out_bytes), flops=tok * (4 * d * d + 2 * d * sub), bound="hbm")
    acc["scan"] = dict(bytes=0, flops=0, bound="hbm")
    if w.readout.startswith("causal"):
        acc["mix"]["bound"] = "mfma" if M <= 256 else "alu"
    total_bytes = tok * d * (3 * in_b + out_bytes) + (0 if w.readout == "mala" else M * M * 4)
    total_flops = acc["summary"]["flops"] + acc["mix+readout"]["flops"]
    return acc, total_bytes, total_flops


def to_dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0")


COLD_FLUSH_BYTES = 512 << 20


def cold_steps(plan, args_fwd, stream, n: int):
    """Median time of one forward with no input cache-resident: a 512 MiB scratch buffer is
    written between calls (outside the timed events), so Q, K, V come from HBM."""
    import torch
    scratch = torch.empty(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    times = []
    for i in range(n):
        scratch.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan.forward(*args_fwd, stream)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del scratch
    return float(np.median(times))


def _raw_forward(plan, q, k, v, mc, o, ws, stream):
    """A zero-argument callable issuing mhla_forward through the C ABI with the pointers bound
    once (the binding's per-call shape checks would add host time to short steps)."""
    import ctypes

    import token_blocked_linear_amd as T
    lib = T.load_library()
    args = (plan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(mc.data_ptr() if mc is not None else None),
            ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
            ctypes.c_void_p(stream.cuda_stream))
    fwd = lib.mhla_forward

    def call():
        st = fwd(*args)
        if st != 0:
            raise T.MhlaError(st, "mhla_forward")
    return call


# Which parity bar the timed output meets (tests/test_gpu_parity.py asserts each of these).
def parity_bar(name: str, out_dtype: str) -> str:
    if out_dtype == "fp32" or name in BF16_OUT_PLAIN_BAR:
        return "max|o-o_ref|/RMS(o_ref) <= 2e-2 (plain)"
    return ("|o-o_ref| <= 2e-2*RMS(o_ref) + 2^-8*|o_ref| per element (the bar plus the bf16 output's own "
            "rounding); the fp32 output meets the plain bar")


def run_workload(name: str, steps: int, warmup: int, out_dtype: str, n_cold: int = 20, inputs=None,
                 readout=None):
    """Pass 1: `steps` back-to-back forwards with no events (e2e time); pass 2: `steps` forwards
    with the library's per-kernel events (kernel times); then the cold-cache median."""
    import torch
    import token_blocked_linear_amd as T

    w = synth.WORKLOADS[name]
    if readout is not None:
        w = w.with_(readout=readout)
    q, k, v, mc = inputs if inputs is not None else synth.make_inputs(w)[:4]
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=out_dtype, readout=w.readout)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    tmc = None if mc is None else torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    o = torch.empty(w.qkv_shape, dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                    device="cuda:0")
    ws = plan.alloc_workspace()
    stream = torch.cuda.current_stream()
    plan.check_args(tq, tk, tv, tmc, o, ws)
    call = _raw_forward(plan, tq, tk, tv, tmc, o, ws, stream)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # pass 2: per-kernel events
    T.mhla_timing_reset(plan.handle)
    T.mhla_timing_enable(plan.handle, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    T.mhla_timing_enable(plan.handle, False)
    cold_s = cold_steps(plan, (tq, tk, tv, tmc, o, ws), stream, n_cold) if n_cold > 0 else None
    kernels = {}
    for i in range(plan.info.n_kernels):
        kname, ms, n = T.mhla_timing_read(plan.handle, i)
        kernels[kname] = ms / max(n, 1) * 1e-3          # mean seconds per launch
    ob = 2 if out_dtype == "bf16" else 4
    acc, total_bytes, total_flops = kernel_accounting(w, ob, bool(plan.info.split_operands))
    per_kernel = {kname: price(acc[kname], t) for kname, t in kernels.items()}
    step_s = elapsed / steps
    res = dict(
        workload=w, elapsed=elapsed, step_s=step_s, step_s_with_events=elapsed_ev / steps,
        tokens_per_s=w.batch * w.n_tokens / step_s,
        cold_step_s=cold_s,
        e2e_hbm_frac=total_bytes / step_s / (HBM_PEAK_GBS * 1e9),
        e2e_tflops=total_flops / step_s / 1e12,
        alg_bytes=total_bytes, alg_flops=total_flops,
        kernels=kernels, per_kernel=per_kernel, acc=acc, inputs=(q, k, v, mc),
        workspace_bytes=int(plan.workspace_bytes),
    )
    plan.close()
    del tq, tk, tv, tmc, o, ws
    torch.cuda.empty_cache()
    return res


def roofline_of(res, out_dtype: str):
    """The roofline object for a workload's dominant kernel (the longest mean launch)."""
    w = res["workload"]
    dom = max(res["kernels"], key=lambda k: res["kernels"][k])
    pk = res["per_kernel"][dom]
    a = res["acc"][dom]
    if pk["bound"] == "hbm":
        return {"bound": "hbm", "achieved": pk["alg_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": pk["frac"], "traffic": measured_traffic(w.name, dom, out_dtype), "kernel": dom,
                "alg_bytes_per_launch": a["bytes"], "mean_launch_us": pk["us"]}
    peak = BF16_MFMA_PEAK_TFLOPS if pk["bound"] == "mfma" else FP32_VALU_PEAK_TFLOPS
    return {"bound": pk["bound"], "achieved": pk["TFLOPs"], "peak": peak, "unit": "TFLOP/s",
            "frac": pk["frac"], "traffic": None, "kernel": dom,
            "alg_flops_per_launch": a["flops"], "mean_launch_us": pk["us"]}


def workload_record(res, out_dtype: str):
    w = res["workload"]
    return {"tokens_per_s": round(res["tokens_per_s"], 1), "ms_per_step": round(res["step_s"] * 1e3, 4),
            "ms_per_step_with_kernel_events": round(res["step_s_with_events"] * 1e3, 4),
            "cold_cache_ms": None if res["cold_step_s"] is None else round(res["cold_step_s"] * 1e3, 4),
            "e2e_hbm_frac": round(res["e2e_hbm_frac"], 4), "e2e_TFLOPs": round(res["e2e_tflops"], 2),
            "alg_bytes_per_step": int(res["alg_bytes"]),
            "config": {"batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "grid": list(w.grid),
                       "block": list(w.block), "n_blocks": w.n_blocks, "readout": w.readout,
                       "in_dtype": w.dtype, "out_dtype": out_dtype},
            "workspace_MiB": round(res["workspace_bytes"] / 2 ** 20, 1),
            "parity_bar_met": parity_bar(w.name, out_dtype),
            "roofline": roofline_of(res, out_dtype), "kernels": res["per_kernel"]}


def backward_accounting(w: synth.Workload, grad_bytes: int):
    """Algorithmic bytes and FLOPs per launch of each backward kernel.  Bytes count the problem's
    tensors only (Q, K, V, dO read; dQ, dK, dV, M_c, dM_c); the summaries and g = dO / den are
    intermediates of this decomposition and count as zero, as the forward's summaries do."""
    BH, N, d, M = w.batch * w.heads, w.n_tokens, w.head_dim, w.n_blocks
    in_b, ob = (2 if w.dtype == "bf16" else 4), grad_bytes
    tok = BH * N
    # split-operand MFMA mixing up to 256 blocks, VALU beyond
    mix = dict(bytes=M * M * 4, flops=BH * 2 * M * M * (d * d + d), bound="mfma" if M <= 256 else "alu")
    acc = {
        "bwd_summary": dict(bytes=tok * 2 * d * in_b, flops=tok * (2 * d * d + d), bound="hbm"),
        "bwd_mix": dict(mix),
        "bwd_dq": dict(bytes=tok * d * (in_b + 2 * ob), flops=tok * (4 * d * d + 6 * d), bound="hbm"),
        "bwd_dsummary": dict(bytes=tok * d * in_b, flops=tok * (2 * d * d + d), bound="hbm"),
        "bwd_dmix": dict(mix),
        "bwd_keyside": dict(bytes=tok * d * (2 * in_b + 2 * ob), flops=tok * (4 * d * d + 2 * d), bound="hbm"),
        "bwd_dmc": dict(bytes=M * M * 4, flops=BH * 2 * M * M * (d * d + d), bound="mfma"),
    }
    total_bytes = tok * d * (3 * in_b + 4 * ob) + 2 * M * M * 4
    total_flops = sum(a["flops"] for a in acc.values())
    return acc, total_bytes, total_flops


def price(a, t):
    """Achieved rates of one kernel (accounting `a`, mean seconds `t`) against its bound."""
    gbs = a["bytes"] / t / 1e9
    tfl = a["flops"] / t / 1e12
    if a["bound"] == "hbm":
        frac = gbs / HBM_PEAK_GBS
    elif a["bound"] == "mfma":
        frac = tfl / BF16_MFMA_PEAK_TFLOPS
    else:
        frac = tfl / FP32_VALU_PEAK_TFLOPS
    return dict(us=round(t * 1e6, 2), alg_GBps=round(gbs, 1), TFLOPs=round(tfl, 2), bound=a["bound"],
                frac=round(frac, 4))


def run_backward(name: str, steps: int, warmup: int, grad_dtype: str, inputs):
    """The backward (dQ, dK, dV, dM_c) on the same inputs, dO seeded per workload; per-kernel
    durations from the library's HIP events on the launch stream."""
    import torch
    import token_blocked_linear_amd as T

    w = synth.WORKLOADS[name]
    q, k, v, mc = inputs
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=grad_dtype, readout=w.readout)
    do = synth.make_grad_output(w, np.random.default_rng(w.seed + 1000), grad_dtype)
    tq, tk, tv, tdo = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(do, grad_dtype)
    tmc = None if mc is None else torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    dq, dk, dv = (torch.empty_like(tdo) for _ in range(3))
    dmc = None if tmc is None else torch.empty_like(tmc)
    ws = plan.alloc_backward_workspace()
    stream = torch.cuda.current_stream()
    call = (tq, tk, tv, tmc, tdo, dq, dk, dv, dmc, ws, stream)
    for _ in range(warmup):
        plan.backward(*call)
    torch.cuda.synchronize()
    t0 = time.perf_counter()        # pass 1: no events
    for _ in range(steps):
        plan.backward(*call)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    T.mhla_timing_reset(plan.handle)   # pass 2: per-kernel events
    T.mhla_timing_enable(plan.handle, True)
    for _ in range(steps):
        plan.backward(*call)
    torch.cuda.synchronize()
    T.mhla_timing_enable(plan.handle, False)
    ob = 2 if grad_dtype == "bf16" else 4
    acc, total_bytes, total_flops = backward_accounting(w, ob)
    per_kernel = {}
    for i in range(7):
        kname, ms, n = T.mhla_backward_timing_read(plan.handle, i)
        per_kernel[kname] = price(acc[kname], ms / max(n, 1) * 1e-3)
    plan.close()
    step_s = elapsed / steps
    dom = max(per_kernel, key=lambda k: per_kernel[k]["us"])
    pk, a = per_kernel[dom], acc[dom]
    if pk["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": pk["alg_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": pk["frac"], "kernel": dom, "alg_bytes_per_launch": a["bytes"], "mean_launch_us": pk["us"]}
    else:
        peak = BF16_MFMA_PEAK_TFLOPS if pk["bound"] == "mfma" else FP32_VALU_PEAK_TFLOPS
        roof = {"bound": pk["bound"], "achieved": pk["TFLOPs"], "peak": peak, "unit": "TFLOP/s",
                "frac": pk["frac"], "kernel": dom, "alg_flops_per_launch": a["flops"], "mean_launch_us": pk["us"]}
    return {"grad_dtype": grad_dtype, "ms_per_step": round(step_s * 1e3, 4),
            "tokens_per_s": round(w.batch * w.n_tokens / step_s, 1),
            "e2e_alg_hbm_frac": round(total_bytes / step_s / (HBM_PEAK_GBS * 1e9), 4),
            "e2e_TFLOPs": round(total_flops / step_s / 1e12, 2),
            "roofline": roof, "kernels": per_kernel}


def run_training(name: str, steps: int, warmup: int, grad_dtype: str, inputs):
    """A training step from the forward's saved state: the forward at MHLA_ACCURACY_TRAIN (split
    summaries and mixing, what the backward would recompute; the readout at the bf16 level from
    the mixed stack's high part), then mhla_backward_saved
    from its workspace.  Timed three ways with no events (forward alone, saved backward alone,
    the pair back to back), then the saved backward's kernels with the library's events."""
    import torch
    import token_blocked_linear_amd as T

    w = synth.WORKLOADS[name]
    q, k, v, mc = inputs
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype=grad_dtype, readout=w.readout, accuracy="train")
    do = synth.make_grad_output(w, np.random.default_rng(w.seed + 1000), grad_dtype)
    tq, tk, tv, tdo = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), to_dev(do, grad_dtype)
    tmc = None if mc is None else torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    o = torch.empty_like(tdo)
    dq, dk, dv = (torch.empty_like(tdo) for _ in range(3))
    dmc = None if tmc is None else torch.empty_like(tmc)
    fws = plan.alloc_workspace()
    bws = plan.alloc_backward_saved_workspace()
    stream = torch.cuda.current_stream()

    def fwd():
        plan.forward(tq, tk, tv, tmc, o, fws, stream)

    def bwd():
        plan.backward(tq, tk, tv, tmc, tdo, dq, dk, dv, dmc, bws, stream, fwd_workspace=fws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    t_fwd = timed(fwd)
    t_bwd = timed(bwd)                 # the workspace holds the last forward's state
    t_step = timed(lambda: (fwd(), bwd()))
    T.mhla_timing_reset(plan.handle)
    T.mhla_timing_enable(plan.handle, True)
    for _ in range(steps):
        bwd()
    torch.cuda.synchronize()
    T.mhla_timing_enable(plan.handle, False)
    ob = 2 if grad_dtype == "bf16" else 4
    acc, _, _ = backward_accounting(w, ob)
    per_kernel = {}
    for i in range(7):
        kname, ms, n = T.mhla_backward_timing_read(plan.handle, i)
        if kname in ("bwd_summary", "bwd_mix"):
            continue                   # read from the forward's workspace: not launched
        per_kernel[kname] = price(acc[kname], ms / max(n, 1) * 1e-3)
    plan.close()
    return {"grad_dtype": grad_dtype, "forward_train_ms": round(t_fwd * 1e3, 4),
            "backward_saved_ms": round(t_bwd * 1e3, 4), "step_ms": round(t_step * 1e3, 4),
            "tokens_per_s": round(w.batch * w.n_tokens / t_step, 1), "kernels": per_kernel,
            "protocol": "forward at accuracy train (split summaries and mixing kept in its workspace), then "
                        "mhla_backward_saved from its workspace; each of the three times is K calls with "
                        "no events after W warm-up calls; kernels from a fourth pass with the library's events"}


def decode_accounting(BH: int, d: int, nb: int, t0: int, t1: int, in_b: int, out_b: int) -> int:
    """Algorithmic bytes of decode calls t0 .. t1-1 over BH (batch, head) pairs.  Every token
    reads S~< and R and writes R (fp32 d x d each), reads z~< and r and writes r, reads q, k, v
    and writes o; the first token of block i > 0 also reads the finished R, writes it as S_{i-1},
    reads S_0 .. S_{i-2}, writes S~<_i and writes the restarted R: 4 d^2 (i + 3) bytes."""
    per_tok = 12 * d * d + 12 * d + 3 * d * in_b + d * out_b
    total = (t1 - t0) * per_tok
    for i in range(max(1, -(-t0 // nb)), (t1 - 1) // nb + 1):
        total += 4 * d * d * (i + 3) + 12 * d
    return BH * total


def run_decode(batch: int, heads: int, d: int, n: int, nb: int, seed: int, pool: int = 512,
               in_dtype: str = "bf16", out_dtype: str = "bf16"):
    """Streaming decode through positions 0 .. n-1 of a causal plan (blocks of nb tokens), one
    mhla_decode_step per position.  The inputs of position t are pool[t % pool] (seeded N(0, 1);
    the cost does not depend on the values).  One untimed pass, then a pass timed by the wall
    clock (host launches included: tokens/s) and a pass with HIP events around every call on the
    launch stream (mean time per call, event overhead included, against the algorithmic bytes)."""
    import ctypes

    import torch
    import token_blocked_linear_amd as T

    w = synth.Workload("decode", in_dtype, batch, heads, d, (n,), (nb,), seed, "softmax_gauss", "causal",
                       ragged=n % nb != 0)
    plan = T.Plan(grid=w.grid, block=w.block, batch=batch, heads=heads, head_dim=d, in_dtype=in_dtype,
                  out_dtype=out_dtype, readout="causal", ragged=w.ragged)
    mc = synth.make_mc(w, np.random.default_rng(seed))
    tmc = torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    shape = (pool, batch, heads, d)
    tq, tk, tv = (to_dev(synth.standard_normal_parallel(shape, seed + 1 + i, bf16=in_dtype == "bf16"), in_dtype)
                  for i in range(3))
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    o = torch.empty((pool, batch, heads, d), dtype=odt, device="cuda:0")
    state = plan.alloc_decode_state()
    nbytes = state.numel()
    stream = torch.cuda.current_stream()
    lib = T.load_library()
    ib, ob = tq.element_size() * batch * heads * d, o.element_size() * batch * heads * d
    qp, kp, vp, op = tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr()
    args = (plan.handle, state.data_ptr(), nbytes)
    mcp, sp = ctypes.c_void_p(tmc.data_ptr()), ctypes.c_void_p(stream.cuda_stream)
    step = lib.mhla_decode_step

    def one(t):
        j = t % pool
        st = step(*args, t, qp + j * ib, kp + j * ib, vp + j * ib, mcp, op + j * ob, sp)
        if st != 0:
            raise T.MhlaError(st, "mhla_decode_step")

    for _ in range(2):          # untimed pass, then the wall-clock pass
        plan.decode_reset(state)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(n):
            one(t)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    plan.decode_reset(state)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(1024)]
    kern = 0.0
    for base in range(0, n, len(ev)):
        cnt = min(len(ev), n - base)
        for j in range(cnt):
            ev[j][0].record(stream)
            one(base + j)
            ev[j][1].record(stream)
        torch.cuda.synchronize()
        kern += sum(a.elapsed_time(b) for a, b in ev[:cnt]) * 1e-3
    plan.close()
    in_b, out_b = (2 if in_dtype == "bf16" else 4), (2 if out_dtype == "bf16" else 4)
    alg = decode_accounting(batch * heads, d, nb, 0, n, in_b, out_b)
    gbs = alg / kern / 1e9
    return {"batch": batch, "heads": heads, "head_dim": d, "positions": n, "block_tokens": nb,
            "n_blocks": w.n_blocks, "in_dtype": in_dtype, "out_dtype": out_dtype,
            "state_MiB": round(nbytes / 2 ** 20, 1),
            "wall_us_per_token": round(wall / n * 1e6, 3),
            "tokens_per_s": round(batch * n / wall, 1),
            "event_us_mean": round(kern / n * 1e6, 3),
            "alg_bytes_per_call_mean": int(alg / n),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def run_prefill(batch: int, heads: int, d: int, n: int, nb: int, seed: int, reps: int = 5):
    """mhla_decode_prefill over positions 0 .. n-1 (one call: the chunkwise causal forward at split
    accuracy plus the state's assembly), the median of `reps` calls timed by HIP events on the
    launch stream after one untimed call; against n single decode steps this is what a prompt of n
    positions costs before decoding continues."""
    import torch
    import token_blocked_linear_amd as T

    w = synth.Workload("prefill", "bf16", batch, heads, d, (n,), (nb,), seed, "softmax_gauss", "causal",
                       ragged=n % nb != 0)
    plan = T.Plan(grid=w.grid, block=w.block, batch=batch, heads=heads, head_dim=d, in_dtype="bf16",
                  out_dtype="bf16", readout="causal", ragged=w.ragged)
    mc = synth.make_mc(w, np.random.default_rng(seed))
    tmc = torch.from_numpy(mc.astype(np.float32)).to("cuda:0")
    shape = (batch, heads, n, d)
    tq, tk, tv = (to_dev(synth.standard_normal_parallel(shape, seed + 1 + i, bf16=True), "bf16") for i in range(3))
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    state = plan.alloc_decode_state()
    ws = plan.alloc_prefill_workspace(n)
    stream = torch.cuda.current_stream()
    plan.decode_prefill(state, tq, tk, tv, tmc, o, ws, stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.decode_prefill(state, tq, tk, tv, tmc, o, ws, stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    plan.close()
    ms = float(np.median(times))
    return {"batch": batch, "heads": heads, "head_dim": d, "positions": n, "block_tokens": nb,
            "ms": round(ms, 4), "tokens_per_s": round(batch * n / (ms * 1e-3), 1),
            "protocol": f"median of {reps} calls by HIP events after one untimed call; bf16 inputs and outputs"}


def blas_build() -> str:
    """The BLAS numpy is linked against, as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            return f"{i.get('internal_api')} {i.get('version')} ({os.path.basename(i.get('filepath', ''))}, " \
                   f"{i.get('threading_layer', '?')} threading, {i.get('num_threads')} threads)"
    except Exception:  # noqa: BLE001 - informational only
        pass
    return "unknown"


def cpu_baseline(res, budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on a bounded sample: whole (batch, head) pairs, cycled
    until the time budget is used.  NumPy's BLAS is given every host core."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    w = res["workload"]
    q, k, v, mc = res["inputs"]
    host_cores = os.cpu_count() or 1
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    with threadpool_limits(limits=host_cores, user_api="blas"):
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            p = pairs[done % len(pairs)]
            oracle.forward(q, k, v, mc, w.grid, w.block, mode=w.readout, heads=[p])
            done += 1
        t = time.perf_counter() - t0
    # one (batch, head) pair is 1/H of the work of N tokens in the metric's unit (B*N tokens,
    # every token carrying all H heads)
    return {"value": round(done * w.n_tokens / w.heads / t, 1), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "host_cores": host_cores, "blas": blas_build(),
            "sample": f"{done} whole (batch, head) pairs of {w.name} ({w.n_tokens} tokens each) in "
                      f"{t:.1f} s, counted as {done}/{w.heads} of the heads of {w.n_tokens} tokens"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(synth.WORKLOADS),
                    help="the headline workload (`value`); the metric's other workloads are timed beside it")
    ap.add_argument("--only", action="store_true", help="time the headline workload alone")
    ap.add_argument("--out-dtype", default="bf16", choices=["fp32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-causal", action="store_true", help="skip the causal-readout measurement")
    ap.add_argument("--no-decode", action="store_true", help="skip the streaming-decode measurement")
    ap.add_argument("--no-measured-rates", action="store_true",
                    help="skip the copy / GEMM / MFMA-loop rate probes (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--digest", action="store_true")
    args = ap.parse_args()

    if args.digest:
        print(source_digest())
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
        return

    def progress(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    progress(f"{args.workload} ({args.out_dtype} output)")
    res = run_workload(args.workload, args.steps, args.warmup, args.out_dtype)
    w = res["workload"]
    roof = roofline_of(res, args.out_dtype)
    head_rec = workload_record(res, args.out_dtype)

    progress("measured rates")
    if args.no_measured_rates:
        stream_rates, copy_bw, gemm_tf, mfma_tf = None, float("nan"), float("nan"), None
    else:
        stream_rates = measured_stream_GBps()
        copy_bw = measured_copy_GBps()
        gemm_tf = measured_gemm_TFLOPs()
        mfma_tf = measured_mfma_TFLOPs()
    measured = {"read_GBps": None if stream_rates is None else stream_rates["read"],
                "write_GBps": None if stream_rates is None else stream_rates["write"],
                "copy_kernel_GBps": None if stream_rates is None else stream_rates["copy"],
                "torch_copy_GBps": round(copy_bw, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
                "bf16_mfma_loop_TFLOPs": None if mfma_tf is None else round(mfma_tf, 1),
                "protocol": "1 GiB each; read = non-temporal 16-byte loads, write = default stores, copy = "
                            "read + write bytes; best of 10 launches after a warm-up"}
    roof["measured_copy_GBps"] = round(copy_bw, 1)
    if roof["unit"] == "GB/s":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_bw, 4)
    elif roof["bound"] == "mfma":
        roof["frac_of_measured_gemm"] = round(roof["achieved"] / gemm_tf, 4)

    workloads = {w.name: head_rec}
    if not args.only:
        for name in RANGE_WORKLOADS:
            if name == args.workload:
                continue
            progress(f"{name} ({args.out_dtype} output)")
            r = run_workload(name, args.steps, args.warmup, args.out_dtype)
            workloads[name] = workload_record(r, args.out_dtype)
            if args.out_dtype == "bf16" and name not in BF16_OUT_PLAIN_BAR:
                progress(f"{name} (fp32 output)")
                r2 = run_workload(name, args.steps, args.warmup, "fp32", inputs=r["inputs"])
                workloads[f"{name}_fp32_output"] = workload_record(r2, "fp32")
                del r2
            del r

    # the headline with fp32 output (10 d bytes per token-head)
    other_out = "fp32" if args.out_dtype == "bf16" else "bf16"
    progress(f"{args.workload} ({other_out} output)")
    r2 = run_workload(args.workload, args.steps, args.warmup, other_out, inputs=res["inputs"])
    alt = workload_record(r2, other_out)
    del r2

    causal = None
    if w.ndim == 1 and w.readout == "normalized" and not args.no_causal:
        progress("causal forward")
        rc = run_workload(args.workload, args.steps, args.warmup, args.out_dtype, n_cold=0, inputs=res["inputs"],
                          readout="causal")
        causal = {"readout": "causal (normalised)", "ms_per_step": round(rc["step_s"] * 1e3, 4),
                  "ms_per_step_with_kernel_events": round(rc["step_s_with_events"] * 1e3, 4),
                  "tokens_per_s": round(rc["tokens_per_s"], 1), "kernels": rc["per_kernel"]}
        del rc

    decode = None
    if not args.no_decode:
        progress("decode")
        # the long sequence's heads decoded one position at a time (B = 1), and a batch of 32
        # such sequences over their first 4096 positions
        decode = [run_decode(1, 16, 128, 65536, 256, 701), run_decode(32, 16, 128, 4096, 256, 702)]
        progress("decode prefill")
        prefill = run_prefill(1, 16, 128, 65536, 256, 703)

    bwd = train = None
    if not args.no_backward and w.readout != "mala":
        progress("backward")
        bwd = run_backward(args.workload, args.steps, args.warmup, args.out_dtype, res["inputs"])
        progress("training step from the forward's saved state")
        train = run_training(args.workload, args.steps, args.warmup, args.out_dtype, res["inputs"])
        train["recompute_step_ms"] = round(res["step_s"] * 1e3 + bwd["ms_per_step"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu baseline")
        cpu = cpu_baseline(res)
    line = {
        "metric": "MHLA fwd tokens/sec + % of bf16 MFMA/HBM roofline at N=4096..65536",
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["step_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V rounded to bf16; M_c from the workload's generator)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "grid": list(w.grid), "block": list(w.block), "n_blocks": w.n_blocks,
                   "tokens_per_step": w.batch * w.n_tokens, "readout": w.readout,
                   "in_dtype": w.dtype, "out_dtype": args.out_dtype, "parallelism": "single-gpu"},
        "roofline": roof,
        "end_to_end": {"alg_hbm_frac": round(res["e2e_hbm_frac"], 4), "TFLOPs": round(res["e2e_tflops"], 2),
                       "alg_bytes_per_step": int(res["alg_bytes"])},
        "cold_cache": {"ms_per_step_median": round(res["cold_step_s"] * 1e3, 4),
                       "tokens_per_s": round(w.batch * w.n_tokens / res["cold_step_s"], 1),
                       "protocol": "median of 20 single forwards timed by HIP events on the launch stream, "
                                   "a 512 MiB scratch buffer written between them"},
        "timing_passes": "value / ms_per_step: K back-to-back forwards with no per-kernel events; kernels and "
                         "roofline: a second pass of K forwards with the library's events around each kernel",
        "parity_bar_met": parity_bar(w.name, args.out_dtype),
        "kernels": res["per_kernel"],
        "workloads": workloads,
        "measured": measured,
        "cpu_baseline": cpu,
    }
    line[f"{other_out}_output"] = alt
    if bwd is not None:
        line["backward"] = bwd
        line["training"] = train
    if causal is not None:
        line["causal"] = causal
    if decode is not None:
        line["decode"] = decode
        line["decode_prefill"] = prefill
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
