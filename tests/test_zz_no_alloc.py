"""mhla_forward_noalloc (the forward with the library's own scratch array as workspace) against
mhla_forward with a caller-owned workspace, through the C ABI: two calls in a row, the second on
a smaller input, each bit-equal to the existing entry point's output (same kernels, fixed
summation order); a plan whose workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest

import token_blocked_linear_amd as T

pytestmark = pytest.mark.gpu


def _inputs(plan_kw, seed):
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    n = int(np.prod(plan_kw["grid"]))
    shape = (plan_kw["batch"], plan_kw["heads"], n, plan_kw["head_dim"])
    q, k, v = (torch.randn(shape, device="cuda:0", generator=g).to(torch.bfloat16) for _ in range(3))
    return q, k, v


def _mc(plan, seed):
    import torch
    m = int(plan.info.n_blocks)
    if m == 1:
        return None
    g = torch.Generator(device="cuda:0").manual_seed(seed + 1)
    return torch.softmax(torch.randn(m, m, device="cuda:0", generator=g), dim=1).contiguous()


def _both(plan_kw, seed):
    """(noalloc output, mhla_forward output) for one plan; the C ABI called directly."""
    import torch
    lib = T.load_library()
    plan = T.Plan(**plan_kw)
    q, k, v = _inputs(plan_kw, seed)
    mc = _mc(plan, seed)
    out_dt = torch.bfloat16 if plan_kw.get("out_dtype") == "bf16" else torch.float32
    o_na = torch.full(q.shape, float("nan"), dtype=out_dt, device="cuda:0")
    o_ref = torch.full(q.shape, float("nan"), dtype=out_dt, device="cuda:0")
    stream = torch.cuda.current_stream()
    P = ctypes.c_void_p
    mcp = P(mc.data_ptr() if mc is not None else None)
    st = lib.mhla_forward_noalloc(plan.handle, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), mcp,
                                  P(o_na.data_ptr()), P(stream.cuda_stream))
    assert st == T.MHLA_OK, T.mhla_status_string(st)
    ws = plan.alloc_workspace()
    st = lib.mhla_forward(plan.handle, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), mcp, P(o_ref.data_ptr()),
                          P(ws.data_ptr()), ctypes.c_size_t(ws.numel()), P(stream.cuda_stream))
    assert st == T.MHLA_OK, T.mhla_status_string(st)
    torch.cuda.synchronize()
    res = o_na.float().cpu().numpy(), o_ref.float().cpu().numpy(), plan.workspace_bytes
    plan.close()
    return res


BIG = dict(grid=(16, 32, 32), block=(4, 8, 8), batch=2, heads=16, head_dim=64, in_dtype="bf16", out_dtype="bf16")
SMALL = dict(grid=(1000,), block=(200,), batch=1, heads=3, head_dim=128, in_dtype="bf16", out_dtype="fp32")
LONG = dict(grid=(65536,), block=(256,), batch=1, heads=16, head_dim=128, in_dtype="bf16", out_dtype="bf16")


def test_noalloc_matches_forward_then_smaller_input():
    print("[gpu-case] noalloc: video-shaped plan, then a smaller 1D plan", flush=True)
    a_na, a_ref, ws_a = _both(BIG, 11)
    assert np.all(np.isfinite(a_ref))
    assert np.array_equal(a_na, a_ref)
    b_na, b_ref, ws_b = _both(SMALL, 12)
    assert ws_b < ws_a
    assert np.all(np.isfinite(b_ref))
    assert np.array_equal(b_na, b_ref)


def test_noalloc_long_sequence_fits():
    """The 65536-token, 16-head sequence (132 MiB of workspace) runs from the array."""
    print("[gpu-case] noalloc: long 1D plan", flush=True)
    a_na, a_ref, ws = _both(LONG, 13)
    assert ws <= T.MHLA_NOALLOC_SCRATCH_BYTES
    assert np.array_equal(a_na, a_ref)


def test_noalloc_refuses_a_workspace_beyond_the_array():
    import torch
    print("[gpu-case] noalloc: oversize plan refused", flush=True)
    kw = dict(grid=(65536,), block=(256,), batch=2, heads=16, head_dim=128, in_dtype="bf16", out_dtype="bf16")
    plan = T.Plan(**kw)
    assert plan.workspace_bytes > T.MHLA_NOALLOC_SCRATCH_BYTES
    # full-size buffers (refused before any launch, but sized for the plan all the same)
    shape = (2, 16, 65536, 128)
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
    o = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda:0")
    mc = torch.ones(256, 256, device="cuda:0") / 256
    P = ctypes.c_void_p
    st = T.load_library().mhla_forward_noalloc(plan.handle, P(q.data_ptr()), P(q.data_ptr()), P(q.data_ptr()),
                                               P(mc.data_ptr()), P(o.data_ptr()),
                                               P(torch.cuda.current_stream().cuda_stream))
    assert st == T.MHLA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0))
    plan.close()
