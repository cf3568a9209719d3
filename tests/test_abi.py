"""The C-ABI library on the host (no GPU needed): it loads, exports every function the header
declares, validates descriptors and forward arguments before any launch, and its host-side
fast division is exact."""
import ctypes
import os
import re
import subprocess

import pytest

import token_blocked_linear_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhla.h")


def _lib_or_skip():
    if not os.path.exists(T.library_path()):
        pytest.skip("libmhla.so is not built (run __graft_entry__.build())")
    return T.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mhla_status|const char\*)\s+(mhla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(T.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    _lib_or_skip()
    out = subprocess.run(["nm", "-D", "--defined-only", T.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(mhla_\w+)$", out, re.M))
    for name in _declared_functions():
        assert name in exported, name


def test_peak_probe_library_exports_its_entry():
    """The benchmark's MFMA-loop probe is a library of its own, built beside libmhla.so."""
    path = os.path.join(os.path.dirname(T.library_path()), "libmhla_peak.so")
    if not os.path.exists(path):
        pytest.skip("libmhla_peak.so is not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    assert re.search(r"\sT\smhla_peak_mfma_bf16$", out, re.M)


def test_struct_layouts_match_header():
    # mhla_desc: 8 x int32 (incl. struct_size) + 2 x int64[3] + 3 x int64 + 2 x int32
    #   = 32 + 48 + 24 + 8
    assert ctypes.sizeof(T.MhlaDesc) == 112
    assert T.MhlaDesc.flags.offset == 104
    assert ctypes.sizeof(T.MhlaPlanInfo) == 56


def _desc(**kw):
    base = dict(grid=(64, 64), block=(16, 16), batch=16, heads=8, head_dim=64)
    base.update(kw)
    return T.make_desc(**base)


def _status(desc):
    lib = _lib_or_skip()
    h = ctypes.c_void_p()
    st = lib.mhla_create(ctypes.byref(desc), ctypes.byref(h))
    if st == 0:
        lib.mhla_destroy(h)
    return st


def test_create_accepts_workload_shapes():
    import synth
    for w in synth.WORKLOADS.values():
        d = T.make_desc(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                        in_dtype=w.dtype, out_dtype="fp32", readout=w.readout)
        assert _status(d) == T.MHLA_OK, w.name


@pytest.mark.parametrize("mutate,want", [
    (lambda d: setattr(d, "struct_size", 8), 1),
    (lambda d: setattr(d, "in_dtype", 7), 2),
    (lambda d: setattr(d, "out_dtype", -1), 2),
    (lambda d: setattr(d, "phi", 3), 2),
    (lambda d: setattr(d, "readout", 9), 2),
    (lambda d: setattr(d, "accuracy", 5), 2),
    (lambda d: setattr(d, "accuracy", 4), 2),
    (lambda d: setattr(d, "head_dim", 48), 2),
    (lambda d: setattr(d, "head_dim", 256), 2),
    (lambda d: setattr(d, "ndim", 0), 3),
    (lambda d: setattr(d, "ndim", 4), 3),
    (lambda d: setattr(d, "batch", 0), 3),
    (lambda d: setattr(d, "heads", -2), 3),
    (lambda d: d.block.__setitem__(1, 15), 3),           # 15 does not divide 64
    (lambda d: d.grid.__setitem__(0, 0), 3),
    (lambda d: setattr(d, "readout", T.MHLA_READOUT_MALA), 2),   # MALA needs M == 1
    (lambda d: setattr(d, "mc_per_head", 2), 1),
    (lambda d: setattr(d, "flags", 4), 1),                # unknown flag bit
    (lambda d: setattr(d, "reserved", 1), 1),
])
def test_create_rejections(mutate, want):
    d = _desc()
    mutate(d)
    assert _status(d) == want


def test_earlier_descriptor_layout_is_accepted_without_flags():
    d = _desc()
    d.struct_size = T.MhlaDesc.flags.offset
    d.flags = T.MHLA_FLAG_CLS_TOKEN          # past the earlier layout's end: not read
    assert _status(d) == 0
    d.block[1] = 15                          # and blocks must divide the grid
    assert _status(d) == 3


def _info(**kw):
    p = T.Plan(**dict(dict(batch=1, heads=1, head_dim=64), **kw))
    try:
        return p.info
    finally:
        p.close()


def test_ragged_blocks_and_cls_token_geometry():
    _lib_or_skip()
    # DeiT at 224 px: a 14 x 14 patch grid and a CLS token; 7 x 7 blocks -> 4 + 1 blocks
    i = _info(grid=(14, 14), block=(7, 7), cls_token=True)
    assert (i.n_tokens, i.n_blocks, i.block_tokens) == (197, 5, 49)
    # ragged: 10 x 10 in 4 x 4 blocks -> 3 x 3 blocks of 16, 8, 8, 4 tokens ...
    i = _info(grid=(10, 10), block=(4, 4), ragged=True)
    assert (i.n_tokens, i.n_blocks, i.block_tokens) == (100, 9, 16)
    i = _info(grid=(1000,), block=(300,), ragged=True, cls_token=True)
    assert (i.n_tokens, i.n_blocks, i.block_tokens) == (1001, 5, 300)
    # a block extent beyond the grid's is clipped to it
    i = _info(grid=(5, 40), block=(8, 16), ragged=True)
    assert (i.n_tokens, i.n_blocks, i.block_tokens) == (200, 3, 80)
    # without the flag a non-dividing block is still an error
    assert _status(_desc(grid=(10, 10), block=(4, 4))) == 3
    # MALA with a CLS token has two blocks: not supported
    assert _status(_desc(block=(64, 64), readout="mala", cls_token=True)) == 2


def test_size_limits():
    """One head's bytes (N * d * 4 < 2^31), the (batch, head) pairs and the blocks (<= 65535)."""
    _lib_or_skip()
    n_max = (1 << 31) // (128 * 4) - 1
    assert _status(_desc(grid=(n_max,), block=(n_max,), batch=1, heads=1, head_dim=128)) == 0
    assert _status(_desc(grid=(n_max + 1,), block=(n_max + 1,), batch=1, heads=1, head_dim=128)) == 3
    assert _status(_desc(grid=(8,), block=(4,), batch=65535, heads=1, head_dim=32)) == 0
    assert _status(_desc(grid=(8,), block=(4,), batch=65536, heads=1, head_dim=32)) == 3
    assert _status(_desc(grid=(65535,), block=(1,), batch=1, heads=1, head_dim=32)) == 0
    assert _status(_desc(grid=(65536,), block=(1,), batch=1, heads=1, head_dim=32)) == 3


# Descriptors whose extents are each representable but whose products are not: build_plan must
# bound every factor before it multiplies (an unchecked product once wrapped to N = 0 and the
# plan then divided by it).  Run in a child process so that a crash fails the test instead of
# ending the test session.
OVERFLOW_DESCS = [
    dict(grid=(1 << 31, 1 << 31, 1 << 31), block=(1 << 31, 1 << 31, 1 << 31), ndim3=True),
    dict(grid=((1 << 31) - 1, (1 << 31) - 1, (1 << 31) - 1), block=(1, 1, 1), ndim3=True),
    dict(grid=(1 << 16, 1 << 16), block=(1, 1)),
    dict(grid=(1 << 20, 1 << 20), block=(1 << 20, 1 << 20)),
    dict(grid=(1 << 62,), block=(1 << 62,)),
    dict(grid=(64,), block=(64,), batch=1 << 40, heads=1 << 40),
    dict(grid=(64,), block=(64,), batch=(1 << 31) + 1, heads=2),
]


def test_products_of_large_extents_are_rejected_not_computed():
    _lib_or_skip()
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
import ctypes
import token_blocked_linear_amd as T
cases = {OVERFLOW_DESCS!r}
lib = T.load_library()
for c in cases:
    c = dict(c)
    c.pop("ndim3", None)
    d = T.make_desc(grid=c["grid"], block=c["block"], batch=c.get("batch", 1), heads=c.get("heads", 1),
                    head_dim=64)
    h = ctypes.c_void_p()
    st = lib.mhla_create(ctypes.byref(d), ctypes.byref(h))
    print(st, flush=True)
"""
    r = subprocess.run([__import__("sys").executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    statuses = [int(x) for x in r.stdout.split()]
    assert statuses == [3] * len(OVERFLOW_DESCS), statuses


def test_create_null_arguments():
    lib = _lib_or_skip()
    h = ctypes.c_void_p()
    assert lib.mhla_create(None, ctypes.byref(h)) == T.MHLA_OK + 1
    d = _desc()
    assert lib.mhla_create(ctypes.byref(d), None) == 1
    assert lib.mhla_destroy(None) == 0


def test_feature_maps_accepted():
    for phi in ("elu1", "relu", "exp"):
        assert _status(_desc(phi=phi)) == 0


def test_mala_with_one_block_is_accepted():
    d = _desc(block=(64, 64), readout="mala")
    assert _status(d) == 0


def test_plan_info_and_workspace():
    _lib_or_skip()
    p = T.Plan(grid=(64, 64), block=(16, 16), batch=16, heads=8, head_dim=64)
    info = p.info
    assert (info.n_tokens, info.n_blocks, info.block_tokens) == (4096, 16, 256)
    # 16 blocks: the mixing step runs in the readout's prologue
    assert info.n_kernels == 2 and info.summary_splits >= 1 and info.readout_splits >= 1
    assert p.workspace_bytes == info.workspace_bytes > 0
    assert info.split_operands == 0
    pm = T.Plan(grid=(64, 64), block=(64, 64), batch=16, heads=8, head_dim=64, readout="mala")
    assert pm.info.n_blocks == 1 and pm.info.split_operands == 1 and pm.info.summary_splits > 1
    p32 = T.Plan(grid=(8, 8), block=(4, 4), batch=1, heads=1, head_dim=16, in_dtype="fp32")
    assert p32.info.split_operands == 1
    assert pm.info.n_kernels == 2
    p3 = T.Plan(grid=(128, 128), block=(16, 16), batch=2, heads=4, head_dim=64)
    assert p3.info.n_blocks == 64 and p3.info.n_kernels == 3
    for q in (p, pm, p32, p3):
        q.close()


def test_forward_argument_errors_before_launch():
    """Every case below must be rejected by validation; none reaches a launch (there is no GPU
    here, so a launch would return MHLA_ERR_HIP instead)."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(64, 64), block=(16, 16), batch=16, heads=8, head_dim=64)
    ws = p.workspace_bytes
    A, B, C, O, MC, W = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x100000
    f = lambda *a: lib.mhla_forward(p.handle, *a)  # noqa: E731
    assert f(None, B, C, MC, O, W, ws, None) == 1          # NULL q
    assert f(A, B, C, None, O, W, ws, None) == 1           # NULL M_c with M > 1
    assert f(A, B, C, MC, A, W, ws, None) == 1             # o aliases q
    assert f(A + 2, B, C, MC, O, W, ws, None) == 1         # misaligned q
    assert f(A, B, C, MC, O, None, ws, None) == 4          # no workspace
    assert f(A, B, C, MC, O, W, ws - 1, None) == 4         # workspace too small
    assert f(A, B, C, MC, O, W + 16, ws, None) == 4        # workspace misaligned
    assert lib.mhla_forward(None, A, B, C, MC, O, W, ws, None) == 1
    p.close()


def test_intermediates_argument_errors_before_launch():
    """mhla_forward_intermediates validates before any launch: NULL or unpaired outputs,
    misalignment, a mixed stack that the plan does not keep (its mixing runs in the readout), the
    workspace."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(4096,), block=(64,), batch=1, heads=2, head_dim=64)    # M = 64: a mixing kernel
    pf = T.Plan(grid=(32, 32), block=(8, 8), batch=1, heads=2, head_dim=64)  # M = 16: mixed in the readout
    assert p.info.n_kernels == 3 and pf.info.n_kernels == 2
    K, V, MC, S, Z, ST, ZT, W = (0x10000 * i for i in range(1, 9))
    W = 0x1000000
    f = lambda h, *a: lib.mhla_forward_intermediates(h.handle, *a)  # noqa: E731
    ws = p.workspace_bytes
    assert f(p, None, V, MC, S, Z, ST, ZT, W, ws, None) == 1          # NULL k
    assert f(p, K, V, MC, None, Z, ST, ZT, W, ws, None) == 1          # NULL S
    assert f(p, K, V, MC, S, Z, ST, None, W, ws, None) == 1           # St without zt
    assert f(p, K, V, None, S, Z, ST, ZT, W, ws, None) == 1           # NULL M_c with M > 1
    assert f(p, K + 2, V, MC, S, Z, ST, ZT, W, ws, None) == 1         # misaligned k
    assert f(p, K, V, MC, S + 2, Z, ST, ZT, W, ws, None) == 1         # misaligned S
    assert f(p, K, V, MC, S, Z, ST, ZT, None, ws, None) == 4          # no workspace
    assert f(p, K, V, MC, S, Z, ST, ZT, W, ws - 1, None) == 4         # workspace too small
    assert f(p, K, V, MC, S, Z, ST, ZT, W + 16, ws, None) == 4        # workspace misaligned
    assert f(pf, K, V, MC, S, Z, ST, ZT, W, pf.workspace_bytes, None) == 2   # no mixed stack kept
    assert lib.mhla_forward_intermediates(None, K, V, MC, S, Z, ST, ZT, W, ws, None) == 1
    p.close()
    pf.close()


def test_backward_support_and_workspace():
    _lib_or_skip()
    p = T.Plan(grid=(64, 64), block=(16, 16), batch=16, heads=8, head_dim=64)
    assert T.mhla_backward_workspace_size(p.handle) > 0
    p.close()
    m = T.Plan(grid=(64, 64), block=(64, 64), batch=2, heads=2, head_dim=64, readout="mala")
    assert T.mhla_backward_workspace_size(m.handle) > 0      # MALA: supported
    m.close()
    for kw in (dict(grid=(1000,), block=(100,), readout="causal"), dict(head_dim=16)):
        u = T.Plan(**dict(dict(grid=(64, 64), block=(16, 16), batch=2, heads=2, head_dim=64), **kw))
        with pytest.raises(T.MhlaError) as e:
            T.mhla_backward_workspace_size(u.handle)
        assert e.value.status == 2                           # MHLA_ERR_UNSUPPORTED
        u.close()


def test_mala_backward_rejects_dmc():
    """MALA has no M_c: a dM_c pointer is an argument error, found before any launch."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(64, 64), block=(64, 64), batch=2, heads=2, head_dim=64, readout="mala")
    ws = T.mhla_backward_workspace_size(p.handle)
    Q, K, V, DO, DQ, DK, DV, DMC = (0x10000 * i for i in range(1, 9))
    W = 0x1000000
    assert lib.mhla_backward(p.handle, Q, K, V, None, DO, DQ, DK, DV, DMC, W, ws, None) == 1
    p.close()


def test_backward_argument_errors_before_launch():
    """Rejected by validation, before any launch (a launch here would give MHLA_ERR_HIP)."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(64, 64), block=(16, 16), batch=16, heads=8, head_dim=64)
    ws = T.mhla_backward_workspace_size(p.handle)
    Q, K, V, MC, DO, DQ, DK, DV, DMC, W = (0x10000 * i for i in range(1, 11))
    W = 0x1000000
    f = lambda *a: lib.mhla_backward(p.handle, *a)  # noqa: E731
    assert f(None, K, V, MC, DO, DQ, DK, DV, DMC, W, ws, None) == 1     # NULL q
    assert f(Q, K, V, MC, None, DQ, DK, DV, DMC, W, ws, None) == 1      # NULL dO
    assert f(Q, K, V, MC, DO, DQ, DK, None, DMC, W, ws, None) == 1      # NULL dv
    assert f(Q, K, V, None, DO, DQ, DK, DV, DMC, W, ws, None) == 1      # NULL M_c with M > 1
    assert f(Q, K, V, MC, DO, DO, DK, DV, DMC, W, ws, None) == 1        # dq aliases dO
    assert f(Q, K, V, MC, DO, DQ, DQ, DV, DMC, W, ws, None) == 1        # dk aliases dq
    assert f(Q, K, V, MC, DO, DQ + 8, DK, DV, DMC, W, ws, None) == 1    # misaligned dq
    assert f(Q, K, V, MC, DO, DQ, DK, DV, DMC + 2, W, ws, None) == 1    # misaligned dM_c
    assert f(Q, K, V, MC, DO, DQ, DK, DV, DMC, None, ws, None) == 4     # no workspace
    assert f(Q, K, V, MC, DO, DQ, DK, DV, DMC, W, ws - 1, None) == 4    # workspace too small
    assert f(Q, K, V, MC, DO, DQ, DK, DV, DMC, W + 16, ws, None) == 4   # misaligned workspace
    assert lib.mhla_backward(None, Q, K, V, MC, DO, DQ, DK, DV, DMC, W, ws, None) == 1
    p.close()


def test_decode_support_and_state_size():
    """The decode state: per (batch, head), d^2 + s d floats for each of the M completed blocks,
    the mixed earlier blocks and the running block, where s is the number of channel slices (the
    fewest, of at least max(8, 1024 / d) channels each, that give 512 workgroups); causal plans
    only."""
    _lib_or_skip()
    for (b, h, d, s) in ((2, 3, 64, 4), (1, 16, 128, 16), (64, 8, 64, 1), (16, 8, 32, 1), (32, 8, 128, 2)):
        p = T.Plan(grid=(1000,), block=(128,), batch=b, heads=h, head_dim=d, readout="causal", ragged=True)
        assert p.info.n_blocks == 8
        assert T.mhla_decode_state_size(p.handle) == b * h * (8 + 2) * (d * d + s * d) * 4, (b, h, d)
        p.close()
    # a CLS token is one more block (position 0)
    p = T.Plan(grid=(1000,), block=(125,), batch=1, heads=2, head_dim=64, readout="causal", cls_token=True)
    assert p.info.n_blocks == 9
    assert T.mhla_decode_state_size(p.handle) == 2 * (9 + 2) * (64 * 64 + 4 * 64) * 4
    p.close()
    for kw in (dict(readout="normalized"), dict(readout="unnormalized", cls_token=True)):
        u = T.Plan(**dict(dict(grid=(1000,), block=(125,), batch=1, heads=1, head_dim=64), **kw))
        with pytest.raises(T.MhlaError) as e:
            T.mhla_decode_state_size(u.handle)
        assert e.value.status == 2                           # MHLA_ERR_UNSUPPORTED
        u.close()


def test_decode_argument_errors_before_launch():
    """Rejected by validation, before any launch (a launch here would give MHLA_ERR_HIP)."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(1000,), block=(125,), batch=2, heads=2, head_dim=64, readout="causal")
    n = T.mhla_decode_state_size(p.handle)
    S, Q, K, V, MC, O = 0x1000000, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    f = lambda *a: lib.mhla_decode_step(p.handle, *a)  # noqa: E731
    assert f(S, n, -1, Q, K, V, MC, O, None) == 1          # t before the sequence
    assert f(S, n, 1000, Q, K, V, MC, O, None) == 1        # t past its end
    assert f(S, n, 0, None, K, V, MC, O, None) == 1        # NULL q
    assert f(S, n, 0, Q, K, V, None, O, None) == 1         # NULL M_c with M > 1
    assert f(S, n, 0, Q, K, V, MC, Q, None) == 1           # o aliases q
    assert f(S, n, 0, Q + 1, K, V, MC, O, None) == 1       # misaligned q
    assert f(S, n - 1, 0, Q, K, V, MC, O, None) == 4       # state too small
    assert f(S + 16, n, 0, Q, K, V, MC, O, None) == 4      # state misaligned
    assert lib.mhla_decode_reset(p.handle, S, n - 1, None) == 4
    assert lib.mhla_decode_reset(p.handle, None, n, None) == 1
    assert lib.mhla_decode_step(None, S, n, 0, Q, K, V, MC, O, None) == 1
    p.close()


def test_decode_prefill_sizes_and_argument_errors_before_launch():
    """mhla_decode_prefill: its workspace grows with the prefix; validation rejects bad calls
    before any launch (a launch here would give MHLA_ERR_HIP)."""
    lib = _lib_or_skip()
    p = T.Plan(grid=(1000,), block=(125,), batch=2, heads=2, head_dim=64, readout="causal")
    pc = T.Plan(grid=(999,), block=(125,), batch=1, heads=1, head_dim=64, readout="causal", ragged=True,
                cls_token=True)
    sizes = [T.mhla_decode_prefill_workspace_size(p.handle, n) for n in (1, 125, 126, 1000)]
    assert sizes[0] > 0 and sizes[0] == sizes[1] < sizes[2] < sizes[3]
    assert T.mhla_decode_prefill_workspace_size(pc.handle, 1) == 0     # the CLS token alone: a decode step
    assert T.mhla_decode_prefill_workspace_size(pc.handle, 2) > 0
    for bad in (0, 1001):
        with pytest.raises(T.MhlaError):
            T.mhla_decode_prefill_workspace_size(p.handle, bad)
    fwd = T.Plan(grid=(64, 64), block=(16, 16), batch=1, heads=1, head_dim=64)
    with pytest.raises(T.MhlaError):                                     # not a causal plan
        T.mhla_decode_prefill_workspace_size(fwd.handle, 10)
    n_state = T.mhla_decode_state_size(p.handle)
    S, Q, K, V, MC, O, W = 0x1000000, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x2000000
    ws = sizes[3]
    f = lambda *a: lib.mhla_decode_prefill(p.handle, *a)  # noqa: E731
    assert f(S, n_state, 0, Q, K, V, MC, O, W, ws, None) == 1          # n = 0
    assert f(S, n_state, 1001, Q, K, V, MC, O, W, ws, None) == 1       # n past the capacity
    assert f(S, n_state, 500, None, K, V, MC, O, W, ws, None) == 1     # NULL q
    assert f(S, n_state, 500, Q, K, V, None, O, W, ws, None) == 1      # NULL M_c with M > 1
    assert f(S, n_state, 500, Q, K, V, MC, K, W, ws, None) == 1        # o aliases k
    assert f(S, n_state, 500, Q, K, V, MC, O, S, ws, None) == 1        # workspace is the state
    assert f(S, n_state, 500, Q + 2, K, V, MC, O, W, ws, None) == 1    # misaligned q
    assert f(S, n_state - 1, 500, Q, K, V, MC, O, W, ws, None) == 4    # state too small
    assert f(S, n_state, 1000, Q, K, V, MC, O, W, sizes[2], None) == 4   # workspace too small
    assert f(S, n_state, 500, Q, K, V, MC, O, None, ws, None) == 4     # no workspace
    assert f(S, n_state, 500, Q, K, V, MC, O, W + 16, ws, None) == 4   # workspace misaligned
    assert lib.mhla_decode_prefill(fwd.handle, S, n_state, 10, Q, K, V, MC, O, W, ws, None) == 2
    assert lib.mhla_decode_prefill(None, S, n_state, 10, Q, K, V, MC, O, W, ws, None) == 1
    for x in (p, pc, fwd):
        x.close()


def test_backward_saved_support_sizes_and_argument_errors_before_launch():
    """mhla_backward_saved: supported where the forward keeps split summaries and a mixed stack
    (or reads out MALA); its workspace is smaller than the recomputing backward's; validation
    rejects bad calls before any launch (a launch here would give MHLA_ERR_HIP)."""
    lib = _lib_or_skip()
    split = T.Plan(grid=(4096,), block=(64,), batch=1, heads=2, head_dim=64, accuracy="split")
    mala = T.Plan(grid=(32, 32), block=(32, 32), batch=1, heads=2, head_dim=64, readout="mala")
    bf16 = T.Plan(grid=(4096,), block=(64,), batch=1, heads=2, head_dim=64)            # bf16 stack
    fused = T.Plan(grid=(64, 64), block=(16, 16), batch=1, heads=2, head_dim=64, accuracy="split")  # M = 16
    causal = T.Plan(grid=(4096,), block=(64,), batch=1, heads=2, head_dim=64, readout="causal",
                    accuracy="split")
    train = T.Plan(grid=(4096,), block=(64,), batch=1, heads=2, head_dim=64, accuracy="train")
    assert train.info.split_operands == 1
    assert T.mhla_backward_saved_workspace_size(train.handle) == T.mhla_backward_saved_workspace_size(split.handle)
    train.close()
    for p in (split, mala):
        assert T.mhla_backward_saved_workspace_size(p.handle) < T.mhla_backward_workspace_size(p.handle)
    n = ctypes.c_size_t()
    for p in (bf16, fused, causal):
        assert lib.mhla_backward_saved_workspace_size(p.handle, ctypes.byref(n)) == 2
    Q, K, V, MC, DO, DQ, DK, DV, DMC = (0x10000 * i for i in range(1, 10))
    FW, W = 0x10000000, 0x40000000
    fb = T.mhla_workspace_size(split.handle)
    wb = T.mhla_backward_saved_workspace_size(split.handle)
    f = lambda h, *a: lib.mhla_backward_saved(h, *a)  # noqa: E731
    args = (Q, K, V, MC, DO, DQ, DK, DV, DMC)
    assert f(split.handle, *args, None, fb, W, wb, None) == 1            # no forward workspace
    assert f(split.handle, *args, FW, fb - 1, W, wb, None) == 4          # forward workspace too small
    assert f(split.handle, *args, FW + 16, fb, W, wb, None) == 4         # forward workspace misaligned
    assert f(split.handle, *args, FW, fb, W, wb - 1, None) == 4          # workspace too small
    assert f(split.handle, *args, FW, fb, FW + 256, wb, None) == 1       # workspace inside the forward's
    assert f(split.handle, Q, K, V, MC, DO, FW, DK, DV, DMC, FW, fb, W, wb, None) == 1   # dq in it
    assert f(split.handle, None, K, V, MC, DO, DQ, DK, DV, DMC, FW, fb, W, wb, None) == 1  # NULL q
    assert f(split.handle, Q, K, V, None, DO, DQ, DK, DV, DMC, FW, fb, W, wb, None) == 1  # NULL M_c, M > 1
    for p in (bf16, fused, causal):
        assert f(p.handle, *args, FW, fb, W, wb, None) == 2
    assert f(None, *args, FW, fb, W, wb, None) == 1
    for p in (split, mala, bf16, fused, causal):
        p.close()


def test_decode_binding_rejects_a_host_state():
    """The binding checks the state tensor before handing its pointer to the library."""
    import torch
    _lib_or_skip()
    p = T.Plan(grid=(1000,), block=(125,), batch=1, heads=2, head_dim=64, readout="causal")
    n = T.mhla_decode_state_size(p.handle)
    with pytest.raises(ValueError):
        p.decode_reset(torch.empty(n, dtype=torch.uint8))          # host memory
    p.close()


def test_status_strings():
    _lib_or_skip()
    for s in range(7):
        assert T.mhla_status_string(s)
    assert T.mhla_status_string(0) == "success"
    assert T.mhla_status_string(99) == "unknown status"


def test_timing_api_without_launches():
    _lib_or_skip()
    p = T.Plan(grid=(1024,), block=(16,), batch=1, heads=1, head_dim=32)     # 64 blocks
    T.mhla_timing_enable(p.handle, True)
    name, ms, n = T.mhla_timing_read(p.handle, 0)
    assert (name, ms, n) == ("summary", 0.0, 0)
    assert T.mhla_timing_read(p.handle, 1)[0] == "mix"
    assert T.mhla_timing_read(p.handle, 2)[0] == "readout"
    with pytest.raises(T.MhlaError):
        T.mhla_timing_read(p.handle, 3)
    T.mhla_timing_reset(p.handle)
    names = [T.mhla_backward_timing_read(p.handle, i)[0] for i in range(7)]
    assert names == ["bwd_summary", "bwd_mix", "bwd_dq", "bwd_dsummary", "bwd_dmix", "bwd_keyside", "bwd_dmc"]
    assert T.mhla_backward_timing_read(p.handle, 2)[1:] == (0.0, 0)
    with pytest.raises(T.MhlaError):
        T.mhla_backward_timing_read(p.handle, 7)
    p.close()
    f = T.Plan(grid=(64,), block=(16,), batch=1, heads=1, head_dim=32)       # 4 blocks: fused
    assert [T.mhla_timing_read(f.handle, i)[0] for i in range(2)] == ["summary", "mix+readout"]
    with pytest.raises(T.MhlaError):
        T.mhla_timing_read(f.handle, 2)
    f.close()


def test_fastdiv_exhaustive_on_host(tmp_path):
    """The token -> grid-coordinate division is exact (checked with g++ on the host header)."""
    src = tmp_path / "fd.cpp"
    src.write_text(r'''
#include "fastdiv.hpp"
#include <cstdio>
int main() {
  const unsigned ds[] = {1,2,3,4,5,6,7,8,9,10,12,14,15,16,17,31,32,33,49,63,64,100,255,256,257,
                         1000,1024,4095,4096,65535,65536,1000003,2147483647u};
  for (unsigned d : ds) {
    mhla::FastDiv f = mhla::make_fastdiv(d);
    for (unsigned n = 0; n < 300000; ++n)
      if (mhla::fdiv(n, f) != n / d) { printf("fail %u %u\n", n, d); return 1; }
    for (unsigned n = 2147483647u; n > 2147483647u - 300000u; --n)
      if (mhla::fdiv(n, f) != n / d) { printf("fail %u %u\n", n, d); return 1; }
    for (unsigned n = 1; n < 2147483648u / 7; n = n * 7 + 3)
      if (mhla::fdiv(n, f) != n / d) { printf("fail %u %u\n", n, d); return 1; }
  }
  for (unsigned d = 1; d < 3000; ++d) {
    mhla::FastDiv f = mhla::make_fastdiv(d);
    for (unsigned n = 0; n < 20000; ++n)
      if (mhla::fdiv(n, f) != n / d) { printf("fail %u %u\n", n, d); return 1; }
  }
  printf("ok\n");
  return 0;
}
''')
    exe = tmp_path / "fd"
    csrc = os.path.join(ROOT, "token_blocked_linear_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", csrc, str(src), "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)], capture_output=True, text=True).stdout.strip() == "ok"
