"""Python binding of the gfx950 MHLA forward library (``libmhla.so``, C ABI in include/mhla.h).

The functions carry the C names and only marshal arguments: every step of the forward runs
in the library's HIP kernels.  torch is used for device memory and streams only.  If the
library has not been built the import of this module still succeeds, but every call raises
``MhlaLibraryMissing`` -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "MHLA_OK", "MHLA_DTYPE_BF16", "MHLA_DTYPE_FP32", "MHLA_PHI_ELU1", "MHLA_PHI_RELU", "MHLA_PHI_EXP",
    "MHLA_READOUT_NORMALIZED", "MHLA_READOUT_UNNORMALIZED", "MHLA_READOUT_MALA",
    "MHLA_READOUT_CAUSAL_NORMALIZED", "MHLA_READOUT_CAUSAL_UNNORMALIZED",
    "MHLA_FLAG_RAGGED_BLOCKS", "MHLA_FLAG_CLS_TOKEN",
    "MHLA_ACCURACY_AUTO", "MHLA_ACCURACY_BF16", "MHLA_ACCURACY_SPLIT", "MHLA_ACCURACY_TRAIN",
    "MhlaDesc", "MhlaPlanInfo", "MhlaError", "MhlaLibraryMissing", "library_path", "load_library",
    "mhla_create", "mhla_workspace_size", "mhla_forward", "mhla_destroy", "mhla_status_string",
    "mhla_plan_get_info", "mhla_timing_enable", "mhla_timing_read", "mhla_timing_reset",
    "mhla_backward_workspace_size", "mhla_backward", "mhla_backward_timing_read",
    "mhla_backward_saved_workspace_size", "mhla_backward_saved",
    "mhla_decode_state_size", "mhla_decode_reset", "mhla_decode_step", "mhla_forward_noalloc",
    "mhla_forward_intermediates", "mhla_decode_prefill_workspace_size", "mhla_decode_prefill",
    "MHLA_NOALLOC_SCRATCH_BYTES", "MHLA_ERR_SCRATCH_LIMIT", "make_desc", "Plan", "EXPORTED_SYMBOLS",
]

MHLA_OK = 0
MHLA_DTYPE_BF16, MHLA_DTYPE_FP32 = 0, 1
MHLA_PHI_ELU1, MHLA_PHI_RELU, MHLA_PHI_EXP = 0, 1, 2
MHLA_READOUT_NORMALIZED, MHLA_READOUT_UNNORMALIZED, MHLA_READOUT_MALA = 0, 1, 2
MHLA_READOUT_CAUSAL_NORMALIZED, MHLA_READOUT_CAUSAL_UNNORMALIZED = 3, 4
MHLA_FLAG_RAGGED_BLOCKS, MHLA_FLAG_CLS_TOKEN = 1, 2
MHLA_ACCURACY_AUTO, MHLA_ACCURACY_BF16, MHLA_ACCURACY_SPLIT, MHLA_ACCURACY_TRAIN = 0, 1, 2, 3
MHLA_ERR_SCRATCH_LIMIT = 7
MHLA_NOALLOC_SCRATCH_BYTES = 160 << 20     # the no-alloc forward's scratch array (include/mhla.h)

_READOUTS = {"normalized": MHLA_READOUT_NORMALIZED, "unnormalized": MHLA_READOUT_UNNORMALIZED,
             "mala": MHLA_READOUT_MALA, "causal": MHLA_READOUT_CAUSAL_NORMALIZED,
             "causal_unnormalized": MHLA_READOUT_CAUSAL_UNNORMALIZED}
_DTYPES = {"bf16": MHLA_DTYPE_BF16, "fp32": MHLA_DTYPE_FP32}
_PHIS = {"elu1": MHLA_PHI_ELU1, "relu": MHLA_PHI_RELU, "exp": MHLA_PHI_EXP}
_ACCURACY = {"auto": MHLA_ACCURACY_AUTO, "bf16": MHLA_ACCURACY_BF16, "split": MHLA_ACCURACY_SPLIT,
             "train": MHLA_ACCURACY_TRAIN}

EXPORTED_SYMBOLS = (
    "mhla_create", "mhla_workspace_size", "mhla_forward", "mhla_destroy", "mhla_status_string",
    "mhla_plan_get_info", "mhla_timing_enable", "mhla_timing_read", "mhla_timing_reset",
    "mhla_backward_workspace_size", "mhla_backward", "mhla_backward_timing_read",
    "mhla_decode_state_size", "mhla_decode_reset", "mhla_decode_step", "mhla_forward_noalloc",
    "mhla_forward_intermediates", "mhla_decode_prefill_workspace_size", "mhla_decode_prefill",
    "mhla_backward_saved_workspace_size", "mhla_backward_saved",
)


class MhlaDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("phi", ctypes.c_int32),
        ("readout", ctypes.c_int32),
        ("accuracy", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("mc_per_head", ctypes.c_int32),
        ("grid", ctypes.c_int64 * 3),
        ("block", ctypes.c_int64 * 3),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MhlaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("n_tokens", ctypes.c_int64),
        ("n_blocks", ctypes.c_int64),
        ("block_tokens", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("summary_splits", ctypes.c_int32),
        ("readout_splits", ctypes.c_int32),
        ("n_kernels", ctypes.c_int32),
        ("split_operands", ctypes.c_int32),
    ]


class MhlaLibraryMissing(RuntimeError):
    pass


class MhlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {mhla_status_string(status)} (status {status})")


_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    """The in-tree build; MHLA_LIBRARY may name another build of the same library."""
    override = os.environ.get("MHLA_LIBRARY")
    if override:
        return override
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmhla.so")


def load_library() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MhlaLibraryMissing(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(there is no CPU fallback for the MHLA forward)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.mhla_create.argtypes = [ctypes.POINTER(MhlaDesc), ctypes.POINTER(P)]
    lib.mhla_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.mhla_forward.argtypes = [P, P, P, P, P, P, P, SZ, P]
    lib.mhla_forward_noalloc.argtypes = [P, P, P, P, P, P, P]
    lib.mhla_forward_intermediates.argtypes = [P, P, P, P, P, P, P, P, P, SZ, P]
    lib.mhla_backward_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.mhla_backward.argtypes = [P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.mhla_backward_saved_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.mhla_backward_saved.argtypes = [P, P, P, P, P, P, P, P, P, P, P, SZ, P, SZ, P]
    lib.mhla_destroy.argtypes = [P]
    lib.mhla_status_string.argtypes = [I32]
    lib.mhla_status_string.restype = ctypes.c_char_p
    lib.mhla_plan_get_info.argtypes = [P, ctypes.POINTER(MhlaPlanInfo)]
    lib.mhla_timing_enable.argtypes = [P, I32]
    lib.mhla_timing_read.argtypes = [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64),
                                     ctypes.POINTER(ctypes.c_char_p)]
    lib.mhla_timing_reset.argtypes = [P]
    lib.mhla_backward_timing_read.argtypes = lib.mhla_timing_read.argtypes
    lib.mhla_decode_state_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.mhla_decode_reset.argtypes = [P, P, SZ, P]
    lib.mhla_decode_step.argtypes = [P, P, SZ, I64, P, P, P, P, P, P]
    lib.mhla_decode_prefill_workspace_size.argtypes = [P, I64, ctypes.POINTER(SZ)]
    lib.mhla_decode_prefill.argtypes = [P, P, SZ, I64, P, P, P, P, P, P, SZ, P]
    for name in EXPORTED_SYMBOLS:
        if name != "mhla_status_string":
            getattr(lib, name).restype = I32
    _LIB = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != MHLA_OK:
        raise MhlaError(status, what)


# ------------------------------------------------------------------------------------------
# C-named wrappers
# ------------------------------------------------------------------------------------------

def mhla_status_string(status: int) -> str:
    return load_library().mhla_status_string(int(status)).decode()


def mhla_create(desc: MhlaDesc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().mhla_create(ctypes.byref(desc), ctypes.byref(h)), "mhla_create")
    return h


def mhla_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mhla_workspace_size(h, ctypes.byref(n)), "mhla_workspace_size")
    return n.value


def mhla_forward(h, q: int, k: int, v: int, mc: int, o: int, workspace: int, workspace_bytes: int,
                 stream: int) -> None:
    """Pointers are integer device addresses (0 for NULL); ``stream`` a raw hipStream_t."""
    _check(load_library().mhla_forward(h, q, k, v, mc or None, o, workspace or None,
                                       workspace_bytes, stream or None), "mhla_forward")


def mhla_forward_noalloc(h, q: int, k: int, v: int, mc: int, o: int, stream: int) -> None:
    """mhla_forward with the library's own scratch array as workspace (no allocation); pointers are
    integer device addresses (0 for NULL), ``stream`` a raw hipStream_t."""
    _check(load_library().mhla_forward_noalloc(h, q, k, v, mc or None, o, stream or None), "mhla_forward_noalloc")


def mhla_forward_intermediates(h, k: int, v: int, mc: int, S: int, z: int, St: int, zt: int, workspace: int,
                               workspace_bytes: int, stream: int) -> None:
    """The summaries and mixed summaries in fp32 (St = zt = 0 to stop after the summaries);
    pointers are integer device addresses (0 for NULL), ``stream`` a raw hipStream_t."""
    _check(load_library().mhla_forward_intermediates(h, k, v, mc or None, S, z, St or None, zt or None,
                                                     workspace or None, workspace_bytes, stream or None),
           "mhla_forward_intermediates")


def mhla_backward_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mhla_backward_workspace_size(h, ctypes.byref(n)), "mhla_backward_workspace_size")
    return n.value


def mhla_backward(h, q: int, k: int, v: int, mc: int, dout: int, dq: int, dk: int, dv: int, dmc: int,
                  workspace: int, workspace_bytes: int, stream: int) -> None:
    """Pointers are integer device addresses (0 for NULL); ``stream`` a raw hipStream_t."""
    _check(load_library().mhla_backward(h, q, k, v, mc or None, dout, dq, dk, dv, dmc or None,
                                        workspace or None, workspace_bytes, stream or None), "mhla_backward")


def mhla_backward_saved_workspace_size(h) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mhla_backward_saved_workspace_size(h, ctypes.byref(n)),
           "mhla_backward_saved_workspace_size")
    return n.value


def mhla_backward_saved(h, q: int, k: int, v: int, mc: int, dout: int, dq: int, dk: int, dv: int, dmc: int,
                        fwd_workspace: int, fwd_workspace_bytes: int, workspace: int, workspace_bytes: int,
                        stream: int) -> None:
    """As mhla_backward, reading the forward's summaries from ``fwd_workspace`` (integer device
    addresses, 0 for NULL; ``stream`` a raw hipStream_t)."""
    _check(load_library().mhla_backward_saved(h, q, k, v, mc or None, dout, dq, dk, dv, dmc or None,
                                              fwd_workspace or None, fwd_workspace_bytes, workspace or None,
                                              workspace_bytes, stream or None), "mhla_backward_saved")


def mhla_decode_state_size(h) -> int:
    n = ctypes.c_size_t()
    _check(load_library().mhla_decode_state_size(h, ctypes.byref(n)), "mhla_decode_state_size")
    return n.value


def mhla_decode_reset(h, state: int, state_bytes: int, stream: int) -> None:
    _check(load_library().mhla_decode_reset(h, state, state_bytes, stream or None), "mhla_decode_reset")


def mhla_decode_step(h, state: int, state_bytes: int, t: int, q: int, k: int, v: int, mc: int, o: int,
                     stream: int) -> None:
    """One token per (batch, head) at position ``t``; pointers are integer device addresses."""
    _check(load_library().mhla_decode_step(h, state, state_bytes, t, q, k, v, mc or None, o, stream or None),
           "mhla_decode_step")


def mhla_decode_prefill_workspace_size(h, n: int) -> int:
    b = ctypes.c_size_t()
    _check(load_library().mhla_decode_prefill_workspace_size(h, int(n), ctypes.byref(b)),
           "mhla_decode_prefill_workspace_size")
    return b.value


def mhla_decode_prefill(h, state: int, state_bytes: int, n: int, q: int, k: int, v: int, mc: int, o: int,
                        workspace: int, workspace_bytes: int, stream: int) -> None:
    """Positions 0 .. n-1 of every (batch, head) into the decode state; pointers are integer device
    addresses (0 for NULL), ``stream`` a raw hipStream_t."""
    _check(load_library().mhla_decode_prefill(h, state, state_bytes, int(n), q, k, v, mc or None, o,
                                              workspace or None, workspace_bytes, stream or None),
           "mhla_decode_prefill")


def mhla_destroy(h) -> None:
    _check(load_library().mhla_destroy(h), "mhla_destroy")


def mhla_plan_get_info(h) -> MhlaPlanInfo:
    info = MhlaPlanInfo()
    info.struct_size = ctypes.sizeof(MhlaPlanInfo)
    _check(load_library().mhla_plan_get_info(h, ctypes.byref(info)), "mhla_plan_get_info")
    return info


def mhla_timing_enable(h, enable: bool) -> None:
    _check(load_library().mhla_timing_enable(h, 1 if enable else 0), "mhla_timing_enable")


def mhla_timing_read(h, index: int):
    ms, n, name = ctypes.c_double(), ctypes.c_int64(), ctypes.c_char_p()
    _check(load_library().mhla_timing_read(h, index, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(name)),
           "mhla_timing_read")
    return name.value.decode(), ms.value, n.value


def mhla_backward_timing_read(h, index: int):
    ms, n, name = ctypes.c_double(), ctypes.c_int64(), ctypes.c_char_p()
    _check(load_library().mhla_backward_timing_read(h, index, ctypes.byref(ms), ctypes.byref(n),
                                                    ctypes.byref(name)), "mhla_backward_timing_read")
    return name.value.decode(), ms.value, n.value


def mhla_timing_reset(h) -> None:
    _check(load_library().mhla_timing_reset(h), "mhla_timing_reset")


# ------------------------------------------------------------------------------------------
# Convenience over torch tensors (marshalling only)
# ------------------------------------------------------------------------------------------

def make_desc(*, grid: Sequence[int], block: Sequence[int], batch: int, heads: int, head_dim: int,
              in_dtype: str = "bf16", out_dtype: str = "fp32", readout: str = "normalized",
              accuracy: str = "auto", mc_per_head: bool = False, phi: str = "elu1",
              ragged: bool = False, cls_token: bool = False) -> MhlaDesc:
    """The plan descriptor of include/mhla.h.  accuracy: "auto", "bf16", "split", or "train" (the
    summaries and mixing split, as mhla_backward_saved needs them; the readout as "auto")."""
    if len(grid) != len(block) or not 1 <= len(grid) <= 3:
        raise ValueError("grid and block must have the same rank, 1 to 3")
    d = MhlaDesc()
    d.struct_size = ctypes.sizeof(MhlaDesc)
    d.in_dtype = _DTYPES[in_dtype]
    d.out_dtype = _DTYPES[out_dtype]
    d.phi = _PHIS[phi]
    d.readout = _READOUTS[readout]
    d.accuracy = _ACCURACY[accuracy]
    d.ndim = len(grid)
    d.mc_per_head = 1 if mc_per_head else 0
    for i, (g, b) in enumerate(zip(grid, block)):
        d.grid[i] = int(g)
        d.block[i] = int(b)
    d.batch, d.heads, d.head_dim = int(batch), int(heads), int(head_dim)
    d.flags = (MHLA_FLAG_RAGGED_BLOCKS if ragged else 0) | (MHLA_FLAG_CLS_TOKEN if cls_token else 0)
    return d


class Plan:
    """Owns one plan handle.  ``forward`` takes torch tensors already on the GPU."""

    def __init__(self, **desc_kwargs):
        self.desc_kwargs = dict(desc_kwargs)
        self.desc = make_desc(**desc_kwargs)
        self.handle = mhla_create(self.desc)
        self.workspace_bytes = mhla_workspace_size(self.handle)
        self.info = mhla_plan_get_info(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            mhla_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_workspace(self, device="cuda"):
        import torch
        return torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=device)

    def expected_shapes(self):
        kw = self.desc_kwargs
        n = 1
        for g in kw["grid"]:
            n *= int(g)
        n += 1 if kw.get("cls_token") else 0
        qkv = (int(kw["batch"]), int(kw["heads"]), n, int(kw["head_dim"]))
        m = int(self.info.n_blocks)
        mc = (int(kw["heads"]), m, m) if kw.get("mc_per_head") else (m, m)
        return qkv, mc

    def check_args(self, q, k, v, mc, o, workspace, ws_bytes=None, check_o=True):
        """Host-side checks that every buffer has the shape, dtype and layout the kernels
        index; the C ABI receives bare pointers and cannot see them."""
        import torch
        ws_bytes = self.workspace_bytes if ws_bytes is None else ws_bytes
        qkv, mc_shape = self.expected_shapes()
        tin = torch.bfloat16 if self.desc_kwargs.get("in_dtype", "bf16") == "bf16" else torch.float32
        tout = torch.bfloat16 if self.desc_kwargs.get("out_dtype", "fp32") == "bf16" else torch.float32
        checks = (("q", q, tin), ("k", k, tin), ("v", v, tin)) + ((("o", o, tout),) if check_o else ())
        for name, t, dt in checks:
            if tuple(t.shape) != qkv or t.dtype != dt or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name}: expected contiguous {dt} cuda tensor of shape {qkv}, "
                                 f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
        if mc is None:
            if self.info.n_blocks != 1:
                raise ValueError("mc is required when there is more than one block")
        elif (tuple(mc.shape) != mc_shape or mc.dtype != torch.float32 or not mc.is_contiguous()
              or not mc.is_cuda):
            raise ValueError(f"mc: expected contiguous float32 cuda tensor {mc_shape}")
        if workspace.dtype != torch.uint8 or workspace.numel() < ws_bytes or not workspace.is_cuda:
            raise ValueError(f"workspace: expected >= {ws_bytes} bytes of uint8 on the GPU")

    def alloc_backward_workspace(self, device="cuda"):
        import torch
        n = mhla_backward_workspace_size(self.handle)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def alloc_backward_saved_workspace(self, device="cuda"):
        import torch
        n = mhla_backward_saved_workspace_size(self.handle)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def backward(self, q, k, v, mc, dout, dq, dk, dv, dmc, workspace, stream=None, fwd_workspace=None):
        """Gradients into dq, dk, dv (the plan's out_dtype, like dout) and dmc (fp32, M_c's shape,
        or None to skip).  With ``fwd_workspace`` (the workspace of this plan's last forward on the
        same q, k, v, mc, unchanged since) the forward's summaries are read from it
        (mhla_backward_saved) and ``workspace`` is the smaller one of
        alloc_backward_saved_workspace."""
        import torch
        ws_need = (mhla_backward_saved_workspace_size(self.handle) if fwd_workspace is not None
                   else mhla_backward_workspace_size(self.handle))
        self.check_args(q, k, v, mc, dout, workspace, ws_need)
        if fwd_workspace is not None:
            fb = mhla_workspace_size(self.handle)
            if fwd_workspace.dtype != torch.uint8 or fwd_workspace.numel() < fb or not fwd_workspace.is_cuda:
                raise ValueError(f"fwd_workspace: expected the forward's workspace (>= {fb} bytes of uint8)")
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            if t.shape != dout.shape or t.dtype != dout.dtype or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name}: expected a contiguous cuda tensor like dout")
        if dmc is not None:
            _, mc_shape = self.expected_shapes()
            if (tuple(dmc.shape) != mc_shape or dmc.dtype != torch.float32 or not dmc.is_contiguous()
                    or not dmc.is_cuda):
                raise ValueError(f"dmc: expected contiguous float32 cuda tensor of shape {mc_shape}")
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), mc.data_ptr() if mc is not None else 0,
                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                dmc.data_ptr() if dmc is not None else 0)
        if fwd_workspace is not None:
            mhla_backward_saved(self.handle, *ptrs, fwd_workspace.data_ptr(), fwd_workspace.numel(),
                                workspace.data_ptr(), workspace.numel(), stream.cuda_stream)
        else:
            mhla_backward(self.handle, *ptrs, workspace.data_ptr(), workspace.numel(), stream.cuda_stream)
        return dq, dk, dv, dmc

    def alloc_decode_state(self, device="cuda"):
        """A decode state for this (causal) plan, cleared on the current stream."""
        import torch
        n = mhla_decode_state_size(self.handle)
        state = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
        self.decode_reset(state)
        return state

    def _check_decode_state(self, state):
        import torch
        need = mhla_decode_state_size(self.handle)
        if (not isinstance(state, torch.Tensor) or not state.is_cuda or not state.is_contiguous()
                or state.numel() * state.element_size() < need):
            raise ValueError(f"state: expected a contiguous cuda tensor of at least {need} bytes")

    def decode_reset(self, state, stream=None):
        import torch
        self._check_decode_state(state)
        if stream is None:
            stream = torch.cuda.current_stream(state.device)
        mhla_decode_reset(self.handle, state.data_ptr(), state.numel() * state.element_size(), stream.cuda_stream)

    def decode_step(self, state, t, q, k, v, mc, o, stream=None):
        """Token ``t`` of every (batch, head): q, k, v [B, H, 1, d] of the plan's in_dtype, o the
        same shape in its out_dtype (written)."""
        import torch
        kw = self.desc_kwargs
        shape = (int(kw["batch"]), int(kw["heads"]), 1, int(kw["head_dim"]))
        tin = torch.bfloat16 if kw.get("in_dtype", "bf16") == "bf16" else torch.float32
        tout = torch.bfloat16 if kw.get("out_dtype", "fp32") == "bf16" else torch.float32
        for name, x, dt in (("q", q, tin), ("k", k, tin), ("v", v, tin), ("o", o, tout)):
            if tuple(x.shape) != shape or x.dtype != dt or not x.is_contiguous() or not x.is_cuda:
                raise ValueError(f"{name}: expected a contiguous {dt} cuda tensor of shape {shape}")
        _, mc_shape = self.expected_shapes()
        if mc is not None and (tuple(mc.shape) != mc_shape or mc.dtype != torch.float32
                               or not mc.is_contiguous() or not mc.is_cuda):
            raise ValueError(f"mc: expected contiguous float32 cuda tensor {mc_shape}")
        self._check_decode_state(state)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        mhla_decode_step(self.handle, state.data_ptr(), state.numel() * state.element_size(), int(t), q.data_ptr(), k.data_ptr(),
                         v.data_ptr(), mc.data_ptr() if mc is not None else 0, o.data_ptr(), stream.cuda_stream)
        return o

    def alloc_prefill_workspace(self, n, device="cuda"):
        import torch
        return torch.empty(max(mhla_decode_prefill_workspace_size(self.handle, int(n)), 256), dtype=torch.uint8,
                           device=device)

    def decode_prefill(self, state, q, k, v, mc, o, workspace, stream=None):
        """Positions 0 .. n-1 of every (batch, head) in one call: q, k, v [B, H, n, d] of the plan's
        in_dtype, o the same shape in its out_dtype (written); the state continues at t = n."""
        import torch
        kw = self.desc_kwargs
        n = int(q.shape[2]) if q.dim() == 4 else -1
        shape = (int(kw["batch"]), int(kw["heads"]), n, int(kw["head_dim"]))
        tin = torch.bfloat16 if kw.get("in_dtype", "bf16") == "bf16" else torch.float32
        tout = torch.bfloat16 if kw.get("out_dtype", "fp32") == "bf16" else torch.float32
        for name, x, dt in (("q", q, tin), ("k", k, tin), ("v", v, tin), ("o", o, tout)):
            if tuple(x.shape) != shape or x.dtype != dt or not x.is_contiguous() or not x.is_cuda:
                raise ValueError(f"{name}: expected a contiguous {dt} cuda tensor of shape {shape}")
        _, mc_shape = self.expected_shapes()
        if mc is not None and (tuple(mc.shape) != mc_shape or mc.dtype != torch.float32
                               or not mc.is_contiguous() or not mc.is_cuda):
            raise ValueError(f"mc: expected contiguous float32 cuda tensor {mc_shape}")
        self._check_decode_state(state)
        need = mhla_decode_prefill_workspace_size(self.handle, n)
        if need and (workspace is None or workspace.dtype != torch.uint8 or workspace.numel() < need
                     or not workspace.is_cuda):
            raise ValueError(f"workspace: expected >= {need} bytes of uint8 on the GPU")
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        mhla_decode_prefill(self.handle, state.data_ptr(), state.numel() * state.element_size(), n, q.data_ptr(),
                            k.data_ptr(), v.data_ptr(), mc.data_ptr() if mc is not None else 0, o.data_ptr(),
                            workspace.data_ptr() if workspace is not None else 0,
                            workspace.numel() if workspace is not None else 0, stream.cuda_stream)
        return o

    def intermediates(self, k, v, mc, workspace, mixed=True, stream=None):
        """The forward's summaries (S [B*H, M, d, d], z [B*H, M, d]) and, with ``mixed``, its mixed
        summaries (St, zt), as fp32 tensors; ``mixed`` needs a plan with a mixing kernel."""
        import torch
        self.check_args(k, k, v, mc, torch.empty(0), workspace, check_o=False)
        if stream is None:
            stream = torch.cuda.current_stream(k.device)
        kw = self.desc_kwargs
        rows, m, d = int(kw["batch"]) * int(kw["heads"]), int(self.info.n_blocks), int(kw["head_dim"])
        S = torch.empty((rows, m, d, d), dtype=torch.float32, device=k.device)
        z = torch.empty((rows, m, d), dtype=torch.float32, device=k.device)
        St = torch.empty_like(S) if mixed else None
        zt = torch.empty_like(z) if mixed else None
        mhla_forward_intermediates(self.handle, k.data_ptr(), v.data_ptr(), mc.data_ptr() if mc is not None else 0,
                                   S.data_ptr(), z.data_ptr(), St.data_ptr() if mixed else 0,
                                   zt.data_ptr() if mixed else 0, workspace.data_ptr(), workspace.numel(),
                                   stream.cuda_stream)
        return (S, z, St, zt) if mixed else (S, z)

    def forward(self, q, k, v, mc, o, workspace, stream=None):
        import torch
        self.check_args(q, k, v, mc, o, workspace)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        mhla_forward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     mc.data_ptr() if mc is not None else 0, o.data_ptr(), workspace.data_ptr(),
                     workspace.numel(), stream.cuda_stream)
        return o
