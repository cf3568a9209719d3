"""Seeded synthetic inputs for the token-level multi-head linear attention forward.

This module only *generates inputs*: shapes, seeded Gaussian Q/K/V, bf16
round-to-nearest-even quantisation of those inputs, and the coefficient-matrix
(M_c) generators.  It holds none of the forward computation, and both the
fp64 oracle and the GPU path consume what it produces.

Workloads (shapes stand in for the pages' own settings; no dataset is used):

* ``tiny``      fp32 validation: 1x1 heads, 8x8 grid, d=16, 2x2 blocks of 4x4.
* ``deit_t``    DeiT-T-shaped classification (MHLA notes, Experiments, ImageNet
                table: DeiT-T, 14x14 patches): 64x3 heads, d=64, 2x2 blocks of 7x7.
* ``image``     high-resolution DiT-style grid (MHLA notes, Key design 4 and
                Ablation (b)): 16x8 heads, d=64, 64x64 grid, 4x4 blocks of 16x16.
* ``image_mala`` the same tensors as ``image`` read out with MALA (M=1).
* ``video3d``   3D video latents in the spirit of the Wan2.1 31.5k-token table
                (MHLA notes, Experiments, video): 2x16 heads, d=64, 16x32x32 grid,
                4x4x4 blocks of 4x8x8.
* ``long1d``    long 1D sequence (MHLA notes, Experiments, NLP): 1x16 heads,
                d=128, N=65536, 256 contiguous blocks of 256 tokens.

Recipe: ``numpy.random.default_rng(seed)``; Q, then K, then V drawn with
``standard_normal(shape, float32)`` in C order, then any M_c noise.  bf16
workloads round Q/K/V to bf16 (RNE) and both sides see the same rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "block_grid_shape", "num_blocks",
    "round_to_bf16", "bf16_bits", "bits_to_f32",
    "mc_softmax_l1", "mc_locality_init", "mc_softmax_l1_noisy_clipped", "mc_softmax_gaussian",
    "make_inputs", "make_mc", "make_grad_output", "standard_normal_parallel",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                       # "fp32" or "bf16": element type of Q, K, V and O
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, ...]            # token grid, last axis fastest
    block: Tuple[int, ...]           # block extents, divide the grid exactly
    seed: int
    mc_kind: str                     # "softmax_l1" | "softmax_l1_noise" | "softmax_gauss" | "none"
    readout: str = "normalized"      # "normalized" | "unnormalized" | "mala"
    phi: str = "elu1"                # feature map: "elu1" | "relu" | "exp"
    ragged: bool = False             # blocks need not divide the grid (the last one is cut short)
    cls: bool = False                # one CLS token before the grid, a block of its own

    @property
    def ndim(self) -> int:
        return len(self.grid)

    @property
    def n_tokens(self) -> int:
        return int(self.cls) + int(np.prod(self.grid))

    @property
    def block_tokens(self) -> int:
        return int(np.prod([min(b, g) for g, b in zip(self.grid, self.block)]))

    @property
    def n_blocks(self) -> int:
        return int(self.cls) + num_blocks(self.grid, self.block, self.ragged)

    @property
    def qkv_shape(self) -> Tuple[int, int, int, int]:
        return (self.batch, self.heads, self.n_tokens, self.head_dim)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "fp32", 1, 1, 16, (8, 8), (4, 4), 1, "softmax_l1"),
    "deit_t": Workload("deit_t", "bf16", 64, 3, 64, (14, 14), (7, 7), 2, "softmax_l1"),
    "image": Workload("image", "bf16", 16, 8, 64, (64, 64), (16, 16), 3, "softmax_l1_noise"),
    "image_mala": Workload("image_mala", "bf16", 16, 8, 64, (64, 64), (64, 64), 3, "none", "mala"),
    "video3d": Workload("video3d", "bf16", 2, 16, 64, (16, 32, 32), (4, 8, 8), 4, "softmax_l1"),
    "long1d": Workload("long1d", "bf16", 1, 16, 128, (65536,), (256,), 5, "softmax_gauss"),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def block_grid_shape(grid, block, ragged=False) -> Tuple[int, ...]:
    """Blocks along each axis; with ``ragged`` a block that does not fit is cut short (rounded up)."""
    grid = tuple(int(g) for g in grid)
    block = tuple(int(b) for b in block)
    if len(grid) != len(block):
        raise ValueError("grid and block must have the same rank")
    for g, b in zip(grid, block):
        if b <= 0 or (g % b != 0 and not ragged):
            raise ValueError(f"block extent {b} does not divide grid extent {g}")
    return tuple(-(-g // b) for g, b in zip(grid, block))


def num_blocks(grid, block, ragged=False) -> int:
    return int(np.prod(block_grid_shape(grid, block, ragged)))


# --------------------------------------------------------------------------------------
# bf16 quantisation of generated inputs (round to nearest, ties to even)
# --------------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 ``x`` rounded to bf16, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of ``x``."""
    return bits_to_f32(bf16_bits(x))


def standard_normal_parallel(shape, seed: int, bf16: bool, threads: int = 16) -> np.ndarray:
    """Large inputs: float32 N(0, 1) of ``shape`` drawn in chunks of 2^24 values, chunk c from
    ``default_rng(SeedSequence(seed).spawn(n_chunks)[c])``, filled by ``threads`` threads (the
    generators release the GIL); rounded to bf16 (RNE) chunk by chunk when ``bf16``."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    chunk = 1 << 24
    seqs = np.random.SeedSequence(seed).spawn((n + chunk - 1) // chunk)
    out = np.empty(n, np.float32)

    def fill(c):
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        x = np.random.default_rng(seqs[c]).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = round_to_bf16(x) if bf16 else x

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(len(seqs))))
    return out.reshape(shape)


# --------------------------------------------------------------------------------------
# Coefficient-matrix generators (inputs of the forward; M_c is a learned parameter)
# --------------------------------------------------------------------------------------

def _block_coords(block_grid) -> np.ndarray:
    """[M, ndim] integer coordinates of every block, raster order, last axis fastest."""
    idx = np.indices(block_grid).reshape(len(block_grid), -1).T
    return idx.astype(np.float64)


def mc_softmax_l1(block_grid) -> np.ndarray:
    """Rows = softmax(-L1 distance between block centres), distances in block-grid units."""
    c = _block_coords(block_grid)
    dist = np.abs(c[:, None, :] - c[None, :, :]).sum(-1)
    logits = -dist
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


def mc_locality_init(block_grid) -> np.ndarray:
    """Locality-biased initialisation (MHLA notes, Key design 3): row i is proportional to
    1 - dist(i,j)/max_k dist(i,k) with Euclidean block-centre distance, rows sum to one.
    A single block has no distance scale; its row is [1]."""
    c = _block_coords(block_grid)
    m = c.shape[0]
    if m == 1:
        return np.ones((1, 1))
    dist = np.sqrt(((c[:, None, :] - c[None, :, :]) ** 2).sum(-1))
    w = 1.0 - dist / dist.max(axis=1, keepdims=True)
    return w / w.sum(axis=1, keepdims=True)


def mc_softmax_l1_noisy_clipped(block_grid, rng: np.random.Generator, scale: float = 0.1) -> np.ndarray:
    """softmax(-L1) plus ``scale``*N(0,1) noise, clipped to [0, 1] without renormalising
    (a trained M_c is clipped into (0,1) at every update, MHLA notes, Key design 3)."""
    base = mc_softmax_l1(block_grid)
    noise = rng.standard_normal(base.shape, dtype=np.float32).astype(np.float64)
    m = np.clip(base + scale * noise, 0.0, 1.0)
    if not np.all(m.max(axis=1) > 0):
        raise RuntimeError("a clipped M_c row lost every positive entry")
    return m


def mc_softmax_gaussian(n_blocks: int, rng: np.random.Generator) -> np.ndarray:
    """Dense M_c: logits ~ N(0, 1/M) (standard deviation 1/sqrt(M)), row softmax."""
    logits = rng.standard_normal((n_blocks, n_blocks), dtype=np.float32).astype(np.float64)
    logits /= math.sqrt(n_blocks)
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------------------
# Full input sets
# --------------------------------------------------------------------------------------

def make_inputs(w: Workload, rng: Optional[np.random.Generator] = None):
    """Return (q, k, v, mc, rng) for workload ``w``.

    q, k, v: float32 arrays of shape [B, H, N, d] holding exactly the values the GPU sees
    (bf16-rounded for bf16 workloads).  mc: float64 [M, M] (or None for MALA), already
    representable in float32 (it is rounded through float32).  ``rng`` is returned so a
    caller can keep drawing from the same stream.
    """
    if rng is None:
        rng = np.random.default_rng(w.seed)
    shape = w.qkv_shape
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype != "fp32":
        raise ValueError(w.dtype)
    mc = make_mc(w, rng)
    return q, k, v, mc, rng


def make_grad_output(w: Workload, rng: np.random.Generator, dtype: str = "fp32") -> np.ndarray:
    """Upstream gradient dL/dO for the backward: [B, H, N, d] standard normal float32, rounded
    to bf16 when ``dtype`` is "bf16" (the element type it crosses the boundary in)."""
    do = rng.standard_normal(w.qkv_shape, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(do)
    if dtype != "fp32":
        raise ValueError(dtype)
    return do


def make_mc(w: Workload, rng: np.random.Generator):
    """M_c for ``w`` ([M, M], M counting a CLS block).  With a CLS token only the kinds that
    need no block-grid geometry apply."""
    bg = block_grid_shape(w.grid, w.block, w.ragged)
    m = w.n_blocks
    if w.mc_kind == "none":
        return None
    if w.cls and w.mc_kind in ("softmax_l1", "softmax_l1_noise", "locality"):
        raise ValueError(f"M_c kind {w.mc_kind} is laid out on the block grid; a CLS block has no place there")
    if w.mc_kind == "softmax_l1":
        mc = mc_softmax_l1(bg)
    elif w.mc_kind == "softmax_l1_noise":
        mc = mc_softmax_l1_noisy_clipped(bg, rng)
    elif w.mc_kind == "softmax_gauss":
        mc = mc_softmax_gaussian(m, rng)
    elif w.mc_kind == "locality":
        mc = mc_locality_init(bg)
    elif w.mc_kind == "identity":
        mc = np.eye(m)
    elif w.mc_kind == "ones":
        mc = np.ones((m, m))
    else:
        raise ValueError(w.mc_kind)
    # M_c crosses the boundary as fp32; both sides use the fp32-representable values.
    return mc.astype(np.float32).astype(np.float64)
