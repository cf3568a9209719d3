"""fp64 CPU oracle for chunkwise-causal MHLA over a 1D token sequence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.  The GPU
library never calls it and shares no code with it; this file imports NumPy and the forward
oracle only.

Sources (page titles and sections):
  [MHLA]  "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
          Method -> Key design 2 (the token-expanded identity q~^T S~_i =
          sum_t m_{i,b(t)} (q~^T K~_t) V_t^T; the normaliser may be dropped for language
          modelling), Key design 4 (MHLA is compatible with chunkwise-parallel training and
          streaming / stateful inference, one head per chunk), Experiments (a 0.3B language
          model, i.e. autoregressive use).

The pages do not define the causal form.  Reading (stated once, used everywhere):
  * Causality masks the token-expanded sum at the token level: query t sees the keys t' <= t,
    each with weight m_{b(t), b(t')} (q~_t . k~_t').  Blocks are contiguous spans of the 1D
    sequence, numbered in order.
  * Hence a query of block i reads every earlier block b < i through its whole summary S_b
    (weight m_ib), its own block through the running prefix of that block up to itself
    (weight m_ii), and nothing of later blocks: entries of M_c above the diagonal are never
    used.
  * Normalised: o_t = num_t / den_t with den_t the same masked sum without V; unnormalised:
    o_t = num_t.
Functions:
  causal_blockwise  the chunkwise steps: S_b, z_b; mixing with the strictly lower part of
                    M_c; a running in-block state updated token by token (the streaming form)
  causal_plain      the masked N x N sum, built explicitly (tiny inputs)
  causal_sampled    the masked sum for a few query tokens (any size)
"""
from __future__ import annotations

import numpy as np

from . import mhla_oracle as F

__all__ = ["causal_blockwise", "causal_plain", "causal_sampled", "forward_causal", "forward_causal_sampled"]


def _blocks_1d(grid, block):
    """Blocks of a 1D sequence (plain, or a RaggedGrid: a shorter last span, a CLS token first)."""
    dims = grid.grid if isinstance(grid, F.RaggedGrid) else tuple(grid)
    if len(dims) != 1:
        raise ValueError("the causal form is defined for a 1D token sequence")
    return F.block_index(grid, block)


def causal_blockwise(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    """One (batch, head): q, k, v [N, d] -> o [N, d]."""
    bidx = _blocks_1d(grid, block)
    n_blocks = int(bidx.max()) + 1
    mc = np.ones((1, 1)) if mc is None else np.asarray(mc, np.float64)
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    v = np.asarray(v, np.float64)
    S, z = F.block_summaries(kt, v, bidx, n_blocks)
    # earlier blocks: S~<_i = sum_{b < i} m_ib S_b (the strictly lower part of M_c)
    St_prev, zt_prev = F.mix_summaries(np.tril(mc, -1), S, z)
    out = np.empty((qt.shape[0], v.shape[1]))
    for i in range(n_blocks):
        sel = np.nonzero(bidx == i)[0]            # the block's tokens, in sequence order
        run_S = np.zeros_like(S[0])               # sum of k~_j v_j^T over the block so far
        run_z = np.zeros_like(z[0])
        for t in sel:
            run_S += np.outer(kt[t], v[t])        # token t sees itself
            run_z += kt[t]
            num = qt[t] @ (St_prev[i] + mc[i, i] * run_S)
            if normalized:
                num = num / (qt[t] @ (zt_prev[i] + mc[i, i] * run_z))
            out[t] = num
    return out


def causal_plain(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    """The masked token-level sum with the N x N weight matrix written out."""
    bidx = _blocks_1d(grid, block)
    mc = np.ones((1, 1)) if mc is None else mc
    A = F.mhla_attention_matrix(F.phi_map(q, phi), F.phi_map(k, phi), mc, bidx)
    A = np.tril(A)                                # t' <= t
    num = A @ np.asarray(v, np.float64)
    return num / A.sum(axis=1)[:, None] if normalized else num


def causal_sampled(q, k, v, mc, grid, block, tokens, normalized=True, phi="elu1"):
    """The masked sum for the query tokens ``tokens`` only, O(N d) each."""
    bidx = _blocks_1d(grid, block)
    mc = np.ones((1, 1)) if mc is None else np.asarray(mc, np.float64)
    kt = F.phi_map(k, phi)
    v = np.asarray(v, np.float64)
    out = np.empty((len(tokens), v.shape[1]))
    for r, t in enumerate(tokens):
        w = mc[bidx[t], bidx[:t + 1]] * (kt[:t + 1] @ F.phi_map(q[t], phi))
        out[r] = (w @ v[:t + 1]) / (w.sum() if normalized else 1.0)
    return out


def forward_causal(q, k, v, mc, grid, block, mode="normalized", heads=None, phi="elu1"):
    """Batched over [B, H, N, d]; ``heads`` restricts to a list of (b, h) pairs."""
    if mode not in ("normalized", "unnormalized"):
        raise ValueError(mode)
    q = np.asarray(q)
    B, H, N, d = q.shape
    n_blocks = int(_blocks_1d(grid, block).max()) + 1
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = np.empty((len(pairs), N, np.asarray(v).shape[-1]))
    for r, (b, h) in enumerate(pairs):
        mch = F._as_head_mc(mc, h, n_blocks)
        out[r] = causal_blockwise(q[b, h], k[b, h], v[b, h], mch, grid, block, mode == "normalized", phi)
    if heads is None:
        return out.reshape(B, H, N, -1)
    return out


def forward_causal_sampled(q, k, v, mc, grid, block, samples, mode="normalized", phi="elu1"):
    """``samples`` = list of (b, h, [tokens]); returns a list of float64 [len(tokens), d]."""
    n_blocks = int(_blocks_1d(grid, block).max()) + 1
    res = []
    for b, h, toks in samples:
        mch = F._as_head_mc(mc, h, n_blocks)
        res.append(causal_sampled(q[b, h], k[b, h], v[b, h], mch, grid, block, toks, mode == "normalized", phi))
    return res
