"""fp64 CPU oracle for the token-level multi-head linear attention (MHLA) forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The GPU library never calls it, and it shares no code with the GPU path: this
file imports NumPy only.

Sources (page titles and sections):
  [MHLA]  "MHLA: Restoring Expressivity of Linear Attention via Token-Level
          Multi-Head" (ICLR 2026 paper notes).  Sections used: Background and
          motivation (feature map, global summary, rank collapse); Method ->
          Overall framework (blocks, S_b, z_b, M_c, flowchart readout); Key
          design 1 (rank bounds); Key design 2 (mixing, token-expanded identity,
          optional normaliser); Key design 4 (complexity).
  [MALA]  "Rectifying Magnitude Neglect in Linear Attention" (ICCV 2025 paper
          notes).  Section Method -> Key design (MALA formula design: score,
          beta, gamma, normalisation, linear form).

Every function works on float64 and follows the pages' steps in their order.
MHLA is exact: the blockwise pipeline is a reorganisation of one token-level
sum (the token-expanded identity of [MHLA] Key design 2), so ``mhla_plain`` and
``mhla_plain_sampled`` write that sum out, and ``mhla_blockwise`` takes the
pages' steps (phi -> per-block S_b, z_b -> mixing with M_c -> readout).

Readings where the pages are silent (full list in the design notes):
  * phi is ELU+1 with alpha = 1 by default; ReLU (max(x, 0)) and exp (elementwise e^x, no
    shift) are the other maps [MALA] Ablation names as working alike.  No 1/sqrt(d)
    scaling before phi.
  * The readout display equation of Key design 2 did not survive extraction;
    the flowchart gives o = q~^T S~_i / q~^T z~_i, used here.
  * S_b has rows indexed by the key feature, columns by the value feature.
  * Tokens are in raster order over the grid (last axis fastest); blocks are
    numbered in raster order over the block grid; row i of M_c belongs to
    query block i.
  * No epsilon in any division; MALA is defined for one block (M = 1) only.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "RaggedGrid",
    "phi_elu1", "phi_relu", "phi_exp", "phi_map", "block_index", "block_summaries", "mix_summaries", "readout",
    "mhla_blockwise", "mhla_plain", "mhla_plain_sampled", "mhla_attention_matrix",
    "mala_linear", "mala_weights", "mala_plain", "mala_plain_sampled",
    "forward", "forward_sampled",
]


# ----------------------------------------------------------------------------------------
# Step 1: positive feature map  ([MHLA] Background: Sim(Q,K) ~ phi(Q) phi(K)^T with a
# positive phi; [MALA] Ablation: ELU+1, ReLU and exp work alike).
# ----------------------------------------------------------------------------------------

def phi_elu1(x):
    """ELU(x) + 1 with alpha = 1:  x + 1 for x > 0,  exp(x) for x <= 0."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_relu(x):
    """ReLU(x) = max(x, 0)."""
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


def phi_exp(x):
    """e^x elementwise (no max subtraction: the pages give none)."""
    return np.exp(np.asarray(x, dtype=np.float64))


def phi_map(x, phi="elu1"):
    """The feature map named by ``phi``: "elu1" (default), "relu" or "exp"."""
    if phi == "elu1":
        return phi_elu1(x)
    if phi == "relu":
        return phi_relu(x)
    if phi == "exp":
        return phi_exp(x)
    raise ValueError(phi)


# ----------------------------------------------------------------------------------------
# Step 2: token -> block assignment ([MHLA] Overall framework: M non-overlapping blocks,
# defined on the 2D/3D spatial grid for vision rather than on the flattened sequence).
# ----------------------------------------------------------------------------------------

class RaggedGrid:
    """A token grid whose blocks may be cut short at the far edge of each axis, optionally
    preceded by one CLS token (token 0) that forms block 0 on its own.  Passed in place of
    ``grid`` (with ``block`` None) wherever the functions below take (grid, block).

    Readings (the pages' rank bound [MHLA] Key design 1 is stated for a general n_b; DeiT
    carries a CLS token beside its 14 x 14 patch grid): blocks tile the grid from its origin
    with the given extents, the last block along an axis keeping what is left; blocks are
    numbered in raster order over the (rounded-up) block grid, after the CLS block.
    """

    def __init__(self, grid, block, cls=False):
        self.grid = tuple(int(g) for g in grid)
        self.block = tuple(int(b) for b in block)
        self.cls = bool(cls)
        if len(self.grid) != len(self.block) or min(self.block) <= 0 or min(self.grid) <= 0:
            raise ValueError("bad grid or block")


def block_index(grid, block) -> np.ndarray:
    """b(t) for every token t of a grid in raster order (last axis fastest).

    A token with grid coordinates (c_0, ..., c_{n-1}) belongs to the block whose
    block-grid coordinates are (c_k // block_k); blocks are numbered in raster order.
    With a RaggedGrid the block grid is rounded up and a CLS token comes first as block 0.
    """
    cls = False
    if isinstance(grid, RaggedGrid):
        grid, block, cls, ragged = grid.grid, grid.block, grid.cls, True
    else:
        ragged = False
    grid = tuple(int(g) for g in grid)
    block = tuple(int(b) for b in block)
    assert len(grid) == len(block)
    for g, b in zip(grid, block):
        if b <= 0 or (g % b and not ragged):
            raise ValueError("block extents must divide the grid")
    coords = np.indices(grid).reshape(len(grid), -1)          # [ndim, N], raster order
    bcoords = coords // np.asarray(block)[:, None]
    bgrid = [-(-g // b) for g, b in zip(grid, block)]
    bidx = np.ravel_multi_index(tuple(bcoords), bgrid).astype(np.int64)
    if cls:
        bidx = np.concatenate([[0], bidx + 1])
    return bidx


# ----------------------------------------------------------------------------------------
# Step 3: local summaries ([MHLA] Overall framework: S_b = sum_{j in b} K~_j V_j^T and
# z_b = sum_{j in b} K~_j).
# ----------------------------------------------------------------------------------------

def block_summaries(kt, v, bidx, n_blocks):
    """kt = phi(K) [N, d], v [N, dv] -> S [M, d, dv], z [M, d]."""
    kt = np.asarray(kt, np.float64)
    v = np.asarray(v, np.float64)
    d, dv = kt.shape[1], v.shape[1]
    S = np.zeros((n_blocks, d, dv))
    z = np.zeros((n_blocks, d))
    order = np.argsort(bidx, kind="stable")
    bounds = np.searchsorted(bidx[order], np.arange(n_blocks + 1))
    for b in range(n_blocks):
        sel = order[bounds[b]:bounds[b + 1]]          # tokens j with b(j) = b
        kb, vb = kt[sel], v[sel]
        S[b] = kb.T @ vb            # sum over tokens of the outer products k~_j v_j^T
        z[b] = kb.sum(axis=0)
    return S, z


# ----------------------------------------------------------------------------------------
# Step 4: multi-head mixing ([MHLA] Key design 2: S~_i = sum_b m_ib S_b, z~_i = sum_b m_ib z_b,
# row i of M_c belongs to query block i).
# ----------------------------------------------------------------------------------------

def mix_summaries(mc, S, z):
    mc = np.asarray(mc, np.float64)
    m = S.shape[0]
    St = (mc @ S.reshape(m, -1)).reshape(S.shape)     # S~_i = sum_b m_ib S_b
    zt = mc @ z                                       # z~_i = sum_b m_ib z_b
    return St, zt


# ----------------------------------------------------------------------------------------
# Step 5: readout ([MHLA] flowchart: o = q~^T S~_i / q~^T z~_i; Key design 2 allows the
# normaliser to be dropped for long sequences).
# ----------------------------------------------------------------------------------------

def readout(qt, St, zt, bidx, normalized=True):
    """Each query token t of block i = b(t) reads q~_t^T S~_i (and q~_t^T z~_i); evaluated block
    by block so no per-token copy of S~ is ever formed."""
    qt = np.asarray(qt, np.float64)
    out = np.empty((qt.shape[0], St.shape[2]))
    for i in range(St.shape[0]):
        sel = np.nonzero(bidx == i)[0]
        if sel.size == 0:
            continue
        num = qt[sel] @ St[i]
        out[sel] = num / (qt[sel] @ zt[i])[:, None] if normalized else num
    return out


def _as_head_mc(mc, h, n_blocks):
    if mc is None:
        return np.ones((n_blocks, n_blocks)) if n_blocks == 1 else None
    mc = np.asarray(mc, np.float64)
    if mc.ndim == 3:
        return mc[h]
    return mc


def mhla_blockwise(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    """MHLA forward for one (batch, head): q, k, v [N, d] -> o [N, d], pages' step order."""
    bidx = block_index(grid, block)
    n_blocks = int(bidx.max()) + 1
    if mc is None:
        if n_blocks != 1:
            raise ValueError("M_c is required when there is more than one block")
        mc = np.ones((1, 1))
    qt, kt = phi_map(q, phi), phi_map(k, phi)
    S, z = block_summaries(kt, v, bidx, n_blocks)
    St, zt = mix_summaries(mc, S, z)
    return readout(qt, St, zt, bidx, normalized)


# ----------------------------------------------------------------------------------------
# The plain token-level definition ([MHLA] Key design 2, token-expanded identity:
# q~^T S~_i = sum_t m_{i,b(t)} (q~^T K~_t) V_t^T).
# ----------------------------------------------------------------------------------------

def mhla_attention_matrix(qt, kt, mc, bidx):
    """A[t, t'] = m_{b(t), b(t')} * (q~_t . k~_t')   (N x N; tiny inputs only)."""
    qt = np.asarray(qt, np.float64)
    kt = np.asarray(kt, np.float64)
    mc = np.asarray(mc, np.float64)
    return mc[np.ix_(bidx, bidx)] * (qt @ kt.T)


def mhla_plain(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    """o_t = sum_t' A[t,t'] v_t' / sum_t' A[t,t'] with the N x N matrix built explicitly."""
    bidx = block_index(grid, block)
    if mc is None:
        mc = np.ones((1, 1))
    A = mhla_attention_matrix(phi_map(q, phi), phi_map(k, phi), mc, bidx)
    num = A @ np.asarray(v, np.float64)
    if not normalized:
        return num
    return num / A.sum(axis=1)[:, None]


def mhla_plain_sampled(q, k, v, mc, grid, block, tokens, normalized=True, phi="elu1"):
    """The plain definition evaluated for the query tokens ``tokens`` only (O(N d) each)."""
    bidx = block_index(grid, block)
    if mc is None:
        mc = np.ones((1, 1))
    mc = np.asarray(mc, np.float64)
    kt = phi_map(k, phi)
    v = np.asarray(v, np.float64)
    out = np.empty((len(tokens), v.shape[1]))
    for r, t in enumerate(tokens):
        qt = phi_map(q[t], phi)
        w = mc[bidx[t], bidx] * (kt @ qt)
        out[r] = (w @ v) / (w.sum() if normalized else 1.0)
    return out


# ----------------------------------------------------------------------------------------
# MALA readout ([MALA] Method -> Key design): Attn(Q_i, K_j) = beta phi(Q_i) phi(K_j)^T - gamma,
# beta = 1 + 1/(phi(Q_i) sum_m phi(K_m)^T), gamma = phi(Q_i) sum_m phi(K_m)^T / N, and the
# linear form Y_i = beta phi(Q_i) sum_j phi(K_j)^T V_j - gamma sum_j V_j.  One block (M = 1).
# ----------------------------------------------------------------------------------------

def mala_linear(q, k, v, phi="elu1"):
    """The linear-complexity form: compute sum_j phi(K_j)^T V_j first, then read out."""
    qt, kt = phi_map(q, phi), phi_map(k, phi)
    v = np.asarray(v, np.float64)
    n = kt.shape[0]
    kv = kt.T @ v                    # sum_j phi(K_j)^T V_j          [d, dv]
    ksum = kt.sum(axis=0)            # sum_m phi(K_m)                 [d]
    vsum = v.sum(axis=0)             # sum_j V_j                      [dv]
    s = qt @ ksum                    # phi(Q_i) sum_m phi(K_m)^T      [N]
    beta = 1.0 + 1.0 / s
    gamma = s / n
    return beta[:, None] * (qt @ kv) - gamma[:, None] * vsum[None, :]


def mala_weights(qt, kt):
    """N x N MALA attention weights W[i, j] = beta_i a_ij - gamma_i with a = phi(Q) phi(K)^T."""
    a = np.asarray(qt, np.float64) @ np.asarray(kt, np.float64).T
    s = a.sum(axis=1)
    n = a.shape[1]
    beta = 1.0 + 1.0 / s
    gamma = s / n
    return beta[:, None] * a - gamma[:, None]


def mala_plain(q, k, v, phi="elu1"):
    return mala_weights(phi_map(q, phi), phi_map(k, phi)) @ np.asarray(v, np.float64)


def mala_plain_sampled(q, k, v, tokens, phi="elu1"):
    kt = phi_map(k, phi)
    v = np.asarray(v, np.float64)
    n = kt.shape[0]
    out = np.empty((len(tokens), v.shape[1]))
    for r, t in enumerate(tokens):
        a = kt @ phi_map(q[t], phi)
        s = a.sum()
        w = (1.0 + 1.0 / s) * a - s / n
        out[r] = w @ v
    return out


# ----------------------------------------------------------------------------------------
# Batched entry points over [B, H, N, d]
# ----------------------------------------------------------------------------------------

def _check_mode(mode, n_blocks):
    if mode not in ("normalized", "unnormalized", "mala"):
        raise ValueError(mode)
    if mode == "mala" and n_blocks != 1:
        raise ValueError("the MALA readout is defined for a single block (M = 1)")


def forward(q, k, v, mc, grid, block, mode="normalized", heads=None, phi="elu1"):
    """Blockwise oracle over [B, H, N, d] inputs; returns float64 [B, H, N, d].

    ``heads`` optionally restricts the computation to a list of (b, h) pairs; the result
    then has shape [len(heads), N, d].
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    n_blocks = int(block_index(grid, block).max()) + 1
    _check_mode(mode, n_blocks)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = np.empty((len(pairs), N, v.shape[-1]))
    for r, (b, h) in enumerate(pairs):
        qh = q[b, h].astype(np.float64)
        kh = np.asarray(k[b, h], np.float64)
        vh = np.asarray(v[b, h], np.float64)
        if mode == "mala":
            out[r] = mala_linear(qh, kh, vh, phi)
        else:
            mch = _as_head_mc(mc, h, n_blocks)
            out[r] = mhla_blockwise(qh, kh, vh, mch, grid, block, mode == "normalized", phi)
    if heads is None:
        return out.reshape(B, H, N, -1)
    return out


def forward_sampled(q, k, v, mc, grid, block, samples, mode="normalized", phi="elu1"):
    """Plain definition at sampled outputs.  ``samples`` = list of (b, h, [tokens]).
    Returns a list of float64 arrays [len(tokens), d]."""
    n_blocks = int(block_index(grid, block).max()) + 1
    _check_mode(mode, n_blocks)
    res = []
    for b, h, toks in samples:
        qh = np.asarray(q[b, h], np.float64)
        kh = np.asarray(k[b, h], np.float64)
        vh = np.asarray(v[b, h], np.float64)
        if mode == "mala":
            res.append(mala_plain_sampled(qh, kh, vh, toks, phi))
        else:
            mch = _as_head_mc(mc, h, n_blocks)
            res.append(mhla_plain_sampled(qh, kh, vh, mch, grid, block, toks, mode == "normalized", phi))
    return res
