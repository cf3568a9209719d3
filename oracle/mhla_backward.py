"""fp64 CPU oracle for the backward pass of the MHLA / MALA forward (gradients of a scalar loss
L = sum(dO * O) with respect to Q, K, V and M_c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.  The GPU
library never calls it and shares no code with it; this file imports NumPy and the forward
oracle only.

Sources (page titles and sections):
  [MHLA]  "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
          Method -> Key design 3: M_c is a learnable parameter trained end to end (clipped to
          (0, 1) after each update -- an optimiser step, not part of the gradient); Overall
          framework and Key design 2 for the forward steps differentiated here.
  [MALA]  "Rectifying Magnitude Neglect in Linear Attention", Method -> Key design (beta,
          gamma and the linear form).

The pages state no gradient formulas; the backward is the chain rule of the forward steps,
taken in reverse order of the forward oracle:
  forward   q~ = phi(q), k~ = phi(k); S_b = sum_{j in b} k~_j v_j^T, z_b = sum k~_j;
            S~ = M_c S, z~ = M_c z; num_t = S~_i^T q~_t, den_t = q~_t . z~_i;
            o_t = num_t / den_t (normalised) or num_t.
  backward  g_t = dO_t / den_t, gden_t = -(dO_t . o_t) / den_t  (normalised; else dO_t, 0)
            dq~_t = S~_i g_t + z~_i gden_t
            dS~_i = sum_{t in i} q~_t g_t^T, dz~_i = sum_{t in i} q~_t gden_t
            dM_c[i, b] = <dS~_i, S_b> + <dz~_i, z_b>
            dS_b = sum_i m_ib dS~_i, dz_b = sum_i m_ib dz~_i
            dk~_j = dS_b v_j + dz_b, dv_j = dS_b^T k~_j
            dq = dq~ * phi'(q), dk = dk~ * phi'(k).
Readings: phi'(0) = 1 for ELU+1 (both one-sided derivatives are 1) and 0 for ReLU.
"""
from __future__ import annotations

import numpy as np

from . import mhla_oracle as F

__all__ = ["dphi_map", "mhla_backward_blockwise", "mala_backward", "backward"]


def dphi_map(x, phi="elu1"):
    """Derivative of the feature map, elementwise."""
    x = np.asarray(x, np.float64)
    if phi == "elu1":
        return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))
    if phi == "relu":
        return (x > 0.0).astype(np.float64)
    if phi == "exp":
        return np.exp(x)
    raise ValueError(phi)


def mhla_backward_blockwise(q, k, v, mc, grid, block, do, normalized=True, phi="elu1"):
    """One (batch, head): returns dq, dk, dv [N, d] and dM_c [M, M]."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    bidx = F.block_index(grid, block)
    n_blocks = int(bidx.max()) + 1
    mc = np.ones((1, 1)) if mc is None else np.asarray(mc, np.float64)
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    # forward steps, kept for the backward
    S, z = F.block_summaries(kt, v, bidx, n_blocks)
    St, zt = F.mix_summaries(mc, S, z)
    # readout backward, block by block
    dSt = np.zeros_like(St)
    dzt = np.zeros_like(zt)
    dqt = np.zeros_like(qt)
    for i in range(n_blocks):
        sel = np.nonzero(bidx == i)[0]
        if sel.size == 0:
            continue
        num = qt[sel] @ St[i]
        if normalized:
            den = qt[sel] @ zt[i]
            o = num / den[:, None]
            g = do[sel] / den[:, None]
            gden = -np.sum(do[sel] * o, axis=1) / den
        else:
            g = do[sel]
            gden = np.zeros(sel.size)
        dqt[sel] = g @ St[i].T + gden[:, None] * zt[i][None, :]
        dSt[i] = qt[sel].T @ g
        dzt[i] = qt[sel].T @ gden
    # mixing backward
    m = n_blocks
    dmc = dSt.reshape(m, -1) @ S.reshape(m, -1).T + dzt @ z.T
    dS = (mc.T @ dSt.reshape(m, -1)).reshape(S.shape)
    dz = mc.T @ dzt
    # summary backward: every token of block b goes through dS_b and dz_b
    dkt = np.empty_like(kt)
    dv = np.empty_like(v)
    for b in range(n_blocks):
        sel = np.nonzero(bidx == b)[0]
        dkt[sel] = v[sel] @ dS[b].T + dz[b][None, :]
        dv[sel] = kt[sel] @ dS[b]
    return dqt * dphi_map(q, phi), dkt * dphi_map(k, phi), dv, dmc


def mala_backward(q, k, v, do, phi="elu1"):
    """One (batch, head), one block: dq, dk, dv of Y = beta q~^T S - gamma u,
    beta = 1 + 1/s, gamma = s / N, s = q~ . z."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    n = kt.shape[0]
    S = kt.T @ v                        # [d, dv]
    z = kt.sum(axis=0)                  # [d]
    u = v.sum(axis=0)                   # [dv]
    s = qt @ z                          # [N]
    beta = 1.0 + 1.0 / s
    gamma = s / n
    a = qt @ S                          # q~^T S   [N, dv]
    # Y = beta a - gamma u
    da = beta[:, None] * do
    dbeta = np.sum(do * a, axis=1)
    dgamma = -(do @ u)
    du = -(gamma @ do)
    ds = dbeta * (-1.0 / s ** 2) + dgamma / n
    dqt = da @ S.T + ds[:, None] * z[None, :]
    dS = qt.T @ da
    dz = qt.T @ ds
    dkt = v @ dS.T + dz[None, :]
    dv = kt @ dS + du[None, :]
    return dqt * dphi_map(q, phi), dkt * dphi_map(k, phi), dv


def backward(q, k, v, mc, grid, block, do, mode="normalized", heads=None, phi="elu1"):
    """Batched over [B, H, N, d].  Returns dq, dk, dv like the inputs and dM_c: summed over
    batch and heads for a shared [M, M] M_c, over batch for a per-head [H, M, M] one, None for
    MALA.  ``heads`` restricts dq, dk, dv to a list of (b, h) pairs ([len(heads), N, d]) and
    dM_c to their contributions."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    n_blocks = int(F.block_index(grid, block).max()) + 1
    F._check_mode(mode, n_blocks)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    dq = np.empty((len(pairs), N, d))
    dk = np.empty((len(pairs), N, d))
    dv = np.empty((len(pairs), N, np.asarray(v).shape[-1]))
    dmc = None
    if mode != "mala":
        per_head = mc is not None and np.ndim(mc) == 3
        dmc = np.zeros((H, n_blocks, n_blocks) if per_head else (n_blocks, n_blocks))
    for r, (b, h) in enumerate(pairs):
        args = (q[b, h], k[b, h], v[b, h])
        if mode == "mala":
            dq[r], dk[r], dv[r] = mala_backward(*args, do[b, h], phi)
        else:
            mch = F._as_head_mc(mc, h, n_blocks)
            dq[r], dk[r], dv[r], g = mhla_backward_blockwise(*args, mch, grid, block, do[b, h],
                                                             mode == "normalized", phi)
            if dmc.ndim == 3:
                dmc[h] += g
            else:
                dmc += g
    if heads is None:
        shape = (B, H, N, -1)
        return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape), dmc
    return dq, dk, dv, dmc
