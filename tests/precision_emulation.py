"""CPU emulation of the bf16 roundings the forward kernels make, used to choose operand
precisions.  Test infrastructure only (it shares nothing with the HIP path and is not the oracle):
each step of "MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head"
(Method -> Overall framework and Key design 2) and of the MALA readout ("Rectifying Magnitude
Neglect in Linear Attention", Method -> Key design) is computed in fp64, with chosen operands
rounded to bf16 (round to nearest even) where a kernel feeds them to a bf16 MFMA or stores them
as bf16, or split into a bf16 pair hi + lo (hi = bf16(x), lo = bf16(x - hi)) where a kernel
splits them.
"""
from __future__ import annotations

import numpy as np

import synth


def bf(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (RNE) and back to float64."""
    return synth.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def split(x: np.ndarray) -> np.ndarray:
    """x as the sum of its two bf16 parts hi + lo (exact to about 2^-17 relative)."""
    hi = bf(x)
    return hi + bf(np.asarray(x, np.float64) - hi)


def phi_elu1(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def mhla_1d(q, k, v, mc, n_b, *, phi_k=False, stack=False, mc_r=False, mixed=False, phi_q=False):
    """One head, a 1D sequence in blocks of n_b tokens.  Flags round: phi(K) (the summary's MFMA
    operand), the bf16 summary stack, M_c (the mixing MFMA's weights), the mixed stack S~ (bf16
    stack or the readout's bf16 LDS operand), phi(Q) (the readout's MFMA operand).  z and z~ stay
    fp32-exact (the kernels carry them as fp32 or hi + lo)."""
    n, d = q.shape
    m = n // n_b
    pk = phi_elu1(k)
    pk_r = bf(pk) if phi_k else pk
    kb = pk_r.reshape(m, n_b, d)
    vb = v.reshape(m, n_b, d)
    s = np.einsum("bjk,bjc->bkc", kb, vb)
    z = np.einsum("bjk->bk", pk.reshape(m, n_b, d))
    if stack:
        s = bf(s)
    w = bf(mc) if mc_r else mc
    st = np.einsum("ib,bkc->ikc", w, s)
    zt = mc @ z
    if mixed:
        st = bf(st)
    pq = phi_elu1(q)
    pq = bf(pq) if phi_q else pq
    qb = pq.reshape(m, n_b, d)
    num = np.einsum("itk,ikc->itc", qb, st)
    den = np.einsum("itk,ik->it", qb, zt)
    return (num / den[..., None]).reshape(n, d)


def mala(q, k, v, *, naive=False, rounding=None):
    """MALA readout of one head (M = 1).  naive: Y = beta q~^T S - gamma u (the page's linear form
    evaluated as written); otherwise Y = u/N + beta q~^T C with C = S - z u^T / N formed in fp32.
    `rounding` (bf, split or None) is applied to the MFMA operands phi(K), phi(Q) and to S (naive)
    or C; the normaliser q~^T z stays fp32-exact."""
    r = rounding or (lambda x: x)
    n, d = q.shape
    pk = phi_elu1(k)
    s = r(pk).T @ v
    z = pk.sum(0)
    u = v.sum(0)
    pq = phi_elu1(q)
    sq = pq @ z
    beta = 1.0 + 1.0 / sq
    if naive:
        return beta[:, None] * (r(pq) @ r(s)) - (sq / n)[:, None] * u[None, :]
    c = s - np.outer(z, u) / n
    return u[None, :] / n + beta[:, None] * (r(pq) @ r(c))


def rel(got, want):
    return float(np.max(np.abs(got - want)) / np.sqrt(np.mean(want ** 2)))
