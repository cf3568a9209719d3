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


def phi_exp(x):
    return np.exp(x)


def causal_1d(q, k, v, mc, n_b, *, q_single=False, k_single=False, p_mode="exact", stack=False):
    """Chunkwise-causal MHLA readout of one head (1D, blocks of n_b tokens, one token slice per
    block) as the bf16-input slice kernel computes it: o_t = (q~_t S0_i + sum_{j<=t in i} P_tj v_j)
    / (q~_t z0_i + sum_{j<=t in i} P_tj) with S0_i = sum_{b<i} m_ib S_b, z0_i likewise and
    P_tj = q~_t . m_ii k~_j.  Rounds: phi(q) and m_ii phi(K) to single bf16 (the scores' and the
    S0 readout's MFMA operands), P to single bf16 ("bf") or hi + lo ("split") as the B operand of
    V^T P, and (stack) the bf16 summary and mixed stacks.  The normaliser sums P unrounded."""
    n, d = q.shape
    m = n // n_b
    pk = phi_elu1(k)
    s = np.einsum("bjk,bjc->bkc", pk.reshape(m, n_b, d), v.reshape(m, n_b, d))
    z = pk.reshape(m, n_b, d).sum(1)
    if stack:
        s = bf(s)
    out = np.empty_like(q)
    rp = {"exact": lambda x: x, "bf": bf, "split": split}[p_mode]
    for i in range(m):
        sl = slice(i * n_b, (i + 1) * n_b)
        s0 = np.einsum("b,bkc->kc", mc[i, :i], s[:i]) if i else np.zeros((d, d))
        if stack:
            s0 = bf(s0)
        z0 = mc[i, :i] @ z[:i] if i else np.zeros(d)
        qt = phi_elu1(q[sl])
        qt = bf(qt) if q_single else qt
        kt = mc[i, i] * pk[sl]
        kt = bf(kt) if k_single else kt
        p = np.tril(qt @ kt.T)
        out[sl] = (qt @ s0 + rp(p) @ v[sl]) / (qt @ z0 + p.sum(1))[:, None]
    return out


def causal_rel(got, want):
    """max |got - want| / max(RMS(want), |want|) elementwise (the causal readout's metric)."""
    rms = float(np.sqrt(np.mean(want ** 2)))
    return float(np.max(np.abs(got - want) / np.maximum(rms, np.abs(want))))


def backward_key_side(q, k, v, mc, do, n_b, phi="elu1", *, ds_single=False, phik_single=False):
    """dK and dV of L = sum(dO * O) for one head of the normalised MHLA readout (1D, blocks of
    n_b), by the chain rule of the forward steps, with the key-side products' operands optionally
    single bf16: dS (in dk~ = dS v + dz and dv = dS^T phi(k)) and phi(K) (in dv).  Everything
    before (S~, g, dS~, dS = M_c^T dS~, dz) is exact."""
    f, df = (phi_elu1, lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))) if phi == "elu1" \
        else (phi_exp, phi_exp)
    n, d = q.shape
    m = n // n_b
    pq, pk = f(q), f(k)
    kb, vb, qb, dob = (x.reshape(m, n_b, d) for x in (pk, v, pq, do))
    s = np.einsum("bjk,bjc->bkc", kb, vb)
    z = kb.sum(1)
    st = np.einsum("ib,bkc->ikc", mc, s)
    zt = mc @ z
    num = np.einsum("itk,ikc->itc", qb, st)
    den = np.einsum("itk,ik->it", qb, zt)
    o = num / den[..., None]
    g = dob / den[..., None]
    gden = -np.einsum("itc,itc->it", dob, o) / den
    dst = np.einsum("itk,itc->ikc", qb, g)
    dzt = np.einsum("itk,it->ik", qb, gden)
    ds = np.einsum("ib,ikc->bkc", mc, dst)
    dz = mc.T @ dzt
    ds_r = bf(ds) if ds_single else ds
    kb_r = bf(kb) if phik_single else kb
    dkt = np.einsum("bkc,bjc->bjk", ds_r, vb) + dz[:, None, :]
    dv = np.einsum("bkc,bjk->bjc", ds_r, kb_r)
    return (dkt.reshape(n, d) * df(k)), dv.reshape(n, d)
