"""Pins that tie the fp64 backward oracle to independent computations.

Each ``pin_*`` takes the backward oracle module and raises AssertionError on disagreement with:
torch float64 autograd of the plain N x N forward definition (a different computation from the
oracle's hand-derived chain rule), central finite differences, or homogeneity identities that
any correct gradient satisfies.  ``test_oracle_backward_mutations.py`` plants mistakes.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.mhla_oracle as F

GEOMS = [((12,), (4,)), ((6, 8), (3, 4)), ((4, 6, 4), (2, 3, 2)), ((10,), (10,))]


def _t(x):
    return torch.tensor(np.asarray(x, np.float64), dtype=torch.float64, requires_grad=True)


def _phi_t(x, phi):
    return {"elu1": lambda: torch.nn.functional.elu(x) + 1.0, "relu": lambda: torch.relu(x),
            "exp": lambda: torch.exp(x)}[phi]()


def autograd_mhla(q, k, v, mc, grid, block, do, normalized, phi):
    """torch float64 autograd of the plain definition: o = (A v) / (A 1), A = m_{b(t)b(t')} q~.k~."""
    bidx = F.block_index(grid, block)
    tq, tk, tv, tm = _t(q), _t(k), _t(v), _t(mc)
    idx = torch.as_tensor(bidx)
    A = tm[idx][:, idx] * (_phi_t(tq, phi) @ _phi_t(tk, phi).T)
    o = A @ tv
    if normalized:
        o = o / A.sum(dim=1, keepdim=True)
    (o * torch.as_tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tm.grad.numpy(), o.detach().numpy()


def autograd_mala(q, k, v, do, phi):
    tq, tk, tv = _t(q), _t(k), _t(v)
    a = _phi_t(tq, phi) @ _phi_t(tk, phi).T
    s = a.sum(dim=1, keepdim=True)
    W = (1.0 + 1.0 / s) * a - s / a.shape[1]
    y = W @ tv
    (y * torch.as_tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), y.detach().numpy()


def _close(a, b, rtol=1e-9, atol=1e-11):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rtol, atol=atol)


def _case(rng, grid, block, d=4, positive_q=False):
    n = int(np.prod(grid))
    m = int(np.prod([g // b for g, b in zip(grid, block)]))
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    if positive_q:
        q = np.abs(q) + 0.1
    mc = rng.uniform(0.05, 1.0, (m, m))
    return q, k, v, do, mc


def pin_bwd_matches_autograd(B):
    rng = np.random.default_rng(31)
    for phi in ("elu1", "relu", "exp"):
        for grid, block in GEOMS:
            q, k, v, do, mc = _case(rng, grid, block, positive_q=(phi == "relu"))
            for norm in (True, False):
                got = B.mhla_backward_blockwise(q, k, v, mc, grid, block, do, norm, phi)
                want = autograd_mhla(q, k, v, mc, grid, block, do, norm, phi)
                for g, w in zip(got, want[:4]):
                    _close(g, w)


def pin_bwd_mala_matches_autograd(B):
    rng = np.random.default_rng(32)
    for phi in ("elu1", "exp", "relu"):
        n, d = 14, 5
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        if phi == "relu":
            q = np.abs(q) + 0.1
        got = B.mala_backward(q, k, v, do, phi)
        want = autograd_mala(q, k, v, do, phi)
        for g, w in zip(got, want[:3]):
            _close(g, w)


def pin_bwd_finite_differences(B):
    """Central differences of L = sum(dO * O) for a few coordinates of every input."""
    rng = np.random.default_rng(33)
    grid, block = (8,), (4,)
    q, k, v, do, mc = _case(rng, grid, block, d=3)
    h = 1e-6

    def loss(q_, k_, v_, mc_):
        return float(np.sum(F.mhla_blockwise(q_, k_, v_, mc_, grid, block, True) * do))

    dq, dk, dv, dmc = B.mhla_backward_blockwise(q, k, v, mc, grid, block, do, True)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("mc", mc, dmc)):
        for idx in [(0, 0), (arr.shape[0] - 1, arr.shape[1] - 1), (1, 1)]:
            plus, minus = [x.copy() for x in (q, k, v, mc)], [x.copy() for x in (q, k, v, mc)]
            pos = ["q", "k", "v", "mc"].index(name)
            plus[pos][idx] += h
            minus[pos][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def pin_bwd_homogeneity(B):
    """Normalised O is homogeneous of degree 0 in M_c, unnormalised of degree 1, both linear in V;
    MALA's Y is linear in V.  Euler's identity then fixes sum(M_c * dM_c) and sum(V * dV)."""
    rng = np.random.default_rng(34)
    for grid, block in GEOMS:
        q, k, v, do, mc = _case(rng, grid, block)
        for norm in (True, False):
            o = F.mhla_blockwise(q, k, v, mc, grid, block, norm)
            dq, dk, dv, dmc = B.mhla_backward_blockwise(q, k, v, mc, grid, block, do, norm)
            od = float(np.sum(o * do))
            _close(np.sum(mc * dmc), 0.0 if norm else od, rtol=1e-9, atol=1e-9)
            _close(np.sum(v * dv), od, rtol=1e-9, atol=1e-9)
    n, d = 12, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    _, _, dv = B.mala_backward(q, k, v, do)
    _close(np.sum(v * dv), np.sum(F.mala_linear(q, k, v) * do), rtol=1e-9, atol=1e-9)


def pin_bwd_batched(B):
    """The batched driver equals per-head calls; a shared M_c gathers every head's dM_c, a
    per-head one keeps them apart."""
    rng = np.random.default_rng(35)
    Bn, H, grid, block, d = 2, 3, (6, 8), (3, 4), 4
    n, m = 48, 4
    q, k, v, do = (rng.standard_normal((Bn, H, n, d)) for _ in range(4))
    mc = rng.uniform(0.05, 1, (m, m))
    mch = rng.uniform(0.05, 1, (H, m, m))
    dq, dk, dv, dmc = B.backward(q, k, v, mc, grid, block, do)
    _, _, _, dmch = B.backward(q, k, v, mch, grid, block, do)
    tot = np.zeros((m, m))
    toth = np.zeros((H, m, m))
    for b in range(Bn):
        for h in range(H):
            r = B.mhla_backward_blockwise(q[b, h], k[b, h], v[b, h], mc, grid, block, do[b, h])
            _close(dq[b, h], r[0])
            _close(dk[b, h], r[1])
            _close(dv[b, h], r[2])
            tot += r[3]
            toth[h] += B.mhla_backward_blockwise(q[b, h], k[b, h], v[b, h], mch[h], grid, block, do[b, h])[3]
    _close(dmc, tot)
    _close(dmch, toth)
    dqm, _, _, none = B.backward(q, k, v, None, grid, grid, do, mode="mala")
    assert none is None
    _close(dqm[1, 2], B.mala_backward(q[1, 2], k[1, 2], v[1, 2], do[1, 2])[0])


def pin_dphi(B):
    x = np.array([-2.0, -1e-9, 0.0, 1e-9, 3.0])
    _close(B.dphi_map(x, "elu1"), [np.exp(-2.0), np.exp(-1e-9), 1.0, 1.0, 1.0], rtol=1e-15, atol=0)
    _close(B.dphi_map(x, "relu"), [0.0, 0.0, 0.0, 1.0, 1.0], rtol=0, atol=0)
    _close(B.dphi_map(x, "exp"), np.exp(x), rtol=1e-15, atol=0)


ALL_BACKWARD_PINS = [pin_dphi, pin_bwd_matches_autograd, pin_bwd_mala_matches_autograd,
                     pin_bwd_finite_differences, pin_bwd_homogeneity, pin_bwd_batched]
