"""Pins that tie the chunkwise-causal oracle to independent computations.

Each ``pin_*`` takes the causal oracle module and raises AssertionError on disagreement with:
the masked N x N sum written out (``causal_plain``), textbook causal linear attention built from
cumulative sums over the whole sequence (M = 1, and block by block for M_c = I), the non-causal
oracle (the sequence's last token sees everything), and the defining properties of causality
(no output depends on a later token; M_c above its diagonal is never read).
``test_oracle_causal.py`` plants mistakes that the pins must catch.
"""
from __future__ import annotations

import numpy as np

import oracle.mhla_oracle as F

PHIS = ("elu1", "relu", "exp")


def _close(a, b, rtol=1e-9, atol=1e-11):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rtol, atol=atol)


def _inputs(rng, n, d=5, positive_q=False):
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    if positive_q:
        q = np.abs(q) + 0.1
    return q, k, v


def textbook_causal(q, k, v, phi, normalized=True):
    """Causal linear attention from prefix sums over the sequence: o_t = q~_t^T P_t / q~_t^T p_t,
    P_t = cumsum_j<=t k~_j v_j^T, p_t = cumsum_j<=t k~_j (torch-free, written independently)."""
    qt = F.phi_map(q, phi)
    kt = F.phi_map(k, phi)
    P = np.cumsum(np.einsum("jf,jc->jfc", kt, np.asarray(v, np.float64)), axis=0)
    p = np.cumsum(kt, axis=0)
    num = np.einsum("tf,tfc->tc", qt, P)
    return num / np.einsum("tf,tf->t", qt, p)[:, None] if normalized else num


def pin_causal_blockwise_equals_plain(C):
    rng = np.random.default_rng(301)
    for (n, nb) in ((24, 6), (30, 5), (16, 1), (12, 12), (35, 7)):
        m = n // nb
        for phi in PHIS:
            q, k, v = _inputs(rng, n, positive_q=phi == "relu")
            mc = rng.uniform(-0.5, 1.0, (m, m))        # any sign, upper triangle populated
            for normalized in (True, False):
                _close(C.causal_blockwise(q, k, v, mc, (n,), (nb,), normalized, phi),
                       C.causal_plain(q, k, v, mc, (n,), (nb,), normalized, phi))


def pin_causal_one_block_is_textbook(C):
    rng = np.random.default_rng(302)
    for phi in PHIS:
        q, k, v = _inputs(rng, 40, positive_q=phi == "relu")
        for normalized in (True, False):
            want = textbook_causal(q, k, v, phi, normalized)
            _close(C.causal_blockwise(q, k, v, None, (40,), (40,), normalized, phi), want)
            _close(C.causal_plain(q, k, v, None, (40,), (40,), normalized, phi), want)


def pin_causal_identity_mixing_is_blockwise_textbook(C):
    rng = np.random.default_rng(303)
    n, nb = 36, 9
    q, k, v = _inputs(rng, n)
    got = C.causal_blockwise(q, k, v, np.eye(n // nb), (n,), (nb,))
    for b in range(n // nb):
        s = slice(b * nb, (b + 1) * nb)
        _close(got[s], textbook_causal(q[s], k[s], v[s], "elu1"))


def pin_causal_last_token_sees_everything(C):
    rng = np.random.default_rng(304)
    for (n, nb) in ((24, 6), (20, 20), (27, 3)):
        q, k, v = _inputs(rng, n)
        mc = rng.uniform(0.0, 1.0, (n // nb, n // nb))
        last = C.causal_blockwise(q, k, v, mc, (n,), (nb,))[-1]
        _close(last, F.mhla_blockwise(q, k, v, mc, (n,), (nb,))[-1])


def pin_causal_upper_triangle_unused(C):
    rng = np.random.default_rng(305)
    n, nb = 24, 4
    m = n // nb
    q, k, v = _inputs(rng, n)
    mc = rng.uniform(0.0, 1.0, (m, m))
    base = C.causal_blockwise(q, k, v, mc, (n,), (nb,))
    up = mc + np.triu(rng.uniform(1.0, 2.0, (m, m)), 1)
    _close(C.causal_blockwise(q, k, v, up, (n,), (nb,)), base)
    low = mc + np.tril(np.full((m, m), 0.5), -1)
    assert np.max(np.abs(C.causal_blockwise(q, k, v, low, (n,), (nb,)) - base)) > 1e-3


def pin_causal_no_output_depends_on_a_later_token(C):
    rng = np.random.default_rng(306)
    n, nb = 30, 6
    q, k, v = _inputs(rng, n)
    mc = rng.uniform(0.0, 1.0, (n // nb, n // nb))
    base = C.causal_blockwise(q, k, v, mc, (n,), (nb,))
    for t in (0, 5, 6, 17, 29):
        q2, k2, v2 = (x.copy() for x in (q, k, v))
        for x in (q2, k2, v2):
            x[t + 1:] = rng.standard_normal(x[t + 1:].shape)
        got = C.causal_blockwise(q2, k2, v2, mc, (n,), (nb,))
        _close(got[:t + 1], base[:t + 1])


def pin_causal_sampled_equals_blockwise(C):
    rng = np.random.default_rng(307)
    n, nb = 200, 25
    q, k, v = _inputs(rng, n, d=8)
    mc = rng.uniform(0.0, 1.0, (n // nb, n // nb))
    toks = [0, 1, 24, 25, 26, 99, 150, 199]
    full = C.causal_blockwise(q, k, v, mc, (n,), (nb,))
    _close(C.causal_sampled(q, k, v, mc, (n,), (nb,), toks), full[toks])


ALL_CAUSAL_PINS = [pin_causal_blockwise_equals_plain, pin_causal_one_block_is_textbook,
                   pin_causal_identity_mixing_is_blockwise_textbook, pin_causal_last_token_sees_everything,
                   pin_causal_upper_triangle_unused, pin_causal_no_output_depends_on_a_later_token,
                   pin_causal_sampled_equals_blockwise]
