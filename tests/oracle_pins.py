"""Pins that tie the fp64 oracle to what the pages and mathematics fix.

Each ``pin_*`` function takes the oracle module and raises AssertionError when the
oracle disagrees with a value worked out by hand, a closed form, a textbook special
case computed independently (torch CPU float64 ops), an invariant, or a rank bound.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutations.py``
plants mistakes in the oracle and checks that some pin fails for each.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RTOL = 1e-10


def _frac(a):
    return np.array([[float(Fraction(str(x))) for x in row] for row in a], dtype=np.float64)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, rtol=RTOL, atol=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------------------
# independent textbook computations (torch, float64, CPU)
# ----------------------------------------------------------------------------------------

def torch_phi(x):
    return torch.nn.functional.elu(torch.as_tensor(np.asarray(x), dtype=torch.float64)) + 1.0


def torch_phi_named(x, phi):
    t = torch.as_tensor(np.asarray(x), dtype=torch.float64)
    return {"elu1": lambda: torch.nn.functional.elu(t) + 1.0, "relu": lambda: torch.relu(t),
            "exp": lambda: torch.exp(t)}[phi]()


def textbook_linear_attention(q, k, v, phi="elu1"):
    """Kernelised attention with an explicit N x N score matrix: (phiQ phiK^T V) / (phiQ phiK^T 1)."""
    qt, kt = torch_phi_named(q, phi), torch_phi_named(k, phi)
    a = qt @ kt.T
    vv = torch.as_tensor(np.asarray(v), dtype=torch.float64)
    return ((a @ vv) / a.sum(dim=1, keepdim=True)).numpy()


def grid_blocks(grid, block):
    """Token lists of every block, by slicing the grid array (independent of the oracle)."""
    ids = np.arange(int(np.prod(grid))).reshape(grid)
    bg = [g // b for g, b in zip(grid, block)]
    out = []
    for bc in np.ndindex(*bg):
        sl = tuple(slice(c * b, (c + 1) * b) for c, b in zip(bc, block))
        out.append(ids[sl].ravel())
    return out


def _rand(rng, n, d):
    return rng.standard_normal((n, d))


# ----------------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------------

def pin_phi(o):
    x = np.array([0.0, 1.0, -1.0, 2.5, -3.0, 1e-300, -1e-300, -800.0])
    want = np.array([1.0, 2.0, math.exp(-1.0), 3.5, math.exp(-3.0), 1.0, 1.0, 0.0])
    _close(o.phi_elu1(x), want, rtol=1e-15, atol=1e-300)
    # continuity at 0 and positivity
    eps = 1e-8
    assert abs(o.phi_elu1(eps) - o.phi_elu1(-eps)) < 3 * eps
    y = np.linspace(-30, 30, 10001)
    assert np.all(o.phi_elu1(y) > 0)
    # the library routine ELU(x) + 1 (torch forms it as expm1(x) + 1: absolute agreement only)
    _close(o.phi_elu1(y), torch_phi(y).numpy(), rtol=1e-14, atol=1e-15)


def pin_golden_mhla_1d(o):
    g = load_golden("mhla_hand_1d.json")
    args = (np.array(g["q"], float), np.array(g["k"], float), np.array(g["v"], float), _frac(g["mc"]),
            g["grid"], g["block"])
    _close(o.mhla_blockwise(*args, normalized=True), _frac(g["o_normalized"]), rtol=1e-14)
    _close(o.mhla_blockwise(*args, normalized=False), _frac(g["o_unnormalized"]), rtol=1e-14)
    _close(o.mhla_plain(*args, normalized=True), _frac(g["o_normalized"]), rtol=1e-14)
    _close(o.mhla_plain(*args, normalized=False), _frac(g["o_unnormalized"]), rtol=1e-14)
    toks = [3, 0, 2]
    _close(o.mhla_plain_sampled(*args, tokens=toks), _frac(g["o_normalized"])[toks], rtol=1e-14)


def pin_golden_mhla_2d(o):
    g = load_golden("mhla_hand_2d.json")
    args = (np.array(g["q"], float), np.array(g["k"], float), np.array(g["v"], float), _frac(g["mc"]),
            g["grid"], g["block"])
    _close(o.mhla_blockwise(*args), _frac(g["o_normalized"]), rtol=1e-14)
    _close(o.mhla_plain(*args), _frac(g["o_normalized"]), rtol=1e-14)


def pin_golden_mala(o):
    g = load_golden("mala_hand.json")
    q, k, v = (np.array(g[x], float) for x in ("q", "k", "v"))
    _close(o.mala_weights(o.phi_elu1(q), o.phi_elu1(k)), _frac(g["weights"]), rtol=1e-14)
    _close(o.mala_linear(q, k, v), _frac(g["y"]), rtol=1e-14)
    _close(o.mala_plain(q, k, v), _frac(g["y"]), rtol=1e-14)
    _close(o.mala_plain_sampled(q, k, v, [1]), _frac(g["y"])[[1]], rtol=1e-14)


GEOMS = [
    ((16,), (4,)), ((12,), (12,)), ((6, 8), (3, 4)), ((6, 8), (6, 2)), ((4, 6, 4), (2, 3, 2)),
    ((8, 8), (4, 4)), ((14, 14), (7, 7)),
]


def pin_blockwise_equals_plain(o, seeds=(0, 1, 2)):
    """Token-expanded identity (MHLA Key design 2): the blockwise pipeline equals the N x N sum,
    also for M_c with negative entries (the identity is pure algebra)."""
    for seed in seeds:
        rng = np.random.default_rng(seed)
        for grid, block in GEOMS:
            n = int(np.prod(grid))
            m = int(np.prod([g // b for g, b in zip(grid, block)]))
            d = 3 + seed
            q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
            mc = rng.uniform(0.05, 1.0, (m, m))
            for norm in (True, False):
                _close(o.mhla_blockwise(q, k, v, mc, grid, block, norm),
                       o.mhla_plain(q, k, v, mc, grid, block, norm), rtol=1e-10, atol=1e-12)
            mc_signed = rng.standard_normal((m, m))
            _close(o.mhla_blockwise(q, k, v, mc_signed, grid, block, False),
                   o.mhla_plain(q, k, v, mc_signed, grid, block, False), rtol=1e-10, atol=1e-10)


def pin_single_block_is_linear_attention(o):
    rng = np.random.default_rng(7)
    for grid in [(20,), (4, 5), (2, 3, 4)]:
        n = int(np.prod(grid))
        q, k, v = _rand(rng, n, 5), _rand(rng, n, 5), _rand(rng, n, 5)
        want = textbook_linear_attention(q, k, v)
        _close(o.mhla_blockwise(q, k, v, None, grid, grid), want)
        _close(o.mhla_blockwise(q, k, v, np.array([[0.37]]), grid, grid), want)   # m_11 cancels


def pin_all_ones_mixing_is_global(o):
    rng = np.random.default_rng(8)
    for grid, block in GEOMS:
        n = int(np.prod(grid))
        m = int(np.prod([g // b for g, b in zip(grid, block)]))
        q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 4)
        _close(o.mhla_blockwise(q, k, v, np.ones((m, m)), grid, block), textbook_linear_attention(q, k, v))


def pin_identity_mixing_is_block_local(o):
    rng = np.random.default_rng(9)
    for grid, block in GEOMS:
        n = int(np.prod(grid))
        m = int(np.prod([g // b for g, b in zip(grid, block)]))
        q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 4)
        got = o.mhla_blockwise(q, k, v, np.eye(m), grid, block)
        want = np.empty_like(got)
        for toks in grid_blocks(grid, block):
            want[toks] = textbook_linear_attention(q[toks], k[toks], v[toks])
        _close(got, want)


def _rank(a):
    s = np.linalg.svd(a, compute_uv=False)
    return int((s > s[0] * 1e-10).sum())


def pin_rank_bounds(o):
    """rank(A_lin) <= d and rank(A_MHLA) <= min(N, sum_b min(n_b, d)) (MHLA Key design 1),
    with d < n_b so the bound is not vacuous; random inputs reach it."""
    rng = np.random.default_rng(10)
    grid, block = (8, 8), (4, 4)
    n, m, nb = 64, 4, 16
    for d in (2, 4, 6):
        q, k = _rand(rng, n, d), _rand(rng, n, d)
        qt, kt = o.phi_elu1(q), o.phi_elu1(k)
        bidx = o.block_index(grid, block)
        bound = min(n, m * min(nb, d))
        r_lin = _rank(o.mhla_attention_matrix(qt, kt, np.ones((m, m)), bidx))
        r_eye = _rank(o.mhla_attention_matrix(qt, kt, np.eye(m), bidx))
        r_rnd = _rank(o.mhla_attention_matrix(qt, kt, rng.uniform(0.1, 1, (m, m)), bidx))
        assert r_lin <= d and r_lin == d, (d, r_lin)
        assert r_eye <= bound and r_eye == bound, (d, r_eye, bound)
        assert r_rnd <= bound and r_rnd == bound, (d, r_rnd, bound)
    # d >= n_b: the bound saturates at N
    d = 16
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    A = o.mhla_attention_matrix(o.phi_elu1(q), o.phi_elu1(k), rng.uniform(0.1, 1, (m, m)),
                                o.block_index(grid, block))
    assert _rank(A) == n


def pin_normalized_invariances(o):
    """Magnitude neglect (MALA, Background: the query norm cancels), M_c row scaling cancels,
    a constant V passes through, linearity in V."""
    rng = np.random.default_rng(11)
    grid, block = (6, 8), (3, 4)
    n, m, d = 48, 4, 5
    bidx = o.block_index(grid, block)
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    mc = rng.uniform(0.1, 1, (m, m))
    qt, kt = o.phi_elu1(q), o.phi_elu1(k)
    S, z = o.block_summaries(kt, v, bidx, m)
    St, zt = o.mix_summaries(mc, S, z)
    base = o.readout(qt, St, zt, bidx)
    scale = rng.uniform(0.1, 10, (n, 1))
    _close(o.readout(qt * scale, St, zt, bidx), base)
    St2, zt2 = o.mix_summaries(mc * rng.uniform(0.1, 10, (m, 1)), S, z)
    _close(o.readout(qt, St2, zt2, bidx), base)
    const = np.tile(rng.standard_normal((1, d)), (n, 1))
    _close(o.mhla_blockwise(q, k, const, mc, grid, block), const)
    v2 = _rand(rng, n, d)
    _close(o.mhla_blockwise(q, k, 2.0 * v - 3.0 * v2, mc, grid, block),
           2.0 * o.mhla_blockwise(q, k, v, mc, grid, block) - 3.0 * o.mhla_blockwise(q, k, v2, mc, grid, block))


def pin_mala_properties(o):
    rng = np.random.default_rng(12)
    n, d = 40, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    qt, kt = o.phi_elu1(q), o.phi_elu1(k)
    W = o.mala_weights(qt, kt)
    _close(W.sum(axis=1), np.ones(n))                                   # weights sum to one
    _close(o.mala_linear(q, k, v), W @ v)                               # linear form == N x N form
    _close(o.mala_plain(q, k, v), W @ v)
    const = np.tile(rng.standard_normal((1, d)), (n, 1))
    _close(o.mala_linear(q, k, const), const)
    # Closed form derived from the linear form: with C = sum_j (k~_j - mean k~) v_j^T,
    # Y = mean(V) + beta * q~^T C.
    C = (kt - kt.mean(axis=0)).T @ v
    beta = 1.0 + 1.0 / (qt @ kt.sum(axis=0))
    _close(o.mala_linear(q, k, v), v.mean(axis=0) + beta[:, None] * (qt @ C))
    # magnitude awareness: unlike normalised linear attention, scaling phi(Q) changes weights,
    # and for positive weights the ratio of a high-score to a low-score key grows (MALA Key design).
    a = 3.0
    W2 = o.mala_weights(a * qt, kt)
    assert np.abs(W2 - W).max() > 1e-3
    for i in range(n):
        pos = W[i] > 0
        if pos.sum() < 2:
            continue
        hi = np.argmax(np.where(pos, W[i], -np.inf))
        lo = np.argmin(np.where(pos, W[i], np.inf))
        if W[i, hi] > W[i, lo] and W2[i, lo] > 0:
            assert W2[i, hi] / W2[i, lo] > W[i, hi] / W[i, lo]


def pin_gather_equals_block_major_1d(o):
    """A 2D/3D tiling equals the 1D path after permuting tokens into block-major order."""
    rng = np.random.default_rng(13)
    for grid, block in GEOMS:
        n = int(np.prod(grid))
        nb = int(np.prod(block))
        m = n // nb
        perm = np.concatenate(grid_blocks(grid, block))
        q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 4)
        mc = rng.uniform(0.05, 1.0, (m, m))
        got = o.mhla_blockwise(q, k, v, mc, grid, block)
        flat = o.mhla_blockwise(q[perm], k[perm], v[perm], mc, (n,), (nb,))
        want = np.empty_like(flat)
        want[perm] = flat
        _close(got, want)


def pin_full_width_tiles_are_spans(o):
    rng = np.random.default_rng(14)
    for grid, block in [((6, 8), (2, 8)), ((4, 3, 5), (2, 3, 5)), ((4, 3, 5), (1, 3, 5))]:
        n = int(np.prod(grid))
        nb = int(np.prod(block))
        m = n // nb
        q, k, v = _rand(rng, n, 3), _rand(rng, n, 3), _rand(rng, n, 3)
        mc = rng.uniform(0.05, 1.0, (m, m))
        _close(o.mhla_blockwise(q, k, v, mc, grid, block), o.mhla_blockwise(q, k, v, mc, (n,), (nb,)))


def pin_batched_forward(o):
    """The [B, H, N, d] driver, shared [M,M] and per-head [H,M,M] M_c, and the sampled driver."""
    rng = np.random.default_rng(15)
    B, H, grid, block, d = 2, 3, (6, 8), (3, 4), 4
    n, m = 48, 4
    q, k, v = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    mc_h = rng.uniform(0.05, 1, (H, m, m))
    out = o.forward(q, k, v, mc_h, grid, block)
    for b in range(B):
        for h in range(H):
            _close(out[b, h], o.mhla_plain(q[b, h], k[b, h], v[b, h], mc_h[h], grid, block))
    samp = o.forward_sampled(q, k, v, mc_h, grid, block, [(1, 2, [0, 5, 47])])
    _close(samp[0], out[1, 2, [0, 5, 47]])
    outm = o.forward(q, k, v, None, grid, grid, mode="mala")
    _close(outm[0, 1], o.mala_plain(q[0, 1], k[0, 1], v[0, 1]))


def pin_phi_maps(o):
    """ReLU and exp ([MALA] Ablation names ELU+1, ReLU and exp): closed-form values and the
    name dispatch."""
    x = np.array([0.0, 1.0, -1.0, 2.5, -3.0, 1e-300, -1e-300, math.log(2.0), -math.log(4.0)])
    _close(o.phi_relu(x), [0.0, 1.0, 0.0, 2.5, 0.0, 1e-300, 0.0, math.log(2.0), 0.0], rtol=1e-15, atol=0)
    _close(o.phi_exp(x), [1.0, math.e, 1 / math.e, math.exp(2.5), math.exp(-3.0), 1.0, 1.0, 2.0, 0.25],
           rtol=1e-15, atol=0)
    assert o.phi_exp(np.array([-800.0]))[0] == 0.0 and np.isinf(o.phi_exp(np.array([800.0]))[0])
    y = np.linspace(-5, 5, 101)
    for name, f in (("elu1", o.phi_elu1), ("relu", o.phi_relu), ("exp", o.phi_exp)):
        _close(o.phi_map(y, name), f(y), rtol=0, atol=0)
    try:
        o.phi_map(y, "gelu")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown feature map accepted")


def pin_other_maps_blockwise_equals_plain(o):
    """The token-expanded identity holds for every feature map (pure algebra), and one block is
    textbook linear attention with that map."""
    rng = np.random.default_rng(21)
    for phi in ("relu", "exp"):
        for grid, block in GEOMS:
            n = int(np.prod(grid))
            m = int(np.prod([g // b for g, b in zip(grid, block)]))
            q, k, v = _rand(rng, n, 6), _rand(rng, n, 6), _rand(rng, n, 6)
            mc = rng.uniform(0.05, 1.0, (m, m))
            for norm in (True, False):
                a = o.mhla_blockwise(q, k, v, mc, grid, block, norm, phi)
                b = o.mhla_plain(q, k, v, mc, grid, block, norm, phi)
                assert np.array_equal(np.isnan(a), np.isnan(b))
                np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12, equal_nan=True)
            toks = [0, n // 2, n - 1]
            np.testing.assert_allclose(o.mhla_plain_sampled(q, k, v, mc, grid, block, toks, True, phi),
                                       o.mhla_plain(q, k, v, mc, grid, block, True, phi)[toks],
                                       rtol=1e-10, atol=1e-12, equal_nan=True)
        for grid in [(20,), (4, 5)]:
            n = int(np.prod(grid))
            q, k, v = _rand(rng, n, 5), _rand(rng, n, 5), _rand(rng, n, 5)
            np.testing.assert_allclose(o.mhla_blockwise(q, k, v, None, grid, grid, True, phi),
                                       textbook_linear_attention(q, k, v, phi), rtol=1e-10,
                                       atol=1e-12, equal_nan=True)


def pin_relu_zero_denominator(o):
    """With ReLU a query whose features are all <= 0 has q~ = 0: numerator and denominator are
    both exactly 0, and the division (no epsilon) gives NaN in the blockwise and plain forms;
    the unnormalised readout gives exact zeros."""
    rng = np.random.default_rng(22)
    grid, block = (12,), (4,)
    q, k, v = np.abs(_rand(rng, 12, 4)), _rand(rng, 12, 4), _rand(rng, 12, 4)
    q[5] = -q[5]
    q[7] = 0.0
    mc = rng.uniform(0.05, 1.0, (3, 3))
    for f in (o.mhla_blockwise, o.mhla_plain):
        with np.errstate(invalid="ignore", divide="ignore"):
            a = f(q, k, v, mc, grid, block, True, "relu")
        assert np.all(np.isnan(a[[5, 7]])) and not np.any(np.isnan(np.delete(a, [5, 7], axis=0)))
        u = f(q, k, v, mc, grid, block, False, "relu")
        assert np.all(u[[5, 7]] == 0.0)


def pin_mala_other_maps(o):
    """MALA under exp and ReLU: weights sum to one, linear form == N x N form."""
    rng = np.random.default_rng(23)
    n, d = 30, 6
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    for phi in ("exp", "relu"):
        qt, kt = o.phi_map(q, phi), o.phi_map(k, phi)
        ok = qt.sum(axis=1) > 0
        W = o.mala_weights(qt[ok], kt)
        _close(W.sum(axis=1), np.ones(ok.sum()))
        _close(o.mala_linear(q, k, v, phi)[ok], W @ v)
        _close(o.mala_plain(q, k, v, phi)[ok], W @ v)
        _close(o.mala_plain_sampled(q, k, v, [int(np.flatnonzero(ok)[0])], phi),
               (W @ v)[:1])


ALL_PINS = [
    pin_phi, pin_golden_mhla_1d, pin_golden_mhla_2d, pin_golden_mala, pin_blockwise_equals_plain,
    pin_single_block_is_linear_attention, pin_all_ones_mixing_is_global, pin_identity_mixing_is_block_local,
    pin_rank_bounds, pin_normalized_invariances, pin_mala_properties, pin_gather_equals_block_major_1d,
    pin_full_width_tiles_are_spans, pin_batched_forward, pin_phi_maps,
    pin_other_maps_blockwise_equals_plain, pin_relu_zero_denominator, pin_mala_other_maps,
]
