"""Pins for ragged blocks (a grid the blocks do not divide) and the CLS token.

Each ``pin_*`` takes the forward oracle module and raises AssertionError on disagreement with:
the plain N x N token-level sum; the strict oracle where the blocks do divide the grid; textbook
linear attention per block for M_c = I, with blocks found by explicit coordinate ranges; the
CLS token's closed form (its output is v_0 when it mixes only with itself); the block sizes
counted from clipped extents; and the general rank bound of the MHLA page (Key design 1),
rank(A) <= min(N, sum_b min(n_b, d)), stated there for any block sizes.
"""
from __future__ import annotations

import itertools

import numpy as np

SHAPES = [((10,), (3,)), ((7, 9), (3, 4)), ((5, 6, 7), (2, 4, 3)), ((4, 4), (4, 4)), ((9,), (20,))]


def _close(a, b, rtol=1e-9, atol=1e-11):
    np.testing.assert_allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rtol, atol=atol)


def _n_tokens(grid, cls):
    return int(np.prod(grid)) + (1 if cls else 0)


def explicit_blocks(grid, block, cls):
    """Token lists of every block from explicit coordinate ranges (raster order everywhere)."""
    nb = [-(-g // b) for g, b in zip(grid, block)]
    blocks = [[0]] if cls else []
    strides = [int(np.prod(grid[k + 1:])) for k in range(len(grid))]
    for bc in itertools.product(*[range(n) for n in nb]):
        ranges = [range(c * b, min((c + 1) * b, g)) for c, b, g in zip(bc, block, grid)]
        toks = [sum(x * s for x, s in zip(xs, strides)) + (1 if cls else 0) for xs in itertools.product(*ranges)]
        blocks.append(sorted(toks))
    return blocks


def _textbook(qt, kt, v):
    return (qt @ (kt.T @ v)) / (qt @ kt.sum(axis=0))[:, None]


def pin_ragged_block_index_matches_explicit_ranges(F):
    for (grid, block), cls in itertools.product(SHAPES, (False, True)):
        bidx = F.block_index(F.RaggedGrid(grid, block, cls), None)
        blocks = explicit_blocks(grid, block, cls)
        assert len(bidx) == _n_tokens(grid, cls)
        assert int(bidx.max()) + 1 == len(blocks)
        for b, toks in enumerate(blocks):
            assert sorted(np.nonzero(bidx == b)[0].tolist()) == toks


def pin_ragged_blockwise_equals_plain(F):
    rng = np.random.default_rng(401)
    for (grid, block), cls in itertools.product(SHAPES, (False, True)):
        g = F.RaggedGrid(grid, block, cls)
        n = _n_tokens(grid, cls)
        m = int(F.block_index(g, None).max()) + 1
        for phi in ("elu1", "relu", "exp"):
            q, k, v = (rng.standard_normal((n, 4)) for _ in range(3))
            if phi == "relu":
                q = np.abs(q) + 0.1
            mc = rng.uniform(0.05, 1.0, (m, m))
            for normalized in (True, False):
                _close(F.mhla_blockwise(q, k, v, mc, g, None, normalized, phi),
                       F.mhla_plain(q, k, v, mc, g, None, normalized, phi))


def pin_dividing_grid_equals_strict(F):
    rng = np.random.default_rng(402)
    for grid, block in (((12,), (4,)), ((6, 8), (3, 4)), ((4, 6, 4), (2, 3, 2))):
        n = int(np.prod(grid))
        m = int(np.prod([g // b for g, b in zip(grid, block)]))
        q, k, v = (rng.standard_normal((n, 5)) for _ in range(3))
        mc = rng.uniform(0.0, 1.0, (m, m))
        _close(F.mhla_blockwise(q, k, v, mc, F.RaggedGrid(grid, block), None),
               F.mhla_blockwise(q, k, v, mc, grid, block))


def pin_identity_mixing_is_textbook_per_block(F):
    rng = np.random.default_rng(403)
    for (grid, block), cls in itertools.product(SHAPES[:3], (False, True)):
        n = _n_tokens(grid, cls)
        blocks = explicit_blocks(grid, block, cls)
        q, k, v = (rng.standard_normal((n, 4)) for _ in range(3))
        got = F.mhla_blockwise(q, k, v, np.eye(len(blocks)), F.RaggedGrid(grid, block, cls), None)
        qt, kt = F.phi_map(q), F.phi_map(k)
        for toks in blocks:
            _close(got[toks], _textbook(qt[toks], kt[toks], v[toks]))


def pin_cls_token_closed_form(F):
    rng = np.random.default_rng(404)
    grid, block = (6, 6), (3, 3)
    q, k, v = (rng.standard_normal((37, 4)) for _ in range(3))
    got = F.mhla_blockwise(q, k, v, np.eye(5), F.RaggedGrid(grid, block, True), None)
    _close(got[0], v[0])                         # a block of one token attends to itself only
    _close(got[1:], F.mhla_blockwise(q[1:], k[1:], v[1:], np.eye(4), grid, block))


def pin_general_rank_bound(F):
    rng = np.random.default_rng(405)
    d = 3
    for (grid, block), cls in (((13,), (5,)), False), (((7, 5), (3, 2)), True), (((10,), (4,)), True):
        g = F.RaggedGrid(grid, block, cls)
        bidx = F.block_index(g, None)
        n, m = len(bidx), int(bidx.max()) + 1
        sizes = np.bincount(bidx)
        bound = min(n, int(np.minimum(sizes, d).sum()))
        qt, kt = F.phi_map(rng.standard_normal((n, d))), F.phi_map(rng.standard_normal((n, d)))
        A = F.mhla_attention_matrix(qt, kt, rng.uniform(0.1, 1.0, (m, m)), bidx)
        assert np.linalg.matrix_rank(A) <= bound
        assert np.linalg.matrix_rank(A) == bound          # attained by generic inputs


ALL_RAGGED_PINS = [pin_ragged_block_index_matches_explicit_ranges, pin_ragged_blockwise_equals_plain,
                   pin_dividing_grid_equals_strict, pin_identity_mixing_is_textbook_per_block,
                   pin_cls_token_closed_form, pin_general_rank_bound]
