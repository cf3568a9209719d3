"""The chunkwise-causal oracle against independent computations; planted mistakes must each be
caught by at least one pin (CPU only)."""
import types

import numpy as np
import pytest

import oracle.mhla_causal as C
import oracle.mhla_oracle as F
from oracle_causal_pins import ALL_CAUSAL_PINS


@pytest.mark.parametrize("pin", ALL_CAUSAL_PINS, ids=lambda p: p.__name__)
def test_causal_pin(pin):
    pin(C)


def _variant(blockwise=None, plain=None, sampled=None):
    """A copy of the causal oracle module with some functions replaced by planted mistakes."""
    m = types.SimpleNamespace(**{n: getattr(C, n) for n in ("causal_blockwise", "causal_plain", "causal_sampled")})
    if blockwise:
        m.causal_blockwise = blockwise
    if plain:
        m.causal_plain = plain
    if sampled:
        m.causal_sampled = sampled
    return m


def _blockwise_with(q, k, v, mc, grid, block, normalized=True, phi="elu1", *, lower_k=-1, see_self=True,
                    diag_weight=True, transpose=False):
    bidx = F.block_index(grid, block)
    m = int(bidx.max()) + 1
    mc = np.ones((1, 1)) if mc is None else np.asarray(mc, np.float64)
    if transpose:
        mc = mc.T
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    v = np.asarray(v, np.float64)
    S, z = F.block_summaries(kt, v, bidx, m)
    St, zt = F.mix_summaries(np.tril(mc, lower_k), S, z)
    out = np.empty((len(q), v.shape[1]))
    for i in range(m):
        rs, rz = np.zeros_like(S[0]), np.zeros_like(z[0])
        w = mc[i, i] if diag_weight else 1.0
        for t in np.nonzero(bidx == i)[0]:
            if see_self:
                rs += np.outer(kt[t], v[t]); rz += kt[t]
            num = qt[t] @ (St[i] + w * rs)
            out[t] = num / (qt[t] @ (zt[i] + w * rz)) if normalized else num
            if not see_self:
                rs += np.outer(kt[t], v[t]); rz += kt[t]
    return out


def _plain_unmasked(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    return F.mhla_plain(q, k, v, mc, grid, block, normalized, phi)


def _plain_strict(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
    bidx = F.block_index(grid, block)
    mc = np.ones((1, 1)) if mc is None else mc
    A = np.tril(F.mhla_attention_matrix(F.phi_map(q, phi), F.phi_map(k, phi), mc, bidx), -1)
    A[0, 0] = 1e-300   # keep the first row defined
    num = A @ np.asarray(v, np.float64)
    return num / A.sum(axis=1)[:, None] if normalized else num


MUTANTS = {
    "diagonal_block_also_mixed": _variant(blockwise=lambda *a, **kw: _blockwise_with(*a, **kw, lower_k=0)),
    "token_does_not_see_itself": _variant(blockwise=lambda *a, **kw: _blockwise_with(*a, **kw, see_self=False)),
    "in_block_weight_dropped": _variant(blockwise=lambda *a, **kw: _blockwise_with(*a, **kw, diag_weight=False)),
    "mc_transposed": _variant(blockwise=lambda *a, **kw: _blockwise_with(*a, **kw, transpose=True)),
    "plain_not_masked": _variant(plain=_plain_unmasked),
    "plain_strictly_masked": _variant(plain=_plain_strict),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_causal_mistake_is_caught(name):
    mutant = MUTANTS[name]
    caught = []
    for pin in ALL_CAUSAL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
