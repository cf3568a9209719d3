"""The fp64 backward oracle against torch autograd, finite differences and homogeneity
identities; planted mistakes must each be caught (CPU only)."""
import numpy as np
import pytest

import oracle.mhla_backward as B
import oracle.mhla_oracle as F
from oracle_backward_pins import ALL_BACKWARD_PINS


@pytest.mark.parametrize("pin", ALL_BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(B)


_ORIG = B.mhla_backward_blockwise
_ORIG_MALA = B.mala_backward
_ORIG_DPHI = B.dphi_map


def _no_gden(q, k, v, mc, grid, block, do, normalized=True, phi="elu1"):
    """The backward with the normaliser's gradient (gden) dropped: only g = dO / den flows."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    bidx = F.block_index(grid, block)
    m = int(bidx.max()) + 1
    mc = np.ones((1, 1)) if mc is None else np.asarray(mc, np.float64)
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    S, z = F.block_summaries(kt, v, bidx, m)
    St, zt = F.mix_summaries(mc, S, z)
    den = np.einsum("td,td->t", qt, zt[bidx]) if normalized else np.ones(len(q))
    g = do / den[:, None]
    dqt = np.einsum("tcd,td->tc", St[bidx], g)
    dSt = np.zeros_like(St)
    for i in range(m):
        sel = bidx == i
        dSt[i] = qt[sel].T @ g[sel]
    dmc = dSt.reshape(m, -1) @ S.reshape(m, -1).T
    dS = (mc.T @ dSt.reshape(m, -1)).reshape(S.shape)
    dkt = np.einsum("jcd,jd->jc", dS[bidx], v)
    dv = np.einsum("jcd,jc->jd", dS[bidx], kt)
    return dqt * B.dphi_map(q, phi), dkt * B.dphi_map(k, phi), dv, dmc


def _mc_not_transposed(q, k, v, mc, grid, block, do, normalized=True, phi="elu1"):
    mc = None if mc is None else np.asarray(mc).T
    dq, dk, dv, dmc = _ORIG(q, k, v, mc, grid, block, do, normalized, phi)
    return dq, dk, dv, dmc.T


def _dmc_transposed(q, k, v, mc, grid, block, do, normalized=True, phi="elu1"):
    dq, dk, dv, dmc = _ORIG(q, k, v, mc, grid, block, do, normalized, phi)
    return dq, dk, dv, dmc.T


def _dphi_one(x, phi="elu1"):
    return np.ones_like(np.asarray(x, np.float64))


def _mala_du_missing(q, k, v, do, phi="elu1"):
    dq, dk, dv = _ORIG_MALA(q, k, v, do, phi)
    qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
    s = qt @ kt.sum(0)
    gamma = s / kt.shape[0]
    return dq, dk, dv + (gamma @ np.asarray(do, np.float64))[None, :]


MUTATIONS = {
    "normaliser_gradient_dropped": ("mhla_backward_blockwise", _no_gden),
    "mc_not_transposed_in_ds": ("mhla_backward_blockwise", _mc_not_transposed),
    "dmc_transposed": ("mhla_backward_blockwise", _dmc_transposed),
    "phi_derivative_dropped": ("dphi_map", _dphi_one),
    "mala_du_missing": ("mala_backward", _mala_du_missing),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(B, attr, fn)
    caught = None
    for pin in ALL_BACKWARD_PINS:
        try:
            pin(B)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught is not None, f"mutation {name} passed every backward pin"
