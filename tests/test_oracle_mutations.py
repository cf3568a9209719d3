"""Plant plausible mistakes in the oracle (CPU only) and check that the pins catch each one.

A pin set that still passes with a transposed operand, a dropped term or a wrong index
would not be pinning anything; every mutation below must make at least one pin fail.
"""
import numpy as np
import pytest

import oracle.mhla_oracle as O
from oracle_pins import ALL_PINS


def _phi_relu1(x):
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + 1.0


def _phi_elu_no_shift(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0.0, x, np.exp(np.minimum(x, 0.0)) - 1.0)


def _block_index_first_axis_fastest(grid, block):
    # tokens enumerated with the FIRST axis fastest (column-major) -- wrong raster order
    coords = np.indices(grid[::-1]).reshape(len(grid), -1)[::-1]
    bcoords = coords // np.asarray(block)[:, None]
    bgrid = [g // b for g, b in zip(grid, block)]
    return np.ravel_multi_index(tuple(bcoords), bgrid).astype(np.int64)


def _block_index_column_major_blocks(grid, block):
    coords = np.indices(grid).reshape(len(grid), -1)
    bcoords = coords // np.asarray(block)[:, None]
    bgrid = [g // b for g, b in zip(grid, block)]
    return np.ravel_multi_index(tuple(bcoords), bgrid, order="F").astype(np.int64)


def _summaries_transposed(kt, v, bidx, n_blocks):
    S, z = _ORIG["block_summaries"](kt, v, bidx, n_blocks)
    return np.transpose(S, (0, 2, 1)).copy(), z


def _summaries_global_z(kt, v, bidx, n_blocks):
    S, z = _ORIG["block_summaries"](kt, v, bidx, n_blocks)
    return S, np.tile(np.asarray(kt, np.float64).sum(0), (n_blocks, 1))


def _mix_transposed(mc, S, z):
    return _ORIG["mix_summaries"](np.asarray(mc).T, S, z)


def _mix_z_unmixed(mc, S, z):
    St, _ = _ORIG["mix_summaries"](mc, S, z)
    return St, z


def _readout_no_den(qt, St, zt, bidx, normalized=True):
    return _ORIG["readout"](qt, St, zt, bidx, False)


def _readout_wrong_block(qt, St, zt, bidx, normalized=True):
    m = St.shape[0]
    return _ORIG["readout"](qt, St, zt, (bidx + 1) % m, normalized)


def _mala_linear_no_one_in_beta(q, k, v, phi="elu1"):
    qt, kt = O.phi_map(q, phi), O.phi_map(k, phi)
    v = np.asarray(v, np.float64)
    s = qt @ kt.sum(0)
    return (1.0 / s)[:, None] * (qt @ (kt.T @ v)) - (s / kt.shape[0])[:, None] * v.sum(0)


def _mala_linear_gamma_wrong_n(q, k, v, phi="elu1"):
    qt, kt = O.phi_map(q, phi), O.phi_map(k, phi)
    v = np.asarray(v, np.float64)
    s = qt @ kt.sum(0)
    return (1 + 1.0 / s)[:, None] * (qt @ (kt.T @ v)) - (s / (kt.shape[0] - 1))[:, None] * v.sum(0)


def _mala_weights_sign(qt, kt):
    return -_ORIG["mala_weights"](qt, kt) + 2.0 / np.asarray(kt).shape[0]


def _phi_relu_leaky(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0.0, x, 0.01 * x)


def _phi_exp_base2(x):
    return np.exp2(np.asarray(x, np.float64))


_ORIG = {name: getattr(O, name) for name in
         ("block_summaries", "mix_summaries", "readout", "mala_weights", "mala_linear")}

MUTATIONS = {
    "phi_relu_plus_one": ("phi_elu1", _phi_relu1),
    "phi_without_plus_one": ("phi_elu1", _phi_elu_no_shift),
    "tokens_first_axis_fastest": ("block_index", _block_index_first_axis_fastest),
    "blocks_column_major": ("block_index", _block_index_column_major_blocks),
    "summary_transposed": ("block_summaries", _summaries_transposed),
    "normaliser_not_per_block": ("block_summaries", _summaries_global_z),
    "mc_transposed": ("mix_summaries", _mix_transposed),
    "normaliser_not_mixed": ("mix_summaries", _mix_z_unmixed),
    "readout_drops_denominator": ("readout", _readout_no_den),
    "readout_wrong_block": ("readout", _readout_wrong_block),
    "mala_beta_missing_one": ("mala_linear", _mala_linear_no_one_in_beta),
    "mala_gamma_wrong_n": ("mala_linear", _mala_linear_gamma_wrong_n),
    "mala_weights_sign": ("mala_weights", _mala_weights_sign),
    "relu_leaky": ("phi_relu", _phi_relu_leaky),
    "exp_base_two": ("phi_exp", _phi_exp_base2),
}


def _first_failing_pin():
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError) as e:  # noqa: F841
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = _first_failing_pin()
    assert caught is not None, f"no pin detects the planted mistake '{name}'"
