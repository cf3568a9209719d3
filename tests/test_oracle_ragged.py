"""Ragged blocks and the CLS token in the forward oracle: pins, and planted mistakes that the pins
must catch (CPU only)."""
import types

import numpy as np
import pytest

import oracle.mhla_oracle as F
from oracle_ragged_pins import ALL_RAGGED_PINS


@pytest.mark.parametrize("pin", ALL_RAGGED_PINS, ids=lambda p: p.__name__)
def test_ragged_pin(pin):
    pin(F)


def _variant(block_index):
    """The forward oracle with block_index replaced; every function that reads it sees the new one."""
    ns = {n: getattr(F, n) for n in dir(F) if not n.startswith("__")}
    m = types.SimpleNamespace(**ns)
    m.block_index = block_index

    def blockwise(q, k, v, mc, grid, block, normalized=True, phi="elu1"):
        bidx = block_index(grid, block)
        nb = int(bidx.max()) + 1
        qt, kt = F.phi_map(q, phi), F.phi_map(k, phi)
        S, z = F.block_summaries(kt, v, bidx, nb)
        St, zt = F.mix_summaries(mc, S, z)
        return F.readout(qt, St, zt, bidx, normalized)
    m.mhla_blockwise = blockwise
    return m


def _floor_block_grid(grid, block):
    """Blocks numbered over the rounded-down block grid (edge blocks collide with others)."""
    if not isinstance(grid, F.RaggedGrid):
        return F.block_index(grid, block)
    g, b = grid.grid, grid.block
    coords = np.indices(g).reshape(len(g), -1)
    bc = coords // np.asarray(b)[:, None]
    bgrid = [max(x // y, 1) for x, y in zip(g, b)]
    bc = np.minimum(bc, np.asarray(bgrid)[:, None] - 1)
    idx = np.ravel_multi_index(tuple(bc), bgrid).astype(np.int64)
    return np.concatenate([[0], idx + 1]) if grid.cls else idx


def _cls_last(grid, block):
    if not isinstance(grid, F.RaggedGrid) or not grid.cls:
        return F.block_index(grid, block)
    idx = F.block_index(F.RaggedGrid(grid.grid, grid.block, False), None)
    return np.concatenate([[idx.max() + 1], idx])


def _cls_in_first_block(grid, block):
    if not isinstance(grid, F.RaggedGrid) or not grid.cls:
        return F.block_index(grid, block)
    idx = F.block_index(F.RaggedGrid(grid.grid, grid.block, False), None)
    return np.concatenate([[0], idx])


MUTANTS = {"floor_block_grid": _floor_block_grid, "cls_numbered_last": _cls_last,
           "cls_inside_first_block": _cls_in_first_block}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_ragged_mistake_is_caught(name):
    mutant = _variant(MUTANTS[name])
    caught = []
    for pin in ALL_RAGGED_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
