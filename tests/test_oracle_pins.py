"""The fp64 oracle against hand-worked values, closed forms, textbook special cases,
invariants and rank bounds (CPU only)."""
import math

import numpy as np
import pytest

import oracle.mhla_oracle as O
import synth
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


def test_mc_softmax_l1_closed_form():
    # 2x2 block grid: L1 distances from block 0 are (0, 1, 1, 2) -> (1, e^-1, e^-1, e^-2) / (1 + e^-1)^2
    mc = synth.mc_softmax_l1((2, 2))
    e = math.exp(-1.0)
    want0 = np.array([1, e, e, e * e]) / (1 + e) ** 2
    np.testing.assert_allclose(mc[0], want0, rtol=1e-14)
    np.testing.assert_allclose(mc[0], [0.534447, 0.196612, 0.196612, 0.072329], atol=5e-7)
    np.testing.assert_allclose(mc.sum(1), 1.0, rtol=1e-14)
    # symmetric geometry: row 3 is row 0 reversed
    np.testing.assert_allclose(mc[3], want0[::-1], rtol=1e-14)


def test_mc_locality_init_closed_form():
    # MHLA Key design 3: row i ~ 1 - dist(i,j)/max_k dist(i,k), Euclidean; 2x2 grid: distances
    # (0, 1, 1, sqrt 2) -> (1, 1 - 1/sqrt2, 1 - 1/sqrt2, 0) / (3 - sqrt 2)
    mc = synth.mc_locality_init((2, 2))
    r = 1 - 1 / math.sqrt(2)
    want0 = np.array([1, r, r, 0]) / (3 - math.sqrt(2))
    np.testing.assert_allclose(mc[0], want0, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(mc[0], [0.630602, 0.184699, 0.184699, 0.0], atol=5e-7)
    np.testing.assert_allclose(synth.mc_locality_init((1,)), [[1.0]])
    # 1D, 3 blocks: row 1 distances (1, 0, 1) -> (0, 1, 0)
    np.testing.assert_allclose(synth.mc_locality_init((3,))[1], [0, 1, 0], atol=1e-300)


def test_mc_generators_rows_and_clip():
    rng = np.random.default_rng(0)
    noisy = synth.mc_softmax_l1_noisy_clipped((4, 4), rng)
    assert noisy.min() >= 0 and noisy.max() <= 1 and np.all(noisy.max(axis=1) > 0)
    g = synth.mc_softmax_gaussian(256, np.random.default_rng(1))
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-12)
    assert g.min() > 0


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-3], np.float32)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> ties to even -> 1.0;
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> even -> 1 + 2^-6
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5], np.float32)
    np.testing.assert_array_equal(synth.round_to_bf16(x)[:5], want)
    assert abs(synth.round_to_bf16(x)[5] - 3.0e-3) <= 3.0e-3 * 2**-8


def test_workload_shapes():
    w = synth.WORKLOADS
    assert (w["tiny"].n_tokens, w["tiny"].n_blocks, w["tiny"].block_tokens) == (64, 4, 16)
    assert (w["deit_t"].n_tokens, w["deit_t"].n_blocks, w["deit_t"].block_tokens) == (196, 4, 49)
    assert (w["image"].n_tokens, w["image"].n_blocks) == (4096, 16)
    assert (w["image_mala"].n_blocks, w["image_mala"].block_tokens) == (1, 4096)
    assert (w["video3d"].n_tokens, w["video3d"].n_blocks, w["video3d"].block_tokens) == (16384, 64, 256)
    assert (w["long1d"].n_tokens, w["long1d"].n_blocks) == (65536, 256)


def test_block_index_raster():
    # 3D: token (a, r, c) in a 4x4x4 grid with 2x2x2 blocks -> block (a//2, r//2, c//2), raster
    bidx = O.block_index((4, 4, 4), (2, 2, 2))
    for a in range(4):
        for r in range(4):
            for c in range(4):
                assert bidx[(a * 4 + r) * 4 + c] == ((a // 2) * 2 + r // 2) * 2 + c // 2
    with pytest.raises(ValueError):
        O.block_index((10,), (3,))


def test_sampled_plain_matches_blockwise_on_workload_shapes():
    """On real workload shapes (one head each), the plain definition at sampled queries equals
    the blockwise oracle."""
    for name in ("deit_t", "image", "image_mala", "video3d"):
        w = synth.WORKLOADS[name]
        rng = np.random.default_rng(100)
        shape = (1, 1, w.n_tokens, w.head_dim)
        q, k, v = (synth.round_to_bf16(rng.standard_normal(shape, dtype=np.float32)) for _ in range(3))
        mc = synth.make_mc(w, rng)
        full = O.forward(q, k, v, mc, w.grid, w.block, mode=w.readout)
        toks = sorted(set(rng.integers(0, w.n_tokens, 12).tolist()) | {0, w.n_tokens - 1})
        samp = O.forward_sampled(q, k, v, mc, w.grid, w.block, [(0, 0, toks)], mode=w.readout)[0]
        np.testing.assert_allclose(full[0, 0, toks], samp, rtol=1e-9, atol=1e-9 * np.abs(full).max())
