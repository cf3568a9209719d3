"""Operand precisions of the forward kernels, decided by emulating their bf16 roundings on the CPU
(tests/precision_emulation.py) against fp64.  Inputs are seeded N(0, 1) rounded to bf16, as the
workloads draw them."""
import math

import numpy as np
import pytest

import synth
from precision_emulation import backward_key_side, bf, causal_1d, causal_rel, mala, mhla_1d, rel, split

BAR = 2e-2


@pytest.fixture(scope="module")
def mhla_case():
    # a long-sequence head: 16384 tokens, 256 blocks of 64, d = 64, a dense row-softmax M_c
    rng = np.random.default_rng(1234)
    n, d, n_b = 16384, 64, 64
    q, k, v = (synth.round_to_bf16(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float64)
               for _ in range(3))
    mc = synth.mc_softmax_gaussian(n // n_b, rng).astype(np.float32).astype(np.float64)
    ref = mhla_1d(q, k, v, mc, n_b)
    return q, k, v, mc, n_b, ref


def test_mc_rounding_dominates_the_bf16_path(mhla_case):
    """Rounding M_c to one bf16 costs more than any other single rounding of the bf16 path (the
    mixing averages summaries of both signs, so a relative error of up to 2^-8 in every weight does not
    average away): the mixing kernel takes M_c as bf16 hi + lo."""
    q, k, v, mc, n_b, ref = mhla_case
    single = {name: rel(mhla_1d(q, k, v, mc, n_b, **{name: True}), ref)
              for name in ("phi_k", "stack", "mc_r", "mixed", "phi_q")}
    print(single)
    others = max(e for name, e in single.items() if name != "mc_r")
    assert single["mc_r"] > 2.0 * others, single
    every = rel(mhla_1d(q, k, v, mc, n_b, phi_k=True, stack=True, mc_r=True, mixed=True, phi_q=True), ref)
    split_mc = rel(mhla_1d(q, k, v, mc, n_b, phi_k=True, stack=True, mixed=True, phi_q=True), ref)
    print(f"all roundings {every:.3e}, with M_c split {split_mc:.3e}")
    assert split_mc < 0.6 * every
    assert every < BAR and split_mc < BAR


def test_bf16_output_rounding_floor(mhla_case):
    """The bf16 output's own rounding, relative to RMS(o), on this head: what is left of the
    2e-2 bar for the kernel is 2e-2 minus this floor (up to 2^-8 * max|o| / RMS(o))."""
    q, k, v, mc, n_b, ref = mhla_case
    floor = rel(synth.round_to_bf16(ref.astype(np.float32)).astype(np.float64), ref)
    peak = float(np.max(np.abs(ref)) / np.sqrt(np.mean(ref ** 2)))
    assert floor <= 2.0 ** -8 * peak
    assert floor >= 2.0 ** -10 * peak
    split_mc = mhla_1d(q, k, v, mc, n_b, phi_k=True, stack=True, mixed=True, phi_q=True)
    both = rel(synth.round_to_bf16(split_mc.astype(np.float32)).astype(np.float64), ref)
    print(f"floor {floor:.3e}, kernel roundings + bf16 output {both:.3e}")
    assert both < BAR


@pytest.fixture(scope="module")
def mala_case():
    rng = np.random.default_rng(4321)
    n, d = 4096, 64
    q, k, v = (synth.round_to_bf16(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float64)
               for _ in range(3))
    return q, k, v, mala(q, k, v)


def test_mala_needs_the_centred_form_and_split_operands(mala_case):
    """The MALA readout: evaluated as the page's linear form with a bf16 S, the subtraction of
    gamma u cancels about ten-fold and the error fails the bar; the centred form C = S - z u^T/N
    with single bf16 operands still sits near the bar; split phi(K), phi(Q) and C (the kernels'
    MALA path) bring it far below."""
    q, k, v, ref = mala_case
    naive = rel(mala(q, k, v, naive=True, rounding=bf), ref)
    centred = rel(mala(q, k, v, rounding=bf), ref)
    both = rel(mala(q, k, v, rounding=split), ref)
    print(f"naive {naive:.3e}, centred single bf16 {centred:.3e}, centred split {both:.3e}")
    assert naive > BAR
    assert centred > 0.5 * BAR
    assert both < BAR / 50


def test_mala_centred_identity_is_exact(mala_case):
    """Y = u/N + beta q~^T C equals beta q~^T S - gamma u without rounding (the identity the
    kernels rely on)."""
    q, k, v, ref = mala_case
    pk = np.where(k > 0, k + 1.0, np.exp(np.minimum(k, 0.0)))
    pq = np.where(q > 0, q + 1.0, np.exp(np.minimum(q, 0.0)))
    s, z, u = pk.T @ v, pk.sum(0), v.sum(0)
    sq = pq @ z
    direct = (1.0 + 1.0 / sq)[:, None] * (pq @ s) - (sq / len(q))[:, None] * u[None, :]
    assert math.isclose(rel(direct, ref), 0.0, abs_tol=1e-12)


@pytest.fixture(scope="module")
def causal_case():
    # one head of 1024 tokens in 4 blocks of 256, d = 64, a row-softmax M_c (the c_m4 GPU case's shape)
    rng = np.random.default_rng(201)
    n, d, n_b = 1024, 64, 256
    q, k, v = (synth.round_to_bf16(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float64)
               for _ in range(3))
    mc = synth.mc_softmax_gaussian(n // n_b, rng).astype(np.float32).astype(np.float64)
    return q, k, v, mc, n_b, causal_1d(q, k, v, mc, n_b)


def test_causal_scores_stay_split(causal_case):
    """The bf16-input causal slice kernel: single bf16 phi(q) and m_ii phi(K) keep the causal
    readout well inside its 2e-2 bar; rounding P (the weights of V) to one bf16 does not -- the
    weighted sums of V cancel, so the weights' error of up to 2^-8 grows with the keys in view -- and P
    therefore stays split (hi + lo)."""
    q, k, v, mc, n_b, ref = causal_case
    kernel = causal_rel(causal_1d(q, k, v, mc, n_b, q_single=True, k_single=True, p_mode="split", stack=True), ref)
    p_single = causal_rel(causal_1d(q, k, v, mc, n_b, p_mode="bf"), ref)
    all_single = causal_rel(causal_1d(q, k, v, mc, n_b, q_single=True, k_single=True, p_mode="bf", stack=True), ref)
    print(f"kernel roundings {kernel:.3e}, P single alone {p_single:.3e}, all single {all_single:.3e}")
    assert kernel < BAR / 2
    assert p_single > BAR and all_single > BAR


@pytest.mark.parametrize("phi", ["elu1", "exp"])
def test_backward_key_side_needs_split_operands(phi):
    """dK = (dS v + dz) phi'(k): the two terms nearly cancel (the gradient of a normalised average
    sums to about zero over the keys), so a single bf16 dS fails the backward's bar under the exp
    map and takes most of it under ELU+1; split operands (the kernels' choice for every backward
    product) leave it far below."""
    rng = np.random.default_rng(77)
    n, d, n_b = 4096, 128, 256
    q, k, v, do = (synth.round_to_bf16(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float64)
                   for _ in range(4))
    mc = synth.mc_softmax_gaussian(n // n_b, rng).astype(np.float32).astype(np.float64)
    dk, dv = backward_key_side(q, k, v, mc, do, n_b, phi)
    dk1, dv1 = backward_key_side(q, k, v, mc, do, n_b, phi, ds_single=True, phik_single=True)
    e_dk, e_dv = rel(dk1, dk), rel(dv1, dv)
    dk2, dv2 = backward_key_side(q, k, v, mc, do, n_b, phi, ds_single=False)
    print(f"{phi}: single dS -> dK {e_dk:.3e}, single dS and phi(K) -> dV {e_dv:.3e}")
    assert rel(dk2, dk) == 0.0
    if phi == "exp":
        assert e_dk > BAR
    else:
        assert e_dk > BAR / 4
    assert e_dv < e_dk
