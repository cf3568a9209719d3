"""GPU parity of the forward's intermediate steps, through mhla_forward_intermediates: the block
summaries S_b, z_b (step 3, "MHLA: Restoring Expressivity of Linear Attention via Token-Level
Multi-Head", Overall framework) and the mixed summaries S~_i, z~_i (Key design 2; for the causal
readouts the strictly lower part of M_c) against the oracle's block_summaries and mix_summaries, so
that an error in one step is seen there and not only through the readout.

Bar: an elementwise rounding bound, computed in fp64 from the oracle's inputs, so that a sum
whose terms cancel is judged against the size of its terms rather than of its result.  eps_op is
the relative rounding of an operand: 2^-8 (bf16's unit roundoff) for one bf16 operand, on the
plans with single bf16 operands; 2^-16 for hi + lo pairs (split accuracy, fp32 inputs, ReLU, exp,
MALA).  eps_st, that of the stored stack, is taken equal to eps_op, the coarsest storage a plan
of that class uses:
  |dS|  <= 2 (eps_op B + eps_st |S| + n 2^-24 B),   B = sum_j |phi(k_j)| |v_j|^T over the block
  |dz|  <= 2 (eps_op + n 2^-24) z                    (phi >= 0: z is its own absolute sum)
  |dS~| <= 2 (|M_c| bound_S + (eps_mc + M 2^-24) |M_c| |S| + eps_st |S~|),   eps_mc = 2^-16
  |dz~| <= 2 (|M_c| bound_z + (eps_mc + M 2^-24) |M_c| z)
(n the tokens of a block, M the blocks; the factor 2 covers the accumulation order of the matrix
cores).  max|dx| / RMS(x) is printed and recorded beside it.
"""
import numpy as np
import pytest

import oracle
import synth
import token_blocked_linear_amd as T
from gpu_util import announce, oracle_geometry, record, to_device

pytestmark = pytest.mark.gpu

EPS_SINGLE = 2.0 ** -8
EPS_SPLIT = 2.0 ** -16
EPS_MC = 2.0 ** -16
EPS_ACC = 2.0 ** -24


def rel(got, want):
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want))) / rms


def oracle_stacks(w, k, v, mc, eps):
    """(values, bounds): S, z, S~, z~ per (batch, head) from the oracle's step functions,
    [B*H, M, ...], and the elementwise rounding bounds of the module docstring."""
    grid, block = oracle_geometry(w)
    bidx = oracle.block_index(grid, block)
    m = int(bidx.max()) + 1
    n = int(np.bincount(bidx).max())
    vals, bnds = [[], [], [], []], [[], [], [], []]
    for b in range(w.batch):
        for h in range(w.heads):
            kt = oracle.phi_map(np.asarray(k[b, h], np.float64), w.phi)
            vv = np.asarray(v[b, h], np.float64)
            S, z = oracle.block_summaries(kt, vv, bidx, m)
            B, _ = oracle.block_summaries(np.abs(kt), np.abs(vv), bidx, m)   # sum |phi(k)| |v|^T
            bS = 2 * (eps * B + eps * np.abs(S) + n * EPS_ACC * B)
            bz = 2 * (eps + n * EPS_ACC) * np.abs(z)
            for lst, x in zip((vals[0], vals[1], bnds[0], bnds[1]), (S, z, bS, bz)):
                lst.append(x)
            if mc is not None:
                mh = np.asarray(mc[h] if np.ndim(mc) == 3 else mc, np.float64)
                if w.readout.startswith("causal"):
                    mh = np.tril(mh, -1)          # query block i reads the blocks b < i
                St, zt = oracle.mix_summaries(mh, S, z)
                am = np.abs(mh)
                prop_S, absS = oracle.mix_summaries(am, bS, bz)[0], oracle.mix_summaries(am, np.abs(S), np.abs(z))
                prop_z = oracle.mix_summaries(am, bS, bz)[1]
                bSt = 2 * (prop_S + (EPS_MC + m * EPS_ACC) * absS[0] + eps * np.abs(St))
                bzt = 2 * (prop_z + (EPS_MC + m * EPS_ACC) * absS[1])
                for lst, x in zip((vals[2], vals[3], bnds[2], bnds[3]), (St, zt, bSt, bzt)):
                    lst.append(x)
    keep = 4 if mc is not None else 2
    return [np.stack(x) for x in vals[:keep]], [np.stack(x) for x in bnds[:keep]]


def check(name, got, want, bound):
    """(fraction of the bound used, max|d| / RMS) for each tensor; asserts the bound."""
    out = {}
    for nm, g, x, bd in zip(("S", "z", "St", "zt"), got, want, bound):
        assert np.all(np.isfinite(g)), (name, nm)
        d = np.abs(np.asarray(g, np.float64) - x)
        frac = float(np.max(d / np.maximum(bd, 1e-300)))
        out[nm] = (frac, rel(g, x))
    print("  " + " ".join(f"{nm}: {f:.2f} of bound, {r:.2e} of RMS" for nm, (f, r) in out.items()))
    record("intermediates", name, **{f"{nm}_bound_frac": f for nm, (f, r) in out.items()},
           **{f"{nm}_rel_rms": r for nm, (f, r) in out.items()})
    for nm, (f, r) in out.items():
        assert f <= 1.0, (name, nm, f, r)


def run_intermediates(w, k, v, mc, *, accuracy="auto", mixed=True):
    import torch
    plan = T.Plan(grid=w.grid, block=w.block, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                  in_dtype=w.dtype, out_dtype="fp32", readout=w.readout, accuracy=accuracy, phi=w.phi,
                  mc_per_head=mc is not None and np.ndim(mc) == 3, ragged=w.ragged, cls_token=w.cls)
    tk, tv = to_device(k, w.dtype), to_device(v, w.dtype)
    tmc = None if mc is None else torch.from_numpy(np.ascontiguousarray(mc, np.float32)).to("cuda:0")
    ws = plan.alloc_workspace()
    res = plan.intermediates(tk, tv, tmc, ws, mixed=mixed)
    torch.cuda.synchronize()
    info = plan.info
    plan.close()
    return [t.cpu().numpy().astype(np.float64) for t in res], info


# (workload, accuracy): one case per summary and mixing path
CASES = [
    # one token slice per block, bf16 operands: bf16 stack, MFMA mixing of the bf16 stack
    (synth.Workload("i_m64_bf16", "bf16", 1, 2, 64, (4096,), (64,), 101, "softmax_l1"), "auto"),
    (synth.Workload("i_m200_d128", "bf16", 1, 2, 128, (3200,), (16,), 102, "softmax_gauss"), "auto"),
    (synth.Workload("i_m144_2d_d32", "bf16", 2, 1, 32, (48, 48), (4, 4), 103, "locality"), "auto"),
    # split accuracy: fp32 partials, split MFMA mixing
    (synth.Workload("i_m64_split", "bf16", 1, 2, 64, (4096,), (64,), 104, "softmax_l1"), "split"),
    # fp32 inputs
    (synth.Workload("i_fp32_m40", "fp32", 2, 1, 64, (40, 32), (4, 8), 105, "softmax_l1"), "auto"),
    # blocks over 256 tokens with few units: several token slices per block (fp32 partials)
    (synth.Workload("i_slices_m20", "bf16", 1, 1, 128, (20 * 512,), (512,), 106, "softmax_l1"), "auto"),
    # M > 256: the VALU mixing
    (synth.Workload("i_m300_valu", "bf16", 1, 1, 32, (300 * 16,), (16,), 107, "softmax_l1"), "auto"),
    (synth.Workload("i_m300_valu_split", "bf16", 1, 1, 32, (300 * 16,), (16,), 113, "softmax_l1"), "split"),
    # ReLU and exp maps
    (synth.Workload("i_relu", "bf16", 1, 2, 64, (2048,), (64,), 108, "softmax_l1", phi="relu"), "auto"),
    (synth.Workload("i_exp", "bf16", 1, 1, 32, (2048,), (32,), 109, "softmax_l1", phi="exp"), "auto"),
    # ragged 2D blocks with a CLS token
    (synth.Workload("i_ragged_cls", "bf16", 1, 2, 64, (30, 34), (4, 4), 110, "softmax_gauss", ragged=True, cls=True),
     "auto"),
    # causal: the strictly lower M_c; several slices per block
    (synth.Workload("i_causal", "bf16", 1, 2, 64, (4096,), (128,), 111, "softmax_l1", readout="causal"), "auto"),
    (synth.Workload("i_causal_slices", "bf16", 1, 1, 64, (24 * 640,), (640,), 112, "softmax_l1", readout="causal"),
     "auto"),
]


def _eps(info):
    return EPS_SPLIT if info.split_operands else EPS_SINGLE


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_intermediates_match_oracle(case):
    w, accuracy = case
    announce(f"intermediates {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} {w.readout} {accuracy}")
    q, k, v, mc, _ = synth.make_inputs(w)
    got, info = run_intermediates(w, k, v, mc, accuracy=accuracy)
    print(f"  n_kernels={info.n_kernels} splits={info.summary_splits} split_operands={info.split_operands}")
    want, bound = oracle_stacks(w, k, v, mc, _eps(info))
    check(w.name, got, want, bound)


def test_intermediates_per_head_mc():
    w = synth.Workload("i_per_head", "bf16", 2, 3, 64, (64, 64), (8, 16), 114, "none")
    announce(w.name)
    q, k, v, _, rng = synth.make_inputs(w)
    m = w.n_blocks
    mc = rng.uniform(0.0, 1.0, (w.heads, m, m)).astype(np.float32).astype(np.float64)
    got, info = run_intermediates(w, k, v, mc)
    want, bound = oracle_stacks(w, k, v, mc, _eps(info))
    check(w.name, got, want, bound)


def test_intermediates_long_sequence_full_size():
    """The long-sequence workload at its full size and in the plan the benchmark times (B = 1,
    16 heads, d = 128, 65536 tokens in 256 blocks): the stacks of heads 0, 7 and 15 against the
    oracle, every element."""
    w = synth.WORKLOADS["long1d"]
    announce(f"intermediates long1d shape={w.qkv_shape}")
    q, k, v, mc, _ = synth.make_inputs(w)
    got, info = run_intermediates(w, k, v, mc)
    assert info.n_kernels == 3 and info.n_blocks == 256
    heads = (0, 7, 15)
    sub = w.with_(name="long1d_heads", heads=len(heads))
    kk, vv = k[:, list(heads)], v[:, list(heads)]
    want, bound = oracle_stacks(sub, kk, vv, mc, _eps(info))
    check("long1d", [g[list(heads)] for g in got], want, bound)


@pytest.mark.parametrize("w", [
    synth.Workload("i_fused_m16", "bf16", 2, 2, 64, (32, 32), (8, 8), 120, "softmax_l1"),
    synth.Workload("i_mala", "bf16", 1, 2, 64, (700,), (700,), 121, "none", "mala"),
    synth.Workload("i_d16", "bf16", 3, 2, 16, (20, 20), (10, 4), 122, "locality"),
], ids=lambda w: w.name)
def test_summaries_of_plans_that_mix_in_the_readout(w):
    """Plans that mix inside the readout (at most 16 blocks; MALA) keep no mixed stack: their
    summaries are checked, and asking for the mixed stack is an unsupported request."""
    announce(f"summaries {w.name} shape={w.qkv_shape} grid={w.grid} block={w.block} {w.readout}")
    q, k, v, mc, _ = synth.make_inputs(w)
    (S, z), info = run_intermediates(w, k, v, mc, mixed=False)
    assert info.n_kernels == 2
    want, bound = oracle_stacks(w, k, v, mc, _eps(info))
    check(w.name, (S, z), want[:2], bound[:2])
    with pytest.raises(T.MhlaError):
        run_intermediates(w, k, v, mc, mixed=True)
