"""CPU checks of the parity rules' f16 query-rounding term (oracle/compare.py)."""
import numpy as np
import torch

from oracle.compare import f16_query_rounding


def test_no_rounding_for_ordinary_queries():
    g = torch.Generator().manual_seed(0)
    iq = torch.randn(4, 128, generator=g, dtype=torch.float64).to(torch.bfloat16).to(torch.float64)
    assert (f16_query_rounding(iq) == 0).all()


def test_scaled_vectors_keep_every_element_within_range():
    # largest 3 -> scale 2^13; 2^-20 -> 2^-7 exact; 2^-40 -> 2^-27 is an f16
    # subnormal (counted whole); a 1.5 x 2^20 vector scales down instead of
    # overflowing (bf16 inputs: 8 significant bits, exact in f16 once in range)
    x = torch.zeros(3, 128, dtype=torch.float64)
    x[0, :3] = torch.tensor([3.0, 2.0 ** -20, -(2.0 ** -40)])
    x[1, :2] = torch.tensor([1.5 * 2.0 ** 20, 3.0])
    x[2] = 0.0
    r = f16_query_rounding(x).numpy()
    assert r[0, 0] == 0 and r[0, 1] == 0 and r[0, 2] == 2.0 ** -40
    assert r[1, 0] == 0 and r[1, 1] == 0 and np.isfinite(r).all()
    assert (r[2] == 0).all()


# ---- the selection rule at a near tie ------------------------------------

import pytest

import oracle
from oracle.compare import check_row, check_rows
from block_sparse_attention_msa_amd import synth


def _all_tied_problem():
    """One row of 21 blocks whose index keys are all the same value, so every
    block scores the same non-zero value: the 15th and 16th best non-recent
    blocks tie exactly and the near-tie branch of the rule applies."""
    w = synth.make_workload(seq_lens=[128 * 20 + 5], plant=0, seed=3)
    w.idx_k.fill_(0x38)                            # E4M3 1.0 in every dim of every key
    P = oracle.Problem.from_workload(w)
    bs, sel, out = P.decode()
    assert abs(bs[0, 0, 0]) > 0 and (bs[0, 0, :20] == bs[0, 0, 0]).all()
    return P, bs, sel, out


def _fake_gpu(P, sel, g, ids):
    """A GPU result that holds `ids` for group g, with the outputs the oracle
    gives for exactly that set (so only the id rule can fail)."""
    s = sel[0].copy()
    s[g] = np.asarray(ids, dtype=np.int32)
    o = P.decode()[2][0].copy()
    hpg = o.shape[0] // s.shape[0]
    o[g * hpg:(g + 1) * hpg] = P.attend(0, g, s[g])
    return o.astype(np.float32), s


def test_near_tie_accepts_a_valid_swap():
    P, bs, sel, out = _all_tied_problem()
    assert sel[0, 1].tolist() == list(range(15)) + [20]
    o, s = _fake_gpu(P, sel, 1, list(range(1, 16)) + [20])     # block 0 out, block 15 in
    info = check_row(P, 0, o, s)
    assert info["near_ties"] == 1


@pytest.mark.parametrize("ids", [
    list(range(14)) + [20, -1],                    # 15 ids and a padding slot
    [0, 0] + list(range(2, 15)) + [20],            # a duplicate id
    list(range(16)),                               # the recent block (20) dropped for a tied block
    [1, 0] + list(range(2, 15)) + [20],            # out of order
    list(range(15)) + [21],                        # a block past the visible ones
    [-1] + list(range(1, 15)) + [20],              # padding in front
])
def test_near_tie_rejects_invalid_selections(ids):
    """A selection that breaks what every selection must be fails even where
    the scores tie, although the outputs match the oracle re-run on it."""
    P, bs, sel, out = _all_tied_problem()
    o, s = _fake_gpu(P, sel, 2, ids)
    with pytest.raises(AssertionError):
        check_row(P, 0, o, s)


def test_difference_without_near_tie_fails():
    """A swap where the scores are far apart is not a near tie."""
    w = synth.make_workload(seq_lens=[128 * 40], plant=3, seed=4)
    P = oracle.Problem.from_workload(w)
    bs, sel, out = P.decode()
    ids = sel[0, 0].tolist()
    order = np.lexsort((np.arange(39), -bs[0, 0, :39]))
    assert abs(bs[0, 0, order[14]] - bs[0, 0, order[15]]) > 1e-3 * abs(bs[0, 0, order[14]])
    swapped = sorted([j for j in ids if j != order[14]] + [int(order[15])])
    o, s = _fake_gpu(P, sel, 0, swapped)
    with pytest.raises(AssertionError):
        check_row(P, 0, o, s)


def test_check_rows_batched_equals_single_rows():
    """The batched form (one oracle call, bounds per sequence) accepts the
    oracle's own results on every row, block scores included, and rejects a
    block score moved past its bound."""
    w = synth.make_workload(seq_lens=[3000, 0, 129, 128 * 17 + 3], q_len=3, plant=2, seed=5, layout="paged")
    P = oracle.Problem.from_workload(w)
    bs, sel, out = P.decode()
    gbs = bs.astype(np.float32)
    ties, worst = check_rows(P, out.astype(np.float32), sel, gbs)
    assert ties == 0 and worst < 1e-6
    bad = gbs.copy()
    bad[1, 1, 2] += abs(bad[1, 1, 2]) * 1e-3 + 1e-3       # row 1: sequence 0, block 2 visible
    with pytest.raises(AssertionError):
        check_rows(P, out.astype(np.float32), sel, bad)
