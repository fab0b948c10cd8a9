"""GPU parity on seeded random cases: batch size, ragged and padded lengths,
q_len, K/V and index-key dtypes, layout, score structure and prefix sharing
drawn from seeded generators, every case through the fused step (the
shared entry point when the case shares a prefix), the stand-alone index scan
and, without sharing, the unfused trio; rows against the fp64 oracle (every
row, or 66 sampled rows of a case with more than 96).  The second generator
reaches the larger shapes: chunks of 17-300 query tokens, decode batches of
100-200 short rows (more (row, group) pairs than two per compute unit) and
contexts up to 300K tokens.  A third generator draws prefix-sharing batches
(1-8 query tokens, groups of up to 64 / q_len requests, so both the narrow and
the wide shared pass).  Every case that the KV-block-major attention takes
(NVFP4 K/V, at most 256 query tokens, no sharing) also runs through it: the
same ids as the fused step, its rows against the oracle."""
import random
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_row
from block_sparse_attention_msa_amd import synth

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    """The i-th case's make_workload arguments (deterministic)."""
    rng = random.Random(1000 + i)
    q_len = rng.choice([1, 1, 1, 1, 2, 3, 4, 5, 8, 9, 16, 33])
    kv = rng.choice(["nvfp4", "nvfp4", "bf16"])
    idx = rng.choice(["fp8", "fp8", "nvfp4", "bf16"])
    S = rng.randint(1, 10)
    lens = [0 if rng.random() < 0.1 else rng.randint(q_len, 20000) for _ in range(S)]
    if all(L == 0 for L in lens):
        lens[0] = rng.randint(q_len, 5000)
    kw = dict(seq_lens=lens, q_len=q_len, kv_dtype=kv, idx_dtype=idx, layout=rng.choice(["paged", "identity"]),
              seed=2000 + i, spare_pages=rng.randint(0, 3))
    kw["max_blocks_per_seq"] = max(1, max((L + 127) // 128 for L in lens)) + rng.randint(0, 5)
    r = rng.random()
    if r < 0.4:
        kw["zipf"] = 1.1
    elif r < 0.7:
        kw["plant"] = rng.randint(1, 6)
    if q_len > 1 and rng.random() < 0.5:
        kw["shared_bias_iq"] = True
    if q_len == 1 and idx in ("fp8", "nvfp4") and S >= 2 and rng.random() < 0.8:
        # sharing sequences are not padded rows, and every member sees the prefix
        lens[:] = [rng.randint(1500, 20000) for _ in range(S)]
        kw["share"] = (rng.randint(2, min(8, S)), rng.randint(0, min(lens) // 128))
        kw["layout"] = "paged"
        kw["max_blocks_per_seq"] = max((L + 127) // 128 for L in lens) + rng.randint(0, 5)
    return kw


def _wide_case(i):
    """The i-th case of the wider generator (deterministic)."""
    rng = random.Random(50000 + i)
    kv = rng.choice(["nvfp4", "nvfp4", "bf16"])
    idx = rng.choice(["fp8", "fp8", "nvfp4", "bf16"])
    kind = rng.random()
    if kind < 0.3:  # a long multi-query chunk
        q_len = rng.choice([17, 33, 64, 100, 128, 256, 300])
        S = rng.randint(1, 3)
        cap = max(q_len, min(60000, 10_000_000 // (q_len * S)))
        lens = [rng.randint(q_len, cap) for _ in range(S)]
    elif kind < 0.55:  # a large batch of short rows
        q_len = rng.choice([1, 1, 2, 4])
        S = rng.randint(100, 200)
        lens = [0 if rng.random() < 0.05 else rng.randint(q_len, 4000) for _ in range(S)]
    elif kind < 0.75:  # long contexts
        q_len = rng.choice([1, 1, 2, 4, 8])
        S = rng.randint(1, 4)
        lens = [rng.randint(q_len, 300_000) for _ in range(S)]
    else:
        q_len = rng.choice([1, 2, 3, 5, 8, 9, 16])
        S = rng.randint(1, 12)
        lens = [0 if rng.random() < 0.1 else rng.randint(q_len, 30000) for _ in range(S)]
    if all(L == 0 for L in lens):
        lens[0] = rng.randint(q_len, 5000)
    kw = dict(seq_lens=lens, q_len=q_len, kv_dtype=kv, idx_dtype=idx, layout=rng.choice(["paged", "identity"]),
              seed=60000 + i, spare_pages=rng.randint(0, 3))
    r = rng.random()
    if r < 0.4:
        kw["zipf"] = 1.1
    elif r < 0.7:
        kw["plant"] = rng.randint(1, 6)
    if q_len > 1 and rng.random() < 0.5:
        kw["shared_bias_iq"] = True
    if q_len == 1 and idx in ("fp8", "nvfp4") and S >= 2 and rng.random() < 0.5:
        hi = 4000 if S > 20 else 40000
        lens[:] = [rng.randint(1500, hi) for _ in range(S)]
        kw["share"] = (rng.randint(2, min(8, S)), rng.randint(0, min(lens) // 128))
        kw["layout"] = "paged"
    kw["max_blocks_per_seq"] = max(1, max((L + 127) // 128 for L in lens)) + rng.randint(0, 5)
    return kw


# two to four of each kind: long chunks, long contexts, large batches with and
# without sharing, mixed small cases with and without sharing; then cases that
# give every attention launch form (output dims split in 4 or 2, 512- or
# 1024-thread workgroups, selection fused or its own launch) with both K/V
# dtypes
WIDE_CASES = [0, 7, 8, 9, 2, 4, 5, 10, 21, 22, 28, 18, 38, 61, 67, 88, 1, 3, 35, 12, 37, 23, 13]


def _share_case(i):
    """The i-th prefix-sharing case (deterministic): consecutive sequences in
    groups of gsize share their first blocks."""
    rng = random.Random(90000 + i)
    q_len = rng.choice([1, 1, 2, 3, 4, 5, 8])
    gsize = rng.randint(2, 64 // q_len)
    S = gsize * rng.randint(1, 2) + rng.randint(0, 1)   # maybe one sequence in no group
    S = min(S, 64)
    lens = [rng.randint(max(q_len, 1500), 8000) for _ in range(S)]
    kw = dict(seq_lens=lens, q_len=q_len, kv_dtype=rng.choice(["nvfp4", "nvfp4", "bf16"]),
              idx_dtype=rng.choice(["fp8", "nvfp4"]), layout="paged", seed=91000 + i,
              share=(gsize, rng.randint(0, (min(lens) - q_len + 1) // 128)))
    kw["max_blocks_per_seq"] = max((L + 127) // 128 for L in lens) + rng.randint(0, 5)
    if rng.random() < 0.5:
        kw["zipf"] = 1.1
    if q_len > 1 and rng.random() < 0.5:
        kw["shared_bias_iq"] = True
    return kw


SHARE_CASES = range(16)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def _run_case(dev, kw, label):
    from block_sparse_attention_msa_amd import msa  # raises if libmsa.so is missing
    print(f"[random] {label}: {kw}", file=sys.stderr, flush=True)
    w = synth.make_workload(device=dev, **kw)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    out, sel = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    if w.share_members is not None:
        share = msa.MsaPrefixShare.from_workload(w)
        msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out, sel, ws)
        msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs)
    else:
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
        msa.msa_indexer_score(shape, cache, w.iq, bs)
        sel2 = torch.empty_like(sel)
        out2 = torch.empty_like(out)
        msa.msa_block_topk(shape, w.seq_lens, bs, sel2)
        msa.msa_sparse_attn_decode(shape, cache, w.q, sel2, out2, msa.alloc_workspace(shape, dev, attn_only=True))
        torch.cuda.synchronize()
        assert torch.equal(sel, sel2) and torch.equal(out, out2)
    torch.cuda.synchronize()
    P = oracle.Problem.from_workload(w)
    o, s_, b_ = out.cpu().numpy(), sel.cpu().numpy(), bs.cpu().numpy()
    assert np.isfinite(o).all()
    rows = list(range(w.rows))
    if w.rows > 96:
        rows = sorted(set(random.Random(w.rows).sample(rows, 64) + [0, w.rows - 1]))
    for row in rows:
        check_row(P, row, o[row], s_[row], b_[row])
    if w.share_members is None and w.kv_dtype == "nvfp4" and w.q_len <= 256 and w.max_blocks_per_seq <= 8192:
        wsb = torch.empty(msa.msa_block_major_workspace_size(shape), dtype=torch.uint8, device=dev)
        out_b, sel_b = msa.alloc_outputs(w)
        msa.msa_decode_block_major(shape, cache, w.q, w.iq, out_b, sel_b, wsb)
        torch.cuda.synchronize()
        assert torch.equal(sel_b, sel)
        ob = out_b.cpu().numpy()
        assert np.isfinite(ob).all()
        for row in rows:
            check_row(P, row, ob[row], s_[row], b_[row])


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(dev, i):
    _run_case(dev, _case(i), f"case {i}")


@pytest.mark.parametrize("i", WIDE_CASES)
def test_random_wide_case(dev, i):
    _run_case(dev, _wide_case(i), f"wide case {i}")


@pytest.mark.parametrize("i", SHARE_CASES)
def test_random_share_case(dev, i):
    _run_case(dev, _share_case(i), f"share case {i}")
