"""GPU parity on seeded random cases: batch size, ragged and padded lengths,
q_len, K/V and index-key dtypes, layout, score structure and prefix sharing
drawn from one seeded generator, every case through the fused step (the
shared entry point when the case shares a prefix), the stand-alone index scan
and, without sharing, the unfused trio; every row against the fp64 oracle."""
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


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(dev, i):
    from block_sparse_attention_msa_amd import msa  # raises if libmsa.so is missing
    kw = _case(i)
    print(f"[random] case {i}: {kw}", file=sys.stderr, flush=True)
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
    for row in range(w.rows):
        check_row(P, row, o[row], s_[row], b_[row])
