"""The allocation-free entry point msa_decode_noalloc (the library's static
device scratch as the workspace) against msa_decode with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller batch, and a
large batch with no selected-ids output (the selection then runs as its own
launch and keeps its ids in the scratch).  Outputs and ids must be equal bit
for bit: the same kernels run on the same inputs."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_rows
from block_sparse_attention_msa_amd import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _both(msa, w, want_sel=True):
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    out1, sel1 = msa.alloc_outputs(w)
    ws = torch.full((msa.msa_workspace_size(shape),), 0x7F, dtype=torch.uint8, device=w.q.device)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1 if want_sel else None, ws)
    out2, sel2 = msa.alloc_outputs(w)
    out2.fill_(float("nan"))
    sel2.fill_(-7)
    msa.msa_decode_noalloc(shape, cache, w.q, w.iq, out2, sel2 if want_sel else None)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    if want_sel:
        assert torch.equal(sel1, sel2)
    return out2, sel1


def test_noalloc_matches_decode_two_calls_second_smaller():
    from block_sparse_attention_msa_amd import msa
    dev = torch.device("cuda:0")
    big = synth.make_workload(seq_lens=[9000 + 331 * i for i in range(24)] + [0, 129], zipf=1.1, layout="paged",
                              seed=120, device=dev)
    small = synth.make_workload(seq_lens=[3000, 128 * 17, 5], plant=3, layout="paged", seed=121, device=dev)
    for label, w in (("first call, 26 rows", big), ("second call, 3 rows", small)):
        _say(f"[noalloc] {label}")
        out, sel = _both(msa, w)
        P = oracle.Problem.from_workload(w)
        check_rows(P, out.cpu().numpy(), sel.cpu().numpy())


def test_noalloc_bf16_split_counters_in_scratch():
    """bf16 K/V with few (row, group) pairs: the kept blocks are split over
    workgroups whose arrival counters sit in the static scratch after the
    partials.  The scratch keeps the previous call's bytes (counters left at
    their final counts included); each call's scan zeroes them, so two calls
    in a row, the second smaller, both match msa_decode bit for bit."""
    from block_sparse_attention_msa_amd import msa
    dev = torch.device("cuda:0")
    a = synth.make_workload(seq_lens=[5000, 128 * 9, 0, 700, 20000], plant=3, layout="paged", kv_dtype="bf16",
                            idx_dtype="bf16", seed=123, device=dev)
    b = synth.make_workload(seq_lens=[3000, 129], plant=2, layout="paged", kv_dtype="bf16", idx_dtype="fp8",
                            seed=124, device=dev)
    for label, w in (("bf16 split, 5 rows", a), ("bf16 split, 2 rows", b)):
        _say(f"[noalloc] {label}")
        out, sel = _both(msa, w)
        P = oracle.Problem.from_workload(w)
        check_rows(P, out.cpu().numpy(), sel.cpu().numpy())


def test_noalloc_selection_launch_ids_in_scratch():
    """160 decode rows: more (row, group) pairs than two per compute unit, so
    the selection runs as its own launch; with no sel_blocks output its ids
    live in the scratch after the block scores."""
    from block_sparse_attention_msa_amd import msa
    dev = torch.device("cuda:0")
    w = synth.make_workload(seq_lens=[1700 + (97 * i) % 2500 for i in range(160)], zipf=1.1, layout="paged",
                            seed=122, device=dev)
    assert w.rows * 4 > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    _say("[noalloc] 160 rows, no ids output")
    _both(msa, w, want_sel=False)
    _both(msa, w, want_sel=True)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the static scratch is refused before
    any launch, with the sizes in the message."""
    from block_sparse_attention_msa_amd import msa
    shape = msa.MsaShape(1024, 1, 16, 4, 16384, 16, msa.MSA_KV_NVFP4, msa.MSA_IDX_FP8_E4M3, 0.088, 1.0, 1.0, 1.0)
    assert msa.msa_workspace_size(shape) > msa.MSA_NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    cache = msa.MsaCache(*([fake] * 8))
    st = msa.lib().msa_decode_noalloc(ctypes.byref(shape), ctypes.byref(cache), fake, fake, fake, fake, None)
    assert st == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in msa.last_error()
