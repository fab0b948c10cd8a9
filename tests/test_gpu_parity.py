"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every workload is compared on every query row, the full-size ones (batch
32 x 128K paged, batch 4 x 512K paged, the 2 x 256-token chunk on 128K, the
speculative-verify and prefix-sharing batches) included, each in the launch
configuration the bench times.  Rules (ids
bit-exact except near ties, out within 2e-3 + 1e-2|ref|, block scores within
the fp32 rounding bound) are in oracle/compare.py.
"""
import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import check_row, check_rows
from block_sparse_attention_msa_amd import synth

pytestmark = pytest.mark.gpu


def _msa():
    from block_sparse_attention_msa_amd import msa  # raises if libmsa.so is missing
    return msa


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_all(w):
    """Fused path plus the unfused trio; returns host arrays."""
    msa = _msa()
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    dev = w.q.device
    out, sel = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    sel2 = torch.empty_like(sel)
    out2 = torch.empty_like(out)
    msa.msa_indexer_score(shape, cache, w.iq, bs)
    msa.msa_block_topk(shape, w.seq_lens, bs, sel2)
    msa.msa_sparse_attn_decode(shape, cache, w.q, sel2, out2, msa.alloc_workspace(shape, dev, attn_only=True))
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy(), bs.cpu().numpy(), out2.cpu().numpy(), sel2.cpu().numpy()


def check_workload(w, rows=None, label=""):
    """Runs the fused path and the unfused trio, then compares the given rows
    (default: every row) with one batched oracle call."""
    _say(f"[parity] {label or w.name}: seqs={w.num_seqs} q_len={w.q_len} mbps={w.max_blocks_per_seq} "
         f"kv={w.kv_dtype} idx={w.idx_dtype}")
    out, sel, bs, out2, sel2 = run_all(w)
    # the unfused trio runs the same kernels: identical results
    assert np.array_equal(sel, sel2)
    assert np.array_equal(out, out2)
    P = oracle.Problem.from_workload(w)
    rows = list(range(w.rows)) if rows is None else list(rows)
    ties, worst = check_rows(P, out, sel, bs, rows=rows)
    _say(f"[parity] {label or w.name}: rows={len(rows)} of {w.rows} near_ties={ties} max_abs_err={worst:.3g}")
    return out, sel, bs


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def test_tiny_bf16_config(dev):
    w = synth.make_config("tiny_b1_4k_bf16", device=dev)
    _, sel, _ = check_workload(w)
    for g in range(4):
        assert set(w.meta["planted"][(0, g)]) <= set(sel[0, g].tolist())


def test_decode_b8_32k_config(dev):
    w = synth.make_config("decode_b8_32k", device=dev)
    _, sel, _ = check_workload(w)
    for b in range(8):
        for g in range(4):
            assert set(w.meta["planted"][(b, g)]) <= set(sel[b, g].tolist())


def test_paged_b32_128k_config(dev):
    w = synth.make_config("paged_b32_128k", device=dev)
    check_workload(w)


def test_paged_b4_512k_config(dev):
    w = synth.make_config("paged_b4_512k", device=dev)
    _, sel, _ = check_workload(w)
    for b in range(4):
        for g in range(4):
            assert set(w.meta["planted"][(b, g)]) <= set(sel[b, g].tolist())


@pytest.mark.parametrize("kv,idx", [("nvfp4", "fp8"), ("bf16", "bf16"), ("nvfp4", "bf16"), ("bf16", "fp8"),
                                    ("nvfp4", "nvfp4"), ("bf16", "nvfp4")])
def test_ragged_lengths_all_dtypes(dev, kv, idx):
    """Ragged contexts: 1 token, partial blocks, exactly 16 and 17 blocks,
    a padded row, table wider than any sequence, paged layout."""
    lens = [1, 127, 128, 129, 16 * 128, 16 * 128 + 1, 0, 5000, 37 * 128 - 3, 20000]
    w = synth.make_workload(seq_lens=lens, kv_dtype=kv, idx_dtype=idx, plant=3, layout="paged", seed=21,
                            max_blocks_per_seq=200, spare_pages=7, device=dev)
    out, sel, bs = check_workload(w, label=f"ragged {kv}/{idx}")
    assert (out[6] == 0).all() and (sel[6] == -1).all() and np.isneginf(bs[6]).all()


def test_scales_not_one(dev):
    w = synth.make_workload(seq_lens=[9000, 3333], plant=2, seed=22, idx_scale=0.37, sm_scale=0.05, device=dev)
    w.k_scale *= 3.0
    w.v_scale *= 0.25
    check_workload(w, label="scales")


def test_exhaustive_format_codes(dev):
    """Every finite E4M3 index-key byte, every E2M1 nibble and every finite
    E4M3 K/V scale byte appears; checks the hardware conversions end to end."""
    w = synth.make_workload(seq_lens=[128 * 40, 128 * 23 + 77], seed=23, device=dev)
    P = w.num_pages
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8, device=dev)
    n = w.idx_k.numel()
    w.idx_k.view(-1).copy_(codes.repeat(n // codes.numel() + 1)[:n])
    # shuffle the codes per token so every dim chunk sees all of them
    perm = torch.randperm(w.idx_k.shape[1] * w.idx_k.shape[2], generator=torch.Generator().manual_seed(0))
    w.idx_k.copy_(w.idx_k.view(P, -1)[:, perm.to(dev)].view_as(w.idx_k))
    nib = torch.arange(256, dtype=torch.uint8, device=dev)          # all nibble pairs
    for t in (w.k, w.v):
        m = t.numel()
        t.view(-1).copy_(nib.repeat(m // 256 + 1)[:m])
    for t in (w.k_sf, w.v_sf):
        m = t.numel()
        t.view(-1).copy_(codes.repeat(m // codes.numel() + 1)[:m])
    w.k_scale = w.v_scale = 1.0 / (448 * 6)
    w.idx_scale = 1.0 / 64
    check_workload(w, label="exhaustive codes")


@pytest.mark.parametrize("q_len", [1, 4])
def test_exhaustive_nvfp4_index_codes(dev, q_len):
    """NVFP4 index keys: every E2M1 nibble in every position of a token row and
    every finite E4M3 group scale appear; checks the NVFP4 scans' conversions,
    nibble order and scale indexing end to end (q_len 1: the decode scan with
    per-group fp32 scaling; q_len 4: the column scan with exact dequantisation)."""
    w = synth.make_workload(seq_lens=[128 * 37, 128 * 20 + 11], q_len=q_len, idx_dtype="nvfp4", seed=26,
                            layout="paged", device=dev)
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8, device=dev)
    nib = torch.arange(256, dtype=torch.uint8, device=dev)
    m = w.idx_k.numel()
    w.idx_k.view(-1).copy_(nib.repeat(m // 256 + 1)[:m])
    perm = torch.randperm(m, generator=torch.Generator().manual_seed(3)).to(dev)
    w.idx_k.view(-1).copy_(w.idx_k.view(-1)[perm])
    m = w.idx_sf.numel()
    w.idx_sf.view(-1).copy_(codes.repeat(m // codes.numel() + 1)[:m])
    w.idx_scale = 1.0 / 512
    check_workload(w, label="exhaustive NVFP4 index codes")


def test_paged_b32_128k_nvfp4_index(dev):
    """The headline shape with NVFP4 index keys, in the bench's launch
    configuration, every row."""
    w = synth.make_config("paged_b32_128k_nvfp4_idx", device=dev)
    check_workload(w)


def test_selection_kernel_exact_on_ties(dev):
    """msa_block_topk alone: integer-valued scores full of ties and -0/+0;
    ids must equal the oracle's selection of the same fp32 values bit for bit."""
    msa = _msa()
    rng = np.random.default_rng(5)
    lens = [128 * n for n in (17, 18, 64, 300, 1024, 4096, 16384)] + [128 * 200 + 5, 0]
    S = len(lens)
    mb = 16384
    bs = rng.integers(-4, 4, size=(S, 4, mb)).astype(np.float32)
    bs[1, 0, :] = 0.0
    bs[1, 0, ::2] = -0.0
    bs[2, 1, :] = 7.0                       # all equal: lowest ids win
    bs[3, 2, :] = np.linspace(-1, 1, mb, dtype=np.float32)[::-1]
    shape = msa.MsaShape(S, 1, 16, 4, mb, 1, 1, 1, 0.1, 1.0, 1.0, 1.0)
    d_bs = torch.from_numpy(bs).to(dev)
    d_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    d_sel = torch.empty(S, 4, 16, dtype=torch.int32, device=dev)
    msa.msa_block_topk(shape, d_len, d_bs, d_sel)
    got = d_sel.cpu().numpy()
    for b, L in enumerate(lens):
        nbv = (L - 1) // 128 + 1 if L else 0
        for g in range(4):
            ref = oracle.select(bs[b, g].astype(np.float64), nbv)
            assert np.array_equal(got[b, g], ref), (b, g, got[b, g], ref)


@pytest.mark.parametrize("mb,blocks", [
    (256, (16, 64, 65, 200, 255)),                  # one wave, 1, 2 and 4 keys per lane
    (257, (16, 64, 65, 256)),                       # one wave (64 threads) past the one-wave table limit
    (1500, (100, 130, 300, 600, 1200, 1499)),       # two waves (128 threads), 1 to 16 keys per lane
    (3000, (16, 200, 257, 600, 1100, 2100, 2999)),  # four waves, 1, 2, 4, 8 and 16 keys per lane
    (8192, (300, 2100, 4097, 8191)),                # eight waves
])
def test_selection_waves_and_keys_per_lane(dev, mb, blocks):
    """msa_block_topk alone across the selection's layouts (its workgroup has
    one wave per 1,024 blocks of the table): the waves that hold the keys and
    the keys per lane follow the table width and the row length.
    Integer-valued scores (ties, -0 and +0) and a row of equal scores; ids must
    equal the oracle's selection of the same fp32 values bit for bit."""
    msa = _msa()
    rng = np.random.default_rng(mb)
    lens = [128 * n + 1 for n in blocks] + [0]
    S = len(lens)
    bs = rng.integers(-3, 3, size=(S, 4, mb)).astype(np.float32)
    bs[0, 1, ::3] = -0.0
    bs[-2, 2, :] = 1.0  # all equal: the lowest ids win
    shape = msa.MsaShape(S, 1, 16, 4, mb, 1, 1, 1, 0.1, 1.0, 1.0, 1.0)
    d_bs = torch.from_numpy(bs).to(dev)
    d_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    d_sel = torch.empty(S, 4, 16, dtype=torch.int32, device=dev)
    _say(f"[select] table {mb} blocks, rows {list(blocks)}")
    msa.msa_block_topk(shape, d_len, d_bs, d_sel)
    got = d_sel.cpu().numpy()
    for b, L in enumerate(lens):
        nbv = (L - 1) // 128 + 1 if L else 0
        for g in range(4):
            ref = oracle.select(bs[b, g].astype(np.float64), nbv)
            assert np.array_equal(got[b, g], ref), (mb, b, g, got[b, g], ref)


@pytest.mark.parametrize("mb,blocks", [(257, (17, 200, 256)), (3000, (300, 700, 1500, 2999))])
def test_fused_selection_waves(dev, mb, blocks):
    """The fused selection of the attention launch on the same layouts (a table
    just past the one-wave limit; four selection waves with 2, 4, 8 and 16 keys
    per lane), every row against the oracle and bit-equal to the unfused trio."""
    w = synth.make_workload(seq_lens=[128 * n + 5 for n in blocks], max_blocks_per_seq=mb, plant=4, zipf=1.1,
                            layout="paged", seed=mb, device=dev)
    check_workload(w, label=f"fused selection, table {mb} blocks")


def test_fused_selection_on_ties(dev):
    """All index queries zero: every block score is 0 (ties everywhere, -0 and
    +0 alike), so the fused path must keep blocks 0..14 plus the recent block
    (lower ids win ties), with the right pages, and attend over exactly those.
    Rows of 300, 2000 and 5000 blocks take the tie fallbacks of the
    selection (more candidates than one wave holds)."""
    msa = _msa()
    w = synth.make_workload(seq_lens=[128 * 300 + 7, 128 * 2000, 128 * 17, 128 * 5000 + 1], plant=0,
                            layout="paged", seed=44, device=dev)
    w.iq.zero_()
    out, sel, bs = check_workload(w, label="all index scores tied")
    for row, L in enumerate(w.seq_lens.cpu().tolist()):
        r = (L - 1) // 128
        want = list(range(15)) + [r] if r >= 16 else list(range(r + 1)) + [-1] * (15 - r)
        for g in range(4):
            assert sel[row, g].tolist() == want, (row, g, sel[row, g])


@pytest.mark.parametrize("idx", ["fp8", "nvfp4"])
def test_max_context_fused(dev, idx):
    """The largest supported row: 16,384 blocks (2M tokens) next to a short
    one, with FP8 or NVFP4 index keys.  The fused selection then runs 16
    selection waves of 16 keys per lane, which exchange their lane-bests for
    the threshold, and ranks the merged candidates; checked on every row
    against the oracle (block scores, ids, outputs)."""
    w = synth.make_workload(seq_lens=[16384 * 128 - 5, 3000], max_blocks_per_seq=16384, plant=8, zipf=1.1,
                            layout="paged", idx_dtype=idx, seed=45, device=dev)
    check_workload(w, label=f"max context 16,384 blocks, {idx} index keys")


@pytest.mark.parametrize("kv", ["nvfp4", "bf16"])
@pytest.mark.parametrize("mbps", [40, 1024, 1025, 3000, 4096, 6000, 9000])
def test_kept_block_split(dev, kv, mbps):
    """At most 64 (row, group) pairs with bf16 K/V the kept blocks are split
    over 16, 8, 4 or 2 workgroups (by the selection's waves for the row
    length: 1,024 blocks each), and a second launch merges the partials; a
    table row past 8,192 blocks, and NVFP4 K/V, keep the on-chip merge (output
    dims split over 4 workgroups).  Ragged rows, one of them padded and one
    shorter than 16 blocks (parts without keys); fused and stand-alone
    attention identical, every row against the oracle."""
    top = mbps * 128
    lens = [top - 77, 0, 5 * 128 + 3, min(top, 20000)]
    w = synth.make_workload(seq_lens=lens, kv_dtype=kv, idx_dtype="fp8", plant=4, layout="paged", seed=50 + mbps,
                            max_blocks_per_seq=mbps, zipf=1.1, device=dev)
    out, sel, _ = check_workload(w, label=f"kept-block split, {kv} K/V, {mbps} blocks per table row")
    assert (out[1] == 0).all() and (sel[1] == -1).all()


def test_long_table_batch_1024_thread_form(dev):
    """40 rows (160 (row, group) pairs: more than one per two compute units, at
    most two per unit) with block-table rows of 9,000 entries, more than the 512-thread
    attention's selection holds: the fused selection then feeds the
    1024-thread attention without an output-dims split.  NVFP4 K/V, FP8 index
    keys; every row against the oracle (block scores, ids, outputs)."""
    msa = _msa()
    lens = [1000 + (331 * i) % 6000 for i in range(40)]
    w = synth.make_workload(seq_lens=lens, max_blocks_per_seq=9000, zipf=1.1, layout="paged", seed=47, device=dev)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert cus < 2 * (w.rows * 4) and w.rows * 4 <= 2 * cus
    _say(f"[parity] long table batch: seqs={w.num_seqs} mbps={w.max_blocks_per_seq}")
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    out, sel = msa.alloc_outputs(w)
    msa.msa_decode(shape, cache, w.q, w.iq, out, sel, msa.alloc_workspace(shape, dev))
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    msa.msa_indexer_score(shape, cache, w.iq, bs)
    torch.cuda.synchronize()
    P = oracle.Problem.from_workload(w)
    check_rows(P, out.cpu().numpy(), sel.cpu().numpy(), bs.cpu().numpy())


def test_paged_permutation_invariance(dev):
    """Physical page permutation leaves ids and outputs bitwise unchanged."""
    w = synth.make_workload(seq_lens=[7000, 4100, 300], plant=3, seed=24, spare_pages=3, device=dev)
    out0, sel0, _, _, _ = run_all(w)
    perm = torch.randperm(w.num_pages, generator=torch.Generator().manual_seed(1)).to(dev)
    for name in ("idx_k", "k", "v", "k_sf", "v_sf"):
        t = getattr(w, name)
        new = torch.empty_like(t)
        new[perm] = t
        setattr(w, name, new)
    w.block_table = perm[w.block_table.long()].to(torch.int32)
    out1, sel1, _, _, _ = run_all(w)
    assert np.array_equal(sel0, sel1)
    assert np.array_equal(out0, out1)


@pytest.mark.parametrize("kv,idx", [("nvfp4", "fp8"), ("bf16", "bf16")])
@pytest.mark.parametrize("q_len", [2, 4, 5, 8, 9, 64, 80])
def test_multi_query_causal(dev, kv, idx, q_len):
    """q_len > 1 (speculative verify / prefill chunk): every query row has its
    own causal position, block scores, selection and attention; the scan runs
    on MFMA.  Ragged lengths, a sequence made only of the new tokens (its first
    query sees one key), a padded row, rows that do not fill an MFMA tile, and
    (q_len 80: 320 rows) a partial second 256-row chunk of the scan.  FP8 index
    keys with q_len <= 8 take the column scan: q_len 2 and 4 one 16-column
    tile (half and fully used), 5 and 8 two."""
    lens = [q_len, q_len + 1, 127 + q_len, 2177, 0, 16 * 128 + q_len, 5000]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, kv_dtype=kv, idx_dtype=idx, plant=3, layout="paged",
                            seed=30 + q_len, device=dev, max_blocks_per_seq=48)
    out, sel, bs = check_workload(w, label=f"multi-query q_len={q_len} {kv}/{idx}")
    pad = 4 * q_len
    assert (out[pad:pad + q_len] == 0).all() and (sel[pad:pad + q_len] == -1).all()


@pytest.mark.parametrize("q_len", [2, 4, 5, 8, 9, 64, 80])
def test_multi_query_nvfp4_index_keys(dev, q_len):
    """NVFP4 index keys with several query tokens: q_len 2-8 (speculative
    verify) take the f16 column scan; longer chunks the multi-query scan, which
    dequantises each page exactly to bf16 in LDS (its block scores held to the
    exact-product bound, with no query-rounding term).  The cases of the
    multi-query test, q_len 80 with a partial second 256-row chunk."""
    lens = [q_len, q_len + 1, 127 + q_len, 2177, 0, 16 * 128 + q_len, 5000]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, kv_dtype="nvfp4", idx_dtype="nvfp4", plant=3,
                            layout="paged", seed=60 + q_len, device=dev, max_blocks_per_seq=48)
    out, sel, bs = check_workload(w, label=f"multi-query q_len={q_len} nvfp4 index keys")
    pad = 4 * q_len
    assert (out[pad:pad + q_len] == 0).all() and (sel[pad:pad + q_len] == -1).all()


def test_multi_query_nvfp4_extreme_index_queries(dev):
    """NVFP4 index keys, q_len 4: index queries with elements 2^-30 below their
    vector's largest (rounded in the f16 score contraction, covered by the
    bound's rounding term) and queries of magnitude 1e6 (beyond f16 without
    the per-vector power-of-two scaling)."""
    w = synth.make_workload(seq_lens=[4000, 2177, 0, 16 * 128 + 4], q_len=4, kv_dtype="nvfp4", idx_dtype="nvfp4",
                            plant=3, layout="paged", seed=64, device=dev, max_blocks_per_seq=40)
    iq = w.iq.float()
    iq[0:4, :, ::7] *= 2.0 ** -30
    iq[4:8] *= 1.0e6
    w.iq.copy_(iq.to(torch.bfloat16))
    check_workload(w, label="multi-query nvfp4 index keys, extreme index queries")


def _block_major(msa, w, dev):
    """msa_decode_block_major on w (ids also written), plus msa_decode's ids
    and outputs for comparison; host arrays."""
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    out, sel = msa.alloc_outputs(w)
    ws = torch.full((msa.msa_block_major_workspace_size(shape),), 0x7F, dtype=torch.uint8, device=dev)
    msa.msa_decode_block_major(shape, cache, w.q, w.iq, out, sel, ws)
    out1, sel1 = msa.alloc_outputs(w)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1, msa.alloc_workspace(shape, dev))
    out_ns = torch.empty_like(out)
    msa.msa_decode_block_major(shape, cache, w.q, w.iq, out_ns, None, ws)  # ids kept in the workspace
    torch.cuda.synchronize()
    assert torch.equal(out, out_ns)
    return out.cpu().numpy(), sel.cpu().numpy(), out1.cpu().numpy(), sel1.cpu().numpy()


@pytest.mark.parametrize("kv_idx", ["fp8", "nvfp4"])
@pytest.mark.parametrize("q_len", [1, 2, 5, 16, 64, 200])
def test_block_major_attention(dev, q_len, kv_idx):
    """The KV-block-major attention (msa_decode_block_major: selections
    inverted into per-block row lists, each block's K/V dequantised once per
    work item of up to 16 rows, per-(row, slot) partials merged): ids equal
    msa_decode's, outputs within the tolerance of msa_decode's and of the
    oracle on every row.  Ragged lengths: a sequence made only of the new
    tokens, one shorter than 16 blocks (every block kept), a padded row, long
    rows whose blocks are chosen by many rows (shared-bias queries)."""
    msa = _msa()
    lens = [q_len, 127 + q_len, 0, 16 * 128 + q_len, 5000, 9000 + q_len]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, plant=3, zipf=1.1, layout="paged", idx_dtype=kv_idx,
                            shared_bias_iq=q_len > 1, iq_noise=0.5, seed=150 + q_len, device=dev,
                            max_blocks_per_seq=80)
    _say(f"[parity] block-major q_len={q_len} {kv_idx} index keys, rows={w.rows}")
    out, sel, out1, sel1 = _block_major(msa, w, dev)
    assert np.array_equal(sel, sel1)
    P = oracle.Problem.from_workload(w)
    ties, worst = check_rows(P, out, sel)
    np.testing.assert_allclose(out, out1, rtol=1e-2, atol=2e-3)
    pad = 2 * q_len
    assert (out[pad:pad + q_len] == 0).all() and (sel[pad:pad + q_len] == -1).all()
    _say(f"[parity] block-major q_len={q_len}: near_ties={ties} max_abs_err={worst:.3g}")


@pytest.mark.parametrize("name", ["verify_b2_q256_128k", "verify_b2_q256_128k_corr"])
def test_block_major_verify_chunk_configs(dev, name):
    """The 2 x 256-token chunk on 128K (and its variant with strongly
    correlated index queries) through the block-major attention, all 512 rows
    against the oracle; ids equal msa_decode's."""
    msa = _msa()
    w = synth.make_config(name, device=dev)
    out, sel, out1, sel1 = _block_major(msa, w, dev)
    assert np.array_equal(sel, sel1)
    P = oracle.Problem.from_workload(w)
    ties, worst = check_rows(P, out, sel)
    _say(f"[parity] block-major {name}: rows={w.rows} near_ties={ties} max_abs_err={worst:.3g}")


def test_verify_b2_q256_128k_corr_config(dev):
    """The correlated chunk through msa_decode (per-row attention), every row."""
    w = synth.make_config("verify_b2_q256_128k_corr", device=dev)
    check_workload(w)


def test_spec_b32_q4_128k_config(dev):
    """Speculative verify on the decode path: batch 32 x (128K + 4) with 4 query
    tokens each, in the bench's launch configuration, all 128 rows."""
    w = synth.make_config("spec_b32_q4_128k", device=dev)
    check_workload(w)


def test_spec_b32_q4_128k_nvfp4_index(dev):
    """The same with NVFP4 index keys (the f16 column scan), all 128 rows."""
    w = synth.make_config("spec_b32_q4_128k_nvfp4_idx", device=dev)
    check_workload(w)


def test_verify_b2_q256_128k_config(dev):
    """The multi-query verify chunk: 2 sequences x 256 new tokens on 128K,
    all 512 rows."""
    w = synth.make_config("verify_b2_q256_128k", device=dev)
    check_workload(w)


def test_verify_b2_q256_128k_nvfp4_index(dev):
    """The multi-query verify chunk with the index cache in NVFP4, all 512 rows."""
    w = synth.make_config("verify_b2_q256_128k_nvfp4_idx", device=dev)
    check_workload(w)


def test_multi_query_nvfp4_extreme_index_queries_long_chunk(dev):
    """NVFP4 index keys, q_len 12 (the multi-query scan): index queries with
    elements 2^-30 below their vector's largest and queries of magnitude 1e6;
    with keys dequantised to bf16 every product stays exact, so the exact-product
    bound holds with no rounding term."""
    w = synth.make_workload(seq_lens=[4000, 2177, 0, 16 * 128 + 12], q_len=12, kv_dtype="nvfp4", idx_dtype="nvfp4",
                            plant=3, layout="paged", seed=65, device=dev, max_blocks_per_seq=40)
    iq = w.iq.float()
    iq[0:12, :, ::7] *= 2.0 ** -30
    iq[12:24] *= 1.0e6
    w.iq.copy_(iq.to(torch.bfloat16))
    check_workload(w, label="multi-query (q_len 12) nvfp4 index keys, extreme index queries")


def test_workspace_reuse_across_calls_and_shapes(dev):
    """One workspace (uninitialised, larger than needed), consecutive decode
    calls on different data and shapes: no call sees another's scores."""
    msa = _msa()
    ws = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device=dev)
    cases = [dict(seq_lens=[9000, 4000, 129], seed=40), dict(seq_lens=[9000, 4000, 129], seed=41),
             dict(seq_lens=[3000, 0, 20000, 777, 128 * 17], seed=42), dict(seq_lens=[9000, 4000, 129], seed=40)]
    for c in cases:
        w = synth.make_workload(plant=3, layout="paged", device=dev, **c)
        shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
        out, sel = msa.alloc_outputs(w)
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
        torch.cuda.synchronize()
        P = oracle.Problem.from_workload(w)
        check_rows(P, out.cpu().numpy(), sel.cpu().numpy())


@pytest.mark.parametrize("q_len", [1, 64])
def test_decode_without_selected_ids_output(dev, q_len):
    """msa_decode with sel_blocks NULL: the same outputs as with it, both when
    the selection is fused into the attention (q_len 1: 32 (row, group)
    pairs) and when it runs as its own launch with its ids in the workspace
    (q_len 64: 2,048 pairs, more than two per compute unit)."""
    msa = _msa()
    lens = [9000, 4000 + q_len, 129 + q_len, 3000, 0, 2500, 7000, 128 * 9 + q_len]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, plant=3, layout="paged", seed=70 + q_len, device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    out, sel = msa.alloc_outputs(w)
    ws = torch.full((msa.lib().msa_workspace_size(ctypes.byref(shape)),), 0x7F, dtype=torch.uint8, device=dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
    out2 = torch.empty_like(out)
    msa.msa_decode(shape, cache, w.q, w.iq, out2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    P = oracle.Problem.from_workload(w)
    check_rows(P, out2.cpu().numpy(), sel.cpu().numpy())


@pytest.mark.parametrize("idx,share", [("fp8", None), ("fp8", (8, 12)), ("nvfp4", (5, 9))])
def test_large_decode_batch_three_launches(dev, idx, share):
    """q_len 1 with 160 sequences: 640 (row, group) pairs, more than two per
    compute unit, so msa_decode runs the selection as its own launch between
    the scan and the attention; also through the shared entry point with
    prefix sharing (FP8 and NVFP4 index keys).  Every row against the oracle."""
    msa = _msa()
    lens = [1700 + (97 * i) % 2500 for i in range(160)]
    w = synth.make_workload(seq_lens=lens, share=share, zipf=1.1, layout="paged", idx_dtype=idx, seed=95,
                            device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    assert w.rows * 4 > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out, sel = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    if share is None:
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
    else:
        msa.msa_decode_shared(shape, cache, msa.MsaPrefixShare.from_workload(w), w.q, w.iq, out, sel, ws)
    torch.cuda.synchronize()
    P = oracle.Problem.from_workload(w)
    check_rows(P, out.cpu().numpy(), sel.cpu().numpy())


@pytest.mark.parametrize("group,shared", [(8, 20), (3, 7), (2, 0)])
def test_prefix_sharing_matches_unshared(dev, group, shared):
    """Prefix sharing (groups whose first blocks map to the leader's pages):
    the shared scan's block scores, the selection and the outputs equal the
    unshared calls' bit for bit (each MFMA column is computed alone), and
    every row matches the oracle.  Ragged lengths, a last group shorter than
    the others, and shared = 0 (groups that share nothing)."""
    msa = _msa()
    lens = [2600, 9000, 4000, 2561, 7000, 3333, 5000, 2700, 6000, 2900, 4400]
    w = synth.make_workload(seq_lens=lens, share=(group, shared), zipf=1.1, layout="paged", seed=80 + group,
                            device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w)
    bs1 = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    bs2 = torch.full_like(bs1, float("nan"))
    msa.msa_indexer_score(shape, cache, w.iq, bs1)
    msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs2)
    out1, sel1 = msa.alloc_outputs(w)
    out2, sel2 = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1, ws)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out2, sel2, ws)
    torch.cuda.synchronize()
    assert torch.equal(bs1, bs2)
    assert torch.equal(sel1, sel2) and torch.equal(out1, out2)
    P = oracle.Problem.from_workload(w)
    check_rows(P, out2.cpu().numpy(), sel2.cpu().numpy(), bs2.cpu().numpy())


def _shared_vs_unshared(msa, w, dev, bit_equal):
    """Runs the shared and the unshared index scan and decode on w; with
    bit_equal (FP8 keys) every block score, id and output must be identical,
    otherwise (NVFP4 keys) the sequences' own blocks must be; every row is
    checked against the oracle (block scores, ids, outputs)."""
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w)
    bs1 = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    bs2 = torch.full_like(bs1, float("nan"))
    msa.msa_indexer_score(shape, cache, w.iq, bs1)
    msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs2)
    out1, sel1 = msa.alloc_outputs(w)
    out2, sel2 = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1, ws)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out2, sel2, ws)
    torch.cuda.synchronize()
    if bit_equal:
        assert torch.equal(bs1, bs2)
        assert torch.equal(sel1, sel2) and torch.equal(out1, out2)
    else:
        for b, own in enumerate(w.seq_shared_blocks.cpu().tolist()):
            rows = slice(b * w.q_len, (b + 1) * w.q_len)
            assert torch.equal(bs1[rows, :, own:], bs2[rows, :, own:]), b
    P = oracle.Problem.from_workload(w)
    ties, worst = check_rows(P, out2.cpu().numpy(), sel2.cpu().numpy(), bs2.cpu().numpy())
    _say(f"[parity] shared vs unshared: rows={w.rows} near_ties={ties} max_abs_err={worst:.3g}")


@pytest.mark.parametrize("idx", ["fp8", "nvfp4"])
def test_prefix_sharing_64_members(dev, idx):
    """A sharing group of 64 decode requests (256 (member, group) columns: 16
    MFMA column tiles over the 8 waves that score each converted page) plus a
    group of 4 in the same launch: FP8 keys bit-equal to the
    unshared calls, NVFP4 keys their own blocks bit-equal; every row against
    the oracle.  Ragged lengths, all longer than the 20-block shared prefix."""
    msa = _msa()
    lens = [2600 + (397 * i) % 5000 for i in range(64)] + [3000, 2700, 4100, 2561]
    w = synth.make_workload(seq_lens=lens[:64], share=(64, 20), zipf=1.1, layout="paged", idx_dtype=idx,
                            seed=130, device=dev)
    assert w.share_members.shape == (1, 64) and (w.share_members >= 0).all()
    _say(f"[parity] 64-member sharing group, {idx} index keys")
    _shared_vs_unshared(msa, w, dev, bit_equal=idx == "fp8")
    # groups of 64 and 4 in one launch
    w2 = synth.make_workload(seq_lens=lens, share=(64, 20), zipf=1.1, layout="paged", idx_dtype=idx, seed=131,
                             device=dev)
    _say(f"[parity] groups of 64 and 4, {idx} index keys")
    _shared_vs_unshared(msa, w2, dev, bit_equal=idx == "fp8")


@pytest.mark.parametrize("idx", ["fp8", "nvfp4"])
@pytest.mark.parametrize("q_len,group", [(2, 32), (4, 16), (4, 3), (8, 8), (5, 2)])
def test_prefix_sharing_multi_query(dev, idx, q_len, group):
    """Prefix sharing with q_len 2..8 query tokens per request (speculative
    verify): groups of up to 64 / q_len members, (member, query, group)
    columns 4 x q_len per member; each query row keeps its own causal
    position.  FP8 keys bit-equal to the unshared calls; NVFP4 keys their own
    blocks bit-equal; every row against the oracle."""
    msa = _msa()
    n = group + 3
    lens = [q_len + 2600 + (331 * i) % 4000 for i in range(n)]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, share=(group, 18), zipf=1.1, layout="paged",
                            idx_dtype=idx, seed=140 + q_len + group, device=dev)
    _say(f"[parity] sharing q_len={q_len} groups of {group}, {idx} index keys")
    _shared_vs_unshared(msa, w, dev, bit_equal=idx == "fp8")


@pytest.mark.parametrize("group,shared", [(8, 20), (3, 7)])
def test_prefix_sharing_nvfp4_index_keys(dev, group, shared):
    """Prefix sharing with NVFP4 index keys: the shared pages are dequantised
    exactly to bf16 once per group (a summation order other than the unshared
    scan's), so every row is checked against the oracle (block scores within
    the exact-product bound, ids, outputs), and the sequences' own blocks,
    scored by the unshared scan's code, equal the unshared call's bit for bit."""
    msa = _msa()
    lens = [2600, 9000, 4000, 2561, 7000, 3333, 5000, 2700, 6000, 2900, 4400]
    w = synth.make_workload(seq_lens=lens, share=(group, shared), zipf=1.1, layout="paged", idx_dtype="nvfp4",
                            seed=90 + group, device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w)
    bs1 = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    bs2 = torch.full_like(bs1, float("nan"))
    msa.msa_indexer_score(shape, cache, w.iq, bs1)
    msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs2)
    out2, sel2 = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out2, sel2, ws)
    torch.cuda.synchronize()
    # blocks at or past a sequence's shared count come from the unshared code
    # (a leader's shared blocks, like its members', from the group rows)
    for b, own in enumerate(w.seq_shared_blocks.cpu().tolist()):
        assert torch.equal(bs1[b, :, own:], bs2[b, :, own:]), b
    P = oracle.Problem.from_workload(w)
    check_rows(P, out2.cpu().numpy(), sel2.cpu().numpy(), bs2.cpu().numpy())


def test_shared_b32_128k_nvfp4_index(dev):
    """Batch 32 x 128K in groups of 8 sharing a 96K prefix with NVFP4 index
    keys, through the shared path in the bench's launch configuration; every
    row checked against the oracle."""
    msa = _msa()
    w = synth.make_config("shared_b32_128k_nvfp4_idx", device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w)
    out, sel = msa.alloc_outputs(w)
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out, sel, ws)
    msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs)
    torch.cuda.synchronize()
    P = oracle.Problem.from_workload(w)
    check_rows(P, out.cpu().numpy(), sel.cpu().numpy(), bs.cpu().numpy())


def test_prefix_sharing_general_descriptors(dev):
    """Sharing descriptors the generator never makes: members out of index
    order with the leader last in id, a one-member group, a member whose whole
    context is the shared prefix (seq_len = shared_blocks x 128), sequences in
    no group, a padded row.  The members' block-table rows are pointed at the
    leader's pages for the shared blocks, then the shared and the unshared
    calls must agree bit for bit, and every row matches the oracle."""
    msa = _msa()
    lens = [3000, 5000, 0, 4200, 12 * 128, 6100, 2300]
    w = synth.make_workload(seq_lens=lens, zipf=1.1, layout="paged", seed=88, device=dev)
    groups = [([5, 1, 4, 3], 12), ([6], 9)]   # (members, leader first; shared blocks)
    bt = w.block_table.clone()
    members = torch.full((len(groups), msa.MSA_SHARE_MAX), -1, dtype=torch.int32)
    shared = torch.zeros(len(groups), dtype=torch.int32)
    per_seq = torch.zeros(len(lens), dtype=torch.int32)
    for gi, (mem, sb) in enumerate(groups):
        assert all(sb * 128 <= lens[b] for b in mem)
        members[gi, :len(mem)] = torch.tensor(mem, dtype=torch.int32)
        shared[gi] = sb
        for b in mem:
            bt[b, :sb] = bt[mem[0], :sb]
            per_seq[b] = sb
    w.block_table = bt
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_tensors(members=members.to(dev), shared_blocks=shared.to(dev),
                                            seq_shared_blocks=per_seq.to(dev))
    bs1 = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    bs2 = torch.full_like(bs1, float("nan"))
    msa.msa_indexer_score(shape, cache, w.iq, bs1)
    msa.msa_indexer_score_shared(shape, cache, share, w.iq, bs2)
    out1, sel1 = msa.alloc_outputs(w)
    out2, sel2 = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1, ws)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out2, sel2, ws)
    torch.cuda.synchronize()
    assert torch.equal(bs1, bs2)
    assert torch.equal(sel1, sel2) and torch.equal(out1, out2)
    P = oracle.Problem.from_workload(w)
    check_rows(P, out2.cpu().numpy(), sel2.cpu().numpy(), bs2.cpu().numpy())


def test_shared_b32_128k_config(dev):
    """Batch 32 x 128K in groups of 8 sharing a 96K prefix, through the shared
    path in the bench's launch configuration: bit-equal to the unshared path
    and every row checked against the oracle."""
    msa = _msa()
    w = synth.make_config("shared_b32_128k", device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w)
    out1, sel1 = msa.alloc_outputs(w)
    out2, sel2 = msa.alloc_outputs(w)
    ws = msa.alloc_workspace(shape, dev)
    msa.msa_decode(shape, cache, w.q, w.iq, out1, sel1, ws)
    msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out2, sel2, ws)
    torch.cuda.synchronize()
    assert torch.equal(sel1, sel2) and torch.equal(out1, out2)
    P = oracle.Problem.from_workload(w)
    check_rows(P, out2.cpu().numpy(), sel2.cpu().numpy())


@pytest.mark.parametrize("case", ["plain", "plain_bf16_split", "shared_fp8", "shared_nvfp4_wide", "multi_query",
                                  "block_major"])
def test_graph_capture_replays(dev, case):
    """msa_decode (or msa_decode_shared) captured in a HIP graph: every replay
    (with eager work and synchronisation in between) equals the eager result
    bit for bit.  plain_bf16_split: bf16 K/V and few (row, group) pairs, so
    the kept blocks are split over workgroups whose partials the last one
    merges; the arrival counters are zeroed by the captured scan, with no
    memset in the graph.  multi_query: 192 rows of 64 query tokens, more
    (row, group) pairs than two per compute unit, so the step is three launches
    (scan, selection, attention); block_major: msa_decode_block_major on the
    same shape (inversion, block-major partials, merge)."""
    msa = _msa()
    if case == "plain":
        w = synth.make_workload(seq_lens=[12000, 5000, 300, 0], plant=3, layout="paged", seed=43, device=dev)
    elif case == "plain_bf16_split":
        w = synth.make_workload(seq_lens=[12000, 5000, 300, 0], plant=3, layout="paged", kv_dtype="bf16",
                                idx_dtype="bf16", seed=45, device=dev)
    elif case in ("multi_query", "block_major"):
        w = synth.make_workload(seq_lens=[20000, 9000, 4000], q_len=64, plant=3, layout="paged", seed=47,
                                shared_bias_iq=True, device=dev)
        assert w.rows * 4 > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    else:
        n = 8 if case == "shared_fp8" else 16
        w = synth.make_workload(seq_lens=[9000 + 97 * i for i in range(n)], plant=3, layout="paged", seed=44,
                                idx_dtype="fp8" if case == "shared_fp8" else "nvfp4", share=(n, 40), device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    share = msa.MsaPrefixShare.from_workload(w) if case.startswith("shared") else None
    out, sel = msa.alloc_outputs(w)
    if case == "block_major":
        ws = torch.empty(msa.msa_block_major_workspace_size(shape), dtype=torch.uint8, device=dev)
    else:
        ws = msa.alloc_workspace(shape, dev)

    def call(stream=None):
        if case == "block_major":
            msa.msa_decode_block_major(shape, cache, w.q, w.iq, out, sel, ws, stream=stream)
        elif share is None:
            msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws, stream=stream)
        else:
            msa.msa_decode_shared(shape, cache, share, w.q, w.iq, out, sel, ws, stream=stream)

    call()
    torch.cuda.synchronize()
    ref_out, ref_sel = out.clone(), sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), rep
        assert torch.equal(sel, ref_sel), rep
        call()  # eager call between replays
        torch.cuda.synchronize()


def test_concurrent_streams(dev):
    """Two steps in flight at once on two streams (default priority), each with
    its own workspace: a batch-4 decode with NVFP4 K/V (two launches), a bf16
    batch whose kept blocks are split and merged through arrival counters, and
    a 64-token chunk (three launches).  The library holds no device state of
    its own on this path, so every result equals the eager, one-at-a-time
    result bit for bit."""
    msa = _msa()
    ws_ = [
        synth.make_workload(seq_lens=[12000, 5000, 300, 0], plant=3, layout="paged", seed=50, device=dev),
        synth.make_workload(seq_lens=[9000, 700], plant=2, layout="paged", kv_dtype="bf16", idx_dtype="bf16",
                            seed=51, device=dev),
        synth.make_workload(seq_lens=[20000, 9000, 4000], q_len=64, plant=3, layout="paged", seed=52,
                            device=dev),
    ]
    runs = []
    for w in ws_:
        shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
        out, sel = msa.alloc_outputs(w)
        ws = msa.alloc_workspace(shape, dev)
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
        torch.cuda.synchronize()
        runs.append((w, shape, cache, out, sel, ws, out.clone(), sel.clone()))
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        for (w, shape, cache, out, sel, ws, _, _) in runs:
            out.fill_(float("nan"))
            sel.fill_(-7)
        torch.cuda.synchronize()
        for s, (w, shape, cache, out, sel, ws, _, _) in zip(streams, runs):
            s.wait_stream(torch.cuda.current_stream())
            msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws, stream=s)
        torch.cuda.synchronize()
        for (w, shape, cache, out, sel, ws, ref_out, ref_sel) in runs:
            assert torch.equal(out, ref_out), (w.name, rep)
            assert torch.equal(sel, ref_sel), (w.name, rep)


def test_split_merge_from_any_workspace(dev):
    """bf16 K/V with few (row, group) pairs: msa_decode's kept-block split
    merges each pair's partials in the workgroup that finishes last, counting
    arrivals on counters in the workspace that the step's scan zeroes.  A
    workspace left full of nonzero bytes (stale counters included) gives the
    same bits as a zeroed one and as the stand-alone attention, whose second
    launch merges the same partials; every row matches the oracle."""
    msa = _msa()
    w = synth.make_workload(seq_lens=[3000, 40000, 129, 0, 1000], plant=3, layout="paged", kv_dtype="bf16",
                            idx_dtype="fp8", seed=46, device=dev)
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    results = []
    for fill in (0, 0x7F, 0xFF, 0x01):
        out, sel = msa.alloc_outputs(w)
        ws = msa.alloc_workspace(shape, dev)
        ws.fill_(fill)
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)
        msa.msa_decode(shape, cache, w.q, w.iq, out, sel, ws)  # counters left by a first call
        torch.cuda.synchronize()
        results.append((out.clone(), sel.clone()))
    for out, sel in results[1:]:
        assert torch.equal(out, results[0][0]) and torch.equal(sel, results[0][1])
    out2 = torch.full_like(results[0][0], float("nan"))
    aws = torch.empty(msa.msa_attn_workspace_size(shape), dtype=torch.uint8, device=dev)
    msa.msa_sparse_attn_decode(shape, cache, w.q, results[0][1], out2, aws)
    torch.cuda.synchronize()
    assert torch.equal(out2, results[0][0])
    P = oracle.Problem.from_workload(w)
    check_rows(P, results[0][0].cpu().numpy(), results[0][1].cpu().numpy())


def test_deterministic(dev):
    w = synth.make_workload(seq_lens=[30000, 12000, 640], plant=4, seed=25, device=dev)
    a = run_all(w)
    b = run_all(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("kv,idx,q_len,scales", [("nvfp4", "fp8", 1, None), ("nvfp4", "nvfp4", 1, None),
                                                 ("bf16", "bf16", 1, None), ("nvfp4", "bf16", 3, None),
                                                 ("nvfp4", "fp8", 3, None), ("bf16", "fp8", 3, None),
                                                 ("nvfp4", "nvfp4", 12, None),
                                                 ("bf16", "bf16", 1, (0.37, 1.7, 0.61)),
                                                 ("bf16", "bf16", 3, (3.0, 0.1, 1.3))])
def test_kv_insert_matches_oracle(dev, kv, idx, q_len, scales):
    """msa_kv_insert writes exactly the oracle's bytes (every pool, bit for
    bit: the quantiser's integer decisions are taken in the same fp32 steps),
    touches nothing else, and the decode over the updated cache matches the
    oracle.  New tokens mix magnitudes from 1e-3 to 30, an all-zero group, a
    group of tiny values, E4M3 ties (x = midpoints) in the index keys and
    negative values that round to zero; a padded sequence writes nothing.
    With `scales` (k, v, idx tensor scales that are neither 1 nor powers of
    two) the bf16 pools store x / scale, which must round (to nearest even)."""
    msa = _msa()
    lens = [300, 0, 128 * 3, 5000 + q_len]
    w = synth.make_workload(seq_lens=lens, q_len=q_len, kv_dtype=kv, idx_dtype=idx, plant=2, layout="paged",
                            seed=50 + q_len, spare_pages=3, device=dev)
    if scales is not None:
        w.k_scale, w.v_scale, w.idx_scale = scales
    P = oracle.Problem.from_workload(w)
    g = torch.Generator(device="cpu").manual_seed(7)
    rows = w.rows
    mag = torch.exp(torch.empty(rows, 1, 1).uniform_(math.log(1e-3), math.log(30.0), generator=g))
    k_new = (torch.randn(rows, 4, 128, generator=g) * mag).to(torch.bfloat16)
    v_new = (torch.randn(rows, 4, 128, generator=g) * mag).to(torch.bfloat16)
    x_new = torch.randn(rows, 128, generator=g).to(torch.bfloat16)
    k_new[0, 0, :16] = 0.0                                    # zero group
    v_new[0, 1, 16:32] = 1e-30                                # tiny group
    k_new[0, 2, 32:48] = torch.tensor([6.0] + [-5.0] * 15)    # saturating codes after scale rounding
    x_new[0, :8] = torch.tensor([1.0625, -1.0625, 0.5625, 3.25, -0.0001, 2.0 ** -10, 1.5 * 2 ** -8, 448.0])
    if x_new.shape[0] > 1:
        x_new[-1, :4] = torch.tensor([1000.0, -1000.0, 0.0, -0.0])   # clamped to +-448 in FP8
    if scales is not None:  # the quotients x / scale (fp32) are not all bf16 values: the stores round
        for x, sc in ((k_new, scales[0]), (v_new, scales[1]), (x_new, scales[2])):
            y = x.float() / torch.tensor(sc, dtype=torch.float32)
            assert (y.to(torch.bfloat16).float() != y).sum() > 100
    before = {k: getattr(w, k).clone() for k in ("k", "v", "k_sf", "v_sf", "idx_k", "idx_sf") if getattr(w, k) is not None}
    shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
    msa.msa_kv_insert(shape, cache, k_new.to(dev), v_new.to(dev), x_new.to(dev))
    torch.cuda.synchronize()
    P.kv_insert(_bits(k_new), _bits(v_new), _bits(x_new))
    h = w.host_arrays()
    changed = 0
    for name in before:
        got, want = h[name], P.arrays[name]
        assert np.array_equal(got, want), f"{name}: {np.count_nonzero(got != want)} bytes differ"
        old = before[name]
        old = _bits(old) if old.dtype == torch.bfloat16 else old.cpu().numpy()
        changed += int(np.count_nonzero(got != old))
    assert changed > 0
    check_workload(w, label=f"decode after insert {kv}/{idx} q_len={q_len}")


@pytest.mark.parametrize("kv,idx", [("nvfp4", "fp8"), ("bf16", "bf16"), ("nvfp4", "nvfp4")])
def test_multi_step_decode_with_inserts(dev, kv, idx):
    """Decode steps as a serving loop runs them: each step appends one token
    per sequence (its row of the block table gets a fresh page when the token
    opens a new block), inserts the token's K/V/index key with msa_kv_insert,
    draws new queries and decodes over the grown cache.  After every insert
    the pools equal the oracle's bytes; every decode matches the oracle on
    every row.  Lengths start just below, on and past page boundaries; one
    row is padded and stays so."""
    msa = _msa()
    lens = [127, 0, 128 * 5 - 2, 1000, 128 * 2]
    steps = 4
    w = synth.make_workload(seq_lens=lens, kv_dtype=kv, idx_dtype=idx, plant=2, layout="paged", seed=61,
                            spare_pages=8, max_blocks_per_seq=max((L + steps - 1) // 128 + 1 for L in lens),
                            device=dev)
    bt0, L0 = w.block_table.cpu(), w.seq_lens.cpu().tolist()
    used = {int(bt0[b, j]) for b, n in enumerate(L0) for j in range((n + 127) // 128)}
    spare = sorted(set(range(w.num_pages)) - used)
    assert len(spare) == 8
    g = torch.Generator(device="cpu").manual_seed(17)
    for step in range(steps):
        L = w.seq_lens.cpu().tolist()
        bt = w.block_table.cpu()
        for b, n in enumerate(L):
            if n == 0:
                continue
            if n % 128 == 0:  # the new token opens block n / 128
                bt[b, n // 128] = spare.pop(0)
            L[b] = n + 1
        w.block_table.copy_(bt.to(dev))
        w.seq_lens.copy_(torch.tensor(L, dtype=torch.int32).to(dev))
        w.q.copy_(torch.randn(w.q.shape, generator=g).to(torch.bfloat16).to(dev))
        w.iq.copy_(torch.randn(w.iq.shape, generator=g).to(torch.bfloat16).to(dev))
        k_new = torch.randn(w.rows, 4, 128, generator=g).to(torch.bfloat16)
        v_new = torch.randn(w.rows, 4, 128, generator=g).to(torch.bfloat16)
        x_new = torch.randn(w.rows, 128, generator=g).to(torch.bfloat16)
        P = oracle.Problem.from_workload(w)  # the grown metadata, the pools before the insert
        shape, cache = msa.MsaShape.from_workload(w), msa.MsaCache.from_workload(w)
        msa.msa_kv_insert(shape, cache, k_new.to(dev), v_new.to(dev), x_new.to(dev))
        torch.cuda.synchronize()
        P.kv_insert(_bits(k_new), _bits(v_new), _bits(x_new))
        h = w.host_arrays()
        for name in ("k", "v", "k_sf", "v_sf", "idx_k", "idx_sf"):
            if h.get(name) is not None:
                assert np.array_equal(h[name], P.arrays[name]), f"step {step}: {name} differs after the insert"
        check_workload(w, label=f"decode step {step} {kv}/{idx}")

