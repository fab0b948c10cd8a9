"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of the oracle to a library routine, a published table,
a closed form, brute force or an invariant the pages state, chosen so that a
plausible slip (wrong bias, dropped term, swapped nibble, wrong tie order,
unmasked tail, off-by-one recent block) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_msa_amd import synth
from _ref import BYTE_MODEL, E2M1_TABLE, bf16_t, dense_seq, e4m3_t, make_problem, nvfp4_t, row_queries


# ---- formats -------------------------------------------------------------

def test_e4m3_all_codes_match_torch_cast():
    """P-a: all 256 OCP E4M3 codes against torch.float8_e4m3fn -> float64."""
    ref = e4m3_t(np.arange(256, dtype=np.uint8)).numpy()
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_e2m1_codes_match_ocp_table():
    """P-b: the 16 E2M1 codes against the OCP MX table (eight magnitudes)."""
    got = np.array([oracle.e2m1(n) for n in range(16)])
    assert np.array_equal(got, E2M1_TABLE.numpy())
    assert len(set(np.abs(got).tolist())) == 8


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=5000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ref = bf16_t(bits).numpy()
    got = np.array([oracle.bf16(int(b)) for b in bits])
    assert np.array_equal(got, ref)


def test_nvfp4_products_exact_and_lut_size():
    """P-c: every E2M1 x E4M3 product has <= 6 significant bits, so it is
    exact in fp32 and in bf16; the full product table is 256 x 8 x 1 B = 2 KB."""
    n = 0
    for s in range(256):
        sv = oracle.e4m3(s)
        if math.isnan(sv):
            continue
        for nib in range(16):
            p = oracle.e2m1(nib) * sv
            assert float(np.float32(p)) == p
            assert torch.tensor(p, dtype=torch.float64).to(torch.bfloat16).double().item() == p
            n += 1
    assert n == 254 * 16
    assert BYTE_MODEL["lut_entries_scales"] * BYTE_MODEL["lut_entries_magnitudes"] == BYTE_MODEL["lut_bytes"]


def test_byte_model_matches_pages():
    """P-d: the stored formats have the byte sizes the pages price: FP8 index
    key 128 B/token/layer, NVFP4 K+V 576 B (x 60 layers = 34,560 B vs FP8's
    61,440 B, 43.75 % less), scan/dense = 12.5 %."""
    w = synth.make_workload(seq_lens=[300, 128], seed=1)
    P = w.num_pages
    idx_b = w.idx_k.numel() * w.idx_k.element_size() / (P * 128)
    kv_b = sum(t.numel() * t.element_size() for t in (w.k, w.v, w.k_sf, w.v_sf)) / (P * 128)
    assert idx_b == BYTE_MODEL["index_key_bytes_per_token_per_layer"]
    dense_fp8 = w.num_kv_heads * 128 * 2
    assert dense_fp8 == BYTE_MODEL["dense_fp8_kv_bytes_per_token_per_layer"]
    layers = BYTE_MODEL["fp8_kv_bytes_per_token_model"] / dense_fp8
    assert layers == 60
    assert kv_b * layers == BYTE_MODEL["nvfp4_kv_bytes_per_token_model"]
    assert 1 - kv_b / dense_fp8 == BYTE_MODEL["nvfp4_saving"]
    assert idx_b / dense_fp8 == BYTE_MODEL["scan_to_dense_ratio"]
    assert BYTE_MODEL["top_blocks"] * BYTE_MODEL["block_tokens"] == BYTE_MODEL["keys_per_query_cap"]


# ---- helpers ---------------------------------------------------------------

def _sdpa(q, K, V, scale, mask=None):
    """fp64 torch SDPA for one query vector q [128] over K,V [n,128]."""
    return torch.nn.functional.scaled_dot_product_attention(
        q[None, None, None, :], K[None, None], V[None, None],
        attn_mask=None if mask is None else mask[None, None, None, :], scale=scale)[0, 0, 0]


def _visible_keys(P, row, sel_g):
    b = row // P.q_len
    L = int(P.arrays["seq_lens"][b])
    pos = L - P.q_len + row % P.q_len
    t = torch.arange(L)
    in_sel = torch.zeros(L, dtype=torch.bool)
    for j in sel_g:
        if j >= 0:
            in_sel |= (t // 128) == int(j)
    return in_sel & (t <= pos)


def _check_row_against_sdpa(P, w, row, sel, out, atol=1e-12):
    b = row // P.q_len
    _, K, V = dense_seq(P, b)
    qv, _ = row_queries(P, row)
    hpg = P.num_q_heads // P.num_kv_heads
    for g in range(P.num_kv_heads):
        mask = _visible_keys(P, row, sel[g])
        assert int(mask.sum()) <= 2048
        for hh in range(hpg):
            h = g * hpg + hh
            ref = _sdpa(qv[h], K[g], V[g], w.sm_scale, mask)
            np.testing.assert_allclose(out[h], ref.numpy(), rtol=1e-11, atol=atol)


# ---- attention -----------------------------------------------------------

@pytest.mark.parametrize("kv,idx", [("nvfp4", "fp8"), ("bf16", "bf16")])
def test_dense_when_at_most_16_blocks(kv, idx):
    """P-e: with <= 16 visible blocks every block is kept, so the oracle is
    plain (causal) dense attention: equal to torch SDPA in fp64."""
    w = synth.make_workload(seq_lens=[1, 127, 128, 129, 1000, 2048, 0], kv_dtype=kv, idx_dtype=idx, seed=3,
                            layout="paged")
    P = make_problem(w)
    _, sel, out = P.decode()
    for row in range(P.rows):
        L = int(P.arrays["seq_lens"][row])
        nbv = (L - 1) // 128 + 1 if L else 0
        assert sel[row, :, :nbv].tolist() == [list(range(nbv))] * 4
        assert (sel[row, :, nbv:] == -1).all()
        if L == 0:
            assert (out[row] == 0).all()
            continue
        _, K, V = dense_seq(P, row)
        qv, _ = row_queries(P, row)
        for h in range(16):
            ref = _sdpa(qv[h], K[h // 4], V[h // 4], w.sm_scale)
            np.testing.assert_allclose(out[row, h], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_dense_multi_query_causal():
    """P-e with q_len > 1: each query row attends causally (t <= its position)."""
    w = synth.make_workload(seq_lens=[900, 2000], q_len=5, seed=4)
    P = make_problem(w)
    _, sel, out = P.decode()
    for row in range(P.rows):
        b, i = divmod(row, 5)
        L = int(P.arrays["seq_lens"][b])
        pos = L - 5 + i
        _, K, V = dense_seq(P, b)
        qv, _ = row_queries(P, row)
        assert sel[row, 0, :(pos // 128) + 1].tolist() == list(range(pos // 128 + 1))
        for h in range(16):
            ref = _sdpa(qv[h], K[h // 4, :pos + 1], V[h // 4, :pos + 1], w.sm_scale)
            np.testing.assert_allclose(out[row, h], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_restricted_dense_equality():
    """P-f: output == dense attention restricted to (selected blocks AND t<=pos),
    torch SDPA fp64 with a boolean mask; also for an arbitrary given set."""
    w = synth.make_workload(seq_lens=[5000, 4097, 2177], plant=4, seed=5, layout="paged")
    P = make_problem(w)
    _, sel, out = P.decode()
    for row in range(P.rows):
        _check_row_against_sdpa(P, w, row, sel[row], out[row])
    rng = np.random.default_rng(1)
    for g in range(4):
        arb = np.full(16, -1, dtype=np.int32)
        picks = np.sort(rng.choice(40, size=7, replace=False))
        arb[:7] = picks
        o = P.attend(0, g, arb)
        mask = _visible_keys(P, 0, arb)
        _, K, V = dense_seq(P, 0)
        qv, _ = row_queries(P, 0)
        for hh in range(4):
            ref = _sdpa(qv[g * 4 + hh], K[g], V[g], w.sm_scale, mask)
            np.testing.assert_allclose(o[hh], ref.numpy(), rtol=1e-11, atol=1e-12)


# ---- selection -----------------------------------------------------------

def test_invariants_random():
    """P-g: |sel| = min(nbv,16), recent block present, ids distinct, ascending,
    in [0, nbv), at most 2,048 keys; across ragged lengths and q_len > 1."""
    for seed, lens, ql in [(6, [2049, 16 * 128, 16 * 128 + 1, 7000, 0, 300], 1), (7, [3000, 5000], 3)]:
        w = synth.make_workload(seq_lens=lens, q_len=ql, plant=2, seed=seed)
        P = make_problem(w)
        _, sel, _ = P.decode()
        for row in range(P.rows):
            b, i = divmod(row, ql)
            L = lens[b]
            if L == 0:
                assert (sel[row] == -1).all()
                continue
            pos = L - ql + i
            nbv = pos // 128 + 1
            for g in range(4):
                s = sel[row, g]
                kept = s[s >= 0]
                assert len(kept) == min(nbv, 16)
                assert (s[len(kept):] == -1).all()
                assert nbv - 1 in kept
                assert (np.diff(kept) > 0).all() and kept.min() >= 0 and kept.max() < nbv
                keys = sum(min(128, pos + 1 - j * 128) for j in kept)
                assert keys <= 2048


def _rank_count_select(bs, nbv):
    r = nbv - 1
    chosen = []
    for j in range(r):
        better = sum(1 for i in range(r) if i != j and (bs[i] > bs[j] or (bs[i] == bs[j] and i < j)))
        if better < 15:
            chosen.append(j)
    return sorted(chosen + [r])


@pytest.mark.parametrize("seed", range(40))
def test_selection_brute_force(seed):
    """P-h: (i) rank-count definition incl. ties (lower index wins);
    (ii) on tie-free scores, the kept set maximises the score sum over all
    15-subsets of the non-recent blocks."""
    rng = np.random.default_rng(seed)
    nbv = int(rng.integers(1, 21))
    if seed % 2:
        bs = rng.integers(-3, 3, size=nbv).astype(np.float64)  # many ties
    else:
        bs = rng.standard_normal(nbv)
    sel = oracle.select(bs, nbv)
    kept = sel[sel >= 0].tolist()
    if nbv <= 16:
        assert kept == list(range(nbv))
        return
    assert kept == _rank_count_select(bs, nbv)
    if seed % 2 == 0:
        r = nbv - 1
        best = max(itertools.combinations(range(r), 15), key=lambda c: sum(bs[list(c)]))
        assert kept == sorted(list(best) + [r])


def test_recent_score_is_irrelevant():
    """The recent block is kept whatever its own score (-1e300 or +1e300)."""
    rng = np.random.default_rng(3)
    bs = rng.standard_normal(40)
    for v in (-1e300, 1e300, 0.0):
        bs2 = bs.copy()
        bs2[39] = v
        s = oracle.select(bs2, 40)
        assert 39 in s and np.array_equal(s, oracle.select(bs, 40))


def test_split_merge_exact():
    """P-k: top-15 of the union of per-split top-15 lists == global top-15
    (total order: score desc, index asc), which the GPU's split scan relies on;
    both equal the oracle's selection."""
    rng = np.random.default_rng(11)
    for trial in range(30):
        nbv = int(rng.integers(17, 600))
        bs = np.round(rng.standard_normal(nbv) * 4) / 4  # ties on purpose
        r = nbv - 1

        def top15(ids):
            ids = np.asarray(ids)
            order = np.lexsort((ids, -bs[ids]))
            return ids[order[:15]]

        cuts = np.sort(rng.choice(np.arange(1, r), size=min(5, r - 1), replace=False))
        parts = np.split(np.arange(r), cuts)
        merged = top15(np.concatenate([top15(p) for p in parts if len(p)]))
        glob = top15(np.arange(r))
        assert sorted(merged.tolist()) == sorted(glob.tolist())
        sel = oracle.select(bs, nbv)
        assert sorted(glob.tolist()) + [r] == sel[sel >= 0].tolist()


def test_maxpool_matches_torch_amax():
    """P-i: block scores == torch.amax over [nb,128] of fp64 token scores
    (idx @ iq with torch's matmul), -inf padding past the end.  The index keys
    are decoded test-side (torch's E4M3 cast, the OCP E2M1 table), for FP8,
    bf16 and NVFP4 index keys."""
    for kv, idx in [("nvfp4", "fp8"), ("bf16", "bf16"), ("nvfp4", "nvfp4")]:
        w = synth.make_workload(seq_lens=[3001, 128 * 20], kv_dtype=kv, idx_dtype=idx, plant=3, seed=8,
                                layout="paged", max_blocks_per_seq=30)
        P = make_problem(w)
        for row in range(P.rows):
            ik, _, _ = dense_seq(P, row)
            _, iq = row_queries(P, row)
            L = ik.shape[0]
            nb = (L - 1) // 128 + 1
            s = ik @ iq.T                                   # [L, G]
            pad = torch.full((nb * 128, 4), -math.inf, dtype=torch.float64)
            pad[:L] = s
            ref = pad.reshape(nb, 128, 4).amax(dim=1).T      # [G, nb]
            for g in range(4):
                bs, nbv = P.block_scores(row, g)
                assert nbv == nb
                np.testing.assert_allclose(bs[:nb], ref[g].numpy(), rtol=1e-12, atol=1e-12)
                assert np.isneginf(bs[nb:]).all()


def test_nvfp4_index_keys_round_trip():
    """NVFP4 index keys: values placed exactly on the format's grid (E2M1 code
    x E4M3 group scale x power-of-two tensor scale, every group holding a +-6)
    survive the generator's quantiser unchanged, and the test-side decode
    (OCP table, torch's E4M3 cast; element 2i in the low nibble) returns them;
    the oracle's block scores of such keys equal fp64 matmul + amax of the
    original floats."""
    rng = np.random.default_rng(11)
    gs = 2.0 ** -7
    grid = E2M1_TABLE.numpy()
    codes = rng.integers(0, 16, size=(3, 128, 8, 16))
    codes[..., 0] = 7                                   # +6 in every group: amax16 = 6 * s * gs
    sc_bytes = rng.integers(0x08, 0x78, size=(3, 128, 8)).astype(np.uint8)  # normal E4M3, below 448
    sc = e4m3_t(sc_bytes).numpy()
    x = torch.from_numpy(grid[codes] * sc[..., None] * gs).reshape(3, 128, 128)
    packed, scales = synth.quant_nvfp4(x, gs)
    assert np.array_equal(scales.numpy(), sc_bytes)
    back = nvfp4_t(packed.numpy(), scales.numpy(), gs)
    assert torch.equal(back, x)
    w = synth.make_workload(seq_lens=[3 * 128 - 9], idx_dtype="nvfp4", seed=12)
    w.idx_k[:] = packed
    w.idx_sf[:] = scales
    w.idx_scale = gs
    P = make_problem(w)
    _, iq = row_queries(P, 0)
    s = x.reshape(3 * 128, 128)[:3 * 128 - 9] @ iq.T
    pad = torch.full((3 * 128, 4), -math.inf, dtype=torch.float64)
    pad[:3 * 128 - 9] = s
    ref = pad.reshape(3, 128, 4).amax(dim=1).T
    for g in range(4):
        bs, nbv = P.block_scores(0, g)
        assert nbv == 3
        np.testing.assert_allclose(bs[:3], ref[g].numpy(), rtol=1e-12, atol=1e-12)


def test_tail_is_masked():
    """R6: tokens past the end carry poison index keys that would win every
    block-max, and are excluded from pooling and attention (checked through
    P-i and P-f above); here: the tail's block is the recent one and a
    selected non-recent block never contains a token >= L."""
    w = synth.make_workload(seq_lens=[128 * 30 + 5], plant=0, seed=9)
    P = make_problem(w)
    bs, sel, out = P.decode()
    ik, _, _ = dense_seq(P, 0)
    _, iq = row_queries(P, 0)
    assert np.isfinite(bs[0, :, :31]).all()
    s_last = (ik[128 * 30:] @ iq.T).amax(dim=0).numpy()
    np.testing.assert_allclose(bs[0, :, 30], s_last, rtol=1e-12)


def test_paged_invariance():
    """P-j: permuting physical pages (and the block table with them) leaves
    the selection and the output bitwise unchanged."""
    w = synth.make_workload(seq_lens=[4000, 2600, 129], plant=3, seed=10, spare_pages=5)
    P = make_problem(w)
    bs0, sel0, out0 = P.decode()
    rng = np.random.default_rng(2)
    perm = rng.permutation(w.num_pages)
    a = P.arrays
    arr = dict(a)
    for key in ("idx_k", "k", "v", "k_sf", "v_sf"):
        new = np.empty_like(a[key])
        new[perm] = a[key]
        arr[key] = new
    arr["block_table"] = perm[a["block_table"]].astype(np.int32)
    P2 = oracle.Problem(num_seqs=w.num_seqs, q_len=1, num_q_heads=16, num_kv_heads=4,
                        max_blocks_per_seq=w.max_blocks_per_seq, num_pages=w.num_pages, kv_dtype="nvfp4",
                        idx_dtype="fp8", sm_scale=w.sm_scale, k_scale=w.k_scale, v_scale=w.v_scale,
                        idx_scale=w.idx_scale, **arr)
    bs1, sel1, out1 = P2.decode()
    assert np.array_equal(sel0, sel1)
    assert np.array_equal(out0, out1)
    assert np.array_equal(bs0, bs1)


def test_scale_invariance():
    """P-l: multiplying every index query by 2^k (exact in bf16) keeps the selection."""
    w = synth.make_workload(seq_lens=[6000, 3000], plant=3, seed=12)
    P = make_problem(w)
    _, sel0, _ = P.decode()
    for k in (-3, 1, 4):
        iq2 = (w.iq.float() * (2.0 ** k)).to(torch.bfloat16)
        assert torch.equal(iq2.float() / (2.0 ** k), w.iq.float())
        arr = dict(P.arrays)
        arr["iq"] = iq2.view(torch.int16).numpy().view(np.uint16)
        P2 = oracle.Problem(num_seqs=2, q_len=1, num_q_heads=16, num_kv_heads=4, max_blocks_per_seq=w.max_blocks_per_seq,
                            num_pages=w.num_pages, kv_dtype="nvfp4", idx_dtype="fp8", sm_scale=w.sm_scale,
                            k_scale=w.k_scale, v_scale=w.v_scale, idx_scale=w.idx_scale, **arr)
        _, sel1, _ = P2.decode()
        assert np.array_equal(sel0, sel1)


def test_planted_blocks_selected_tiny_config():
    """P-m: the 3 planted blocks per group of the tiny bf16 config are kept."""
    w = synth.make_config("tiny_b1_4k_bf16")
    P = make_problem(w)
    _, sel, _ = P.decode()
    for g in range(4):
        assert set(w.meta["planted"][(0, g)]) <= set(sel[0, g].tolist())


@pytest.mark.slow
def test_planted_blocks_selected_b8_32k():
    """P-m on the batch-8 32K config (6 planted blocks per group)."""
    w = synth.make_config("decode_b8_32k")
    P = make_problem(w)
    _, sel, _ = P.decode(want_scores=False)
    for b in range(8):
        for g in range(4):
            assert set(w.meta["planted"][(b, g)]) <= set(sel[b, g].tolist())


# ---- the write side (KV insert quantiser) ---------------------------------

def _e4m3_values():
    return e4m3_t(np.arange(0x7F, dtype=np.uint8)).numpy()     # 0 .. 448, ascending


def test_e4m3_rne_matches_torch_cast():
    """E4M3 rounding of the insert against torch's float8_e4m3fn cast (a
    library round-to-nearest-even, sign kept on zero): every midpoint between
    neighbours (exact ties), the floats next to them, zero, subnormals, values
    that round to zero and random values."""
    v = _e4m3_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)   # the ties are exact in fp32
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
                          v.astype(np.float32), np.random.default_rng(1).uniform(0, 448, 3000).astype(np.float32),
                          np.float32([2.0 ** -10, 2.0 ** -11, 2.0 ** -12, 1e-7, 0.0])])
    pts = np.concatenate([pts, -pts])
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_rne(y) for y in pts], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_bf16_rne_matches_torch_cast():
    """bf16 rounding of the insert (bf16 pools: x / scale stored as bf16)
    against torch's float32 -> bfloat16 cast (a library round-to-nearest-even):
    random floats over the whole exponent range, every pattern whose low 16
    bits are exactly halfway (ties, both parities of the kept bit) and one
    ulp either side of it, subnormals, signed zeros, the largest finite
    values (which round to infinity past half a bf16 unit), and quotients
    x / s with non-unit, non-power-of-two scales s as the insert forms them."""
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 0x7F800000, size=20000, dtype=np.uint32)
    half = (bits & 0xFFFF0000) | 0x8000
    pts = np.concatenate([bits, half, half + 1, half - 1,
                          rng.integers(0, 0x00800000, size=2000, dtype=np.uint32),          # subnormals
                          np.uint32([0, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x00008000, 0x00018000])])
    pts = np.concatenate([pts, pts | 0x80000000]).view(np.float32)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-8, 8, 4000))).astype(np.float32)
    for s in (np.float32(0.37), np.float32(1.7), np.float32(3.0), np.float32(0.1)):
        pts = np.concatenate([pts, x / s])
    ref = torch.from_numpy(pts).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(y)) for y in pts], dtype=np.uint16)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(pts[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    assert np.count_nonzero(ref == 0x7F80) > 0          # overflow to infinity was exercised
    assert len(set(((half >> 16) & 1).tolist())) == 2     # ties with both parities of the kept bit


def test_e2m1_rne_brute_force_and_generator():
    """E2M1 rounding: nearest magnitude by brute force (ties to the even code),
    saturating at 6; and equal to the generator's torch quantiser."""
    grid = E2M1_TABLE.numpy()[:8]
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(2)
    ys = np.concatenate([mids, grid, rng.uniform(-8, 8, 4000), [7.0, 100.0, 6.1, 5.9]]).astype(np.float32)
    ys = np.concatenate([ys, -ys])
    for y in ys:
        a = abs(float(y))
        d = np.abs(grid - a)
        cand = np.flatnonzero(d == d.min())
        code = int(cand[0]) if len(cand) == 1 else int([c for c in cand if c % 2 == 0][0])
        if a > 6:
            code = 7
        want = code | (8 if (y < 0 and code) else 0)
        assert oracle.e2m1_rne(y) == want, (y, oracle.e2m1_rne(y), want)
    gen = synth.quant_e2m1_codes(torch.from_numpy(ys)).numpy()
    assert np.array_equal(np.array([oracle.e2m1_rne(y) for y in ys], dtype=np.uint8), gen)


def test_nvfp4_group_quantiser_matches_generator():
    """Whole NVFP4 groups: with a power-of-two tensor scale the generator's
    torch quantiser performs the same fp32 operations, so the two independent
    implementations must store the same bytes; zero groups store scale 0."""
    rng = np.random.default_rng(3)
    for gs in (2.0 ** -9, 2.0 ** -3, 1.0):
        x = (rng.standard_normal((40, 128)) * rng.uniform(0.01, 3.0, (40, 1))).astype(np.float32)
        x[0, :16] = 0.0
        x[1, 16:32] = 1e-6
        packed, scales = synth.quant_nvfp4(torch.from_numpy(x), gs)
        for r in range(40):
            for c in range(8):
                p8, s = oracle.quant_nvfp4_group(x[r, 16 * c:16 * c + 16], gs)
                assert s == int(scales[r, c]), (gs, r, c)
                assert np.array_equal(p8, packed[r, 8 * c:8 * c + 8].numpy()), (gs, r, c)
        assert int(scales[0, 0]) == 0 and not packed[0, :8].any()


def test_nvfp4_group_quantiser_round_trip():
    """Values on the NVFP4 grid whose group holds a +-6 (so amax / (6 gs) is
    the stored scale exactly) come back unchanged through quantise + decode."""
    rng = np.random.default_rng(4)
    grid = E2M1_TABLE.numpy()
    for _ in range(200):
        gs = 2.0 ** int(rng.integers(-10, 2))
        codes = rng.integers(0, 16, 16)
        codes[rng.integers(0, 16)] = 7 + 8 * int(rng.integers(0, 2))
        s = int(rng.integers(0x08, 0x78))
        x = (grid[codes] * oracle.e4m3(s) * gs).astype(np.float32)
        p8, s_got = oracle.quant_nvfp4_group(x, gs)
        assert s_got == s
        back = np.array([oracle.e2m1((int(p8[k // 2]) >> (4 * (k & 1))) & 15) for k in range(16)]) * oracle.e4m3(s_got) * gs
        assert np.array_equal(back, x.astype(np.float64))


def test_kv_insert_writes_the_right_rows():
    """The insert writes row (b, i) at position seq_lens[b] - q_len + i: token
    row pos % 128 of page block_table[b][pos // 128] (located here with numpy),
    as the generator's quantiser stores those values (power-of-two tensor
    scales, where the two quantisers agree), and touches no other byte; a
    padded sequence writes nothing."""
    for idx_dtype in ("fp8", "nvfp4", "bf16"):
        w = synth.make_workload(seq_lens=[300, 0, 128 * 3], q_len=3, idx_dtype=idx_dtype, layout="paged", seed=13,
                                spare_pages=2)
        w.k_scale, w.v_scale = 2.0 ** -6, 2.0 ** -5
        w.idx_scale = 2.0 ** -4 if idx_dtype == "nvfp4" else 1.0
        P = make_problem(w)
        before = {k: None if v is None else v.copy() for k, v in P.arrays.items()}
        rng = np.random.default_rng(5)
        rows = w.rows
        kf = torch.from_numpy(rng.standard_normal((rows, 4, 128)).astype(np.float32)).to(torch.bfloat16)
        vf = torch.from_numpy(rng.standard_normal((rows, 4, 128)).astype(np.float32)).to(torch.bfloat16)
        xf = torch.from_numpy(rng.standard_normal((rows, 128)).astype(np.float32)).to(torch.bfloat16)
        bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
        P.kv_insert(bits(kf), bits(vf), bits(xf))
        a = P.arrays
        touched = {k: np.zeros(v.shape[:3] if k in ("k", "k_sf", "v_sf") else v.shape[:2], bool)
                   for k, v in a.items() if k in ("k", "k_sf", "v_sf", "idx_k", "idx_sf") and v is not None}
        # V is stored by dim: a written token changes one nibble of byte tok // 2 of each dim row
        v_expect = before["v"].copy()
        for row in range(rows):
            b, i = divmod(row, w.q_len)
            L = int(a["seq_lens"][b])
            if L == 0:
                continue
            pos = L - w.q_len + i
            page, tok = int(a["block_table"][b, pos // 128]), pos % 128
            packed, sc = synth.quant_nvfp4(kf[row].float(), w.k_scale)
            assert np.array_equal(a["k"][page, :, tok], packed.numpy())
            assert np.array_equal(a["k_sf"][page, :, tok], sc.numpy())
            touched["k"][page, :, tok] = touched["k_sf"][page, :, tok] = True
            # V: the token's codes sit in nibble tok % 2 of byte tok // 2 of every dim row
            codes, sc = synth.quant_nvfp4_codes(vf[row].float(), w.v_scale)
            sh = 4 * (tok % 2)
            cell = v_expect[page, :, :, tok // 2]
            v_expect[page, :, :, tok // 2] = (cell & (0xF0 >> sh)) | (codes.numpy().astype(np.uint8) << sh)
            assert np.array_equal(a["v_sf"][page, :, tok], sc.numpy())
            touched["v_sf"][page, :, tok] = True
            if idx_dtype == "nvfp4":
                packed, sc = synth.quant_nvfp4(xf[row].float(), w.idx_scale)
                assert np.array_equal(a["idx_k"][page, tok], packed.numpy())
                assert np.array_equal(a["idx_sf"][page, tok], sc.numpy())
                touched["idx_sf"][page, tok] = True
            elif idx_dtype == "fp8":
                assert np.array_equal(a["idx_k"][page, tok], synth.quant_e4m3(xf[row].float()).numpy())
            else:
                assert np.array_equal(a["idx_k"][page, tok], bits(xf[row]))
            touched["idx_k"][page, tok] = True
        for name, t in touched.items():
            assert np.array_equal(a[name][~t], before[name][~t]), name
        assert np.array_equal(a["v"], v_expect)
