"""Parity rules between the HIP path and the fp64 oracle.  TEST INFRASTRUCTURE.

Rules (the stated tolerances of the method's decode target, with the
readings written out):
  * selected block ids must equal the oracle's exactly, except when the 15th
    and 16th best non-recent blocks (oracle order: score desc, index asc) are
    within `tie_rel` (1e-4) relative of each other; then the GPU set may differ
    only in blocks whose oracle score is within `tie_rel` of the 15th, and the
    output is compared with the oracle re-run on the GPU's own set;
  * outputs: |gpu - oracle| <= atol + rtol * |oracle| elementwise, with
    atol = 2e-3, rtol = 1e-2 (fp32 accumulation);
  * block scores: the GPU's fp32 sums of exact products may differ from the
    fp64 value only by fp32 rounding, |d| <= 2 * 130 * 2^-24 * A, where A is the
    block's largest per-token sum of |iq_d * ik_td| (times idx_scale).  With
    NVFP4 index keys and 2..8 query tokens the score contraction runs in f16
    (NVFP4 keys converted straight to FP16 for the indexer's score MMA, vLLM
    MiniMax-M3.1-Flash post, "NVIDIA Rubin-optimised MSA"): each (row, group) index query is scaled by 2^k so that its
    largest |iq| lies in [2^14, 2^15) and rounded to f16; the bound then adds
    the block's largest per-token sum of |ik_td| * |iq_d - f16(iq_d 2^k) 2^-k|
    (times idx_scale; an element that lands among the f16 subnormals counts
    whole, in case the MFMA flushes it), which is 0 unless some |iq_d| is below
    2^-28 of its vector's largest.
"""
from __future__ import annotations

import numpy as np
import torch

ATOL = 2e-3
RTOL = 1e-2
TIE_REL = 1e-4


def _ik_dense(P, b):
    """The sequence's index keys as fp64 stored values (before idx_scale)."""
    a = P.arrays
    L = int(a["seq_lens"][b])
    nb = (L - 1) // 128 + 1 if L > 0 else 0
    pages = a["block_table"][b, :nb].astype(np.int64)
    raw = a["idx_k"][pages]
    if a.get("idx_sf") is not None:  # NVFP4: E2M1 code (low nibble first) x E4M3 group scale
        from . import e2m1
        table = torch.tensor([e2m1(n) for n in range(16)], dtype=torch.float64)
        p = torch.from_numpy(np.ascontiguousarray(raw)).to(torch.int64)
        codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(nb, 128, 128)
        sc = torch.from_numpy(np.ascontiguousarray(a["idx_sf"][pages])).view(torch.float8_e4m3fn).to(torch.float64)
        ik = table[codes] * sc.repeat_interleave(16, dim=-1)
    elif raw.dtype == np.uint8:
        ik = torch.from_numpy(np.ascontiguousarray(raw)).view(torch.float8_e4m3fn).to(torch.float64)
    else:
        ik = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return ik.reshape(nb * 128, 128), L, nb


def score_abs_bound(P, row):
    """[G][mbps] bound on |gpu - oracle| block scores of one query row."""
    return score_abs_bounds(P, [row])[row]


def score_abs_bounds(P, rows, chunk_cols=256):
    """{row: [G][mbps] bound on |gpu - oracle| block scores} for many query
    rows, decoding each sequence's index keys once (rows of one sequence share
    them) and taking the per-token sums for up to chunk_cols (row, group)
    index queries per matrix product.  The per-token sums run over every token
    of the sequence's blocks, so a multi-query row's bound on its recent block
    also counts tokens past its position: larger, still a bound."""
    rows = sorted(set(int(r) for r in rows))
    G, mb = P.num_kv_heads, P.max_blocks_per_seq
    f16_term = P.arrays.get("idx_sf") is not None and 1 < P.q_len <= 8   # the f16 column scan
    by_seq = {}
    for row in rows:
        by_seq.setdefault(row // P.q_len, []).append(row)
    out = {}
    for b, rs in by_seq.items():
        L = int(P.arrays["seq_lens"][b])
        if L == 0:
            for row in rs:
                out[row] = np.zeros((G, mb))
            continue
        ik, L, nb = _ik_dense(P, b)
        ika = ik[:L].abs()
        iq_all = torch.from_numpy(P.arrays["iq"][rs].view(np.int16)).view(torch.bfloat16).to(torch.float64)
        iq_all = iq_all.reshape(len(rs) * G, -1)                             # [(row, g)][128]
        for c0 in range(0, iq_all.shape[0], chunk_cols):
            iq = iq_all[c0:c0 + chunk_cols]
            A = (ika @ iq.abs().T) * (P.idx_scale * 2.0 * 130.0 * 2.0 ** -24)   # [L, cols]
            if f16_term:
                A = A + (ika @ f16_query_rounding(iq).T) * P.idx_scale
            pad = torch.zeros(nb * 128, A.shape[1], dtype=torch.float64)
            pad[:L] = A
            Ab = pad.reshape(nb, 128, -1).amax(dim=1).T.numpy()                # [cols, nb]
            for k in range(Ab.shape[0] // G):
                row = rs[(c0 + k * G) // G]
                o = np.zeros((G, mb))
                o[:, :nb] = Ab[k * G:(k + 1) * G] + 1e-30
                out[row] = o
    return out


def f16_query_rounding(iq):
    """|iq - f16(iq 2^k) 2^-k| per element of each [G][128] index query, with
    2^k the power of two that puts the vector's largest |iq| in [2^14, 2^15)."""
    x = iq.numpy()
    out = np.zeros_like(x)
    for g in range(x.shape[0]):
        mx = np.abs(x[g]).max()
        e = int(np.frexp(mx)[1]) if mx > 0 else 15
        k = max(-126, min(126, 15 - e))
        y = (x[g] * 2.0 ** k).astype(np.float32)
        q16 = y.astype(np.float16).astype(np.float64) * 2.0 ** -k
        # an f16 subnormal may also be flushed to zero inside the MFMA: count it whole
        out[g] = np.where(np.abs(y) < 2.0 ** -14, np.abs(x[g]), np.abs(x[g] - q16))
    return torch.from_numpy(out)


def _order(bs, r):
    ids = np.arange(r)
    return ids[np.lexsort((ids, -bs[:r]))]


def _row_position(P, row):
    """(pos, recent block r, visible blocks nbv) of a query row; pos -1 for a padded row."""
    L = int(P.arrays["seq_lens"][row // P.q_len])
    if L <= 0:
        return -1, -1, 0
    pos = L - P.q_len + row % P.q_len
    return pos, pos // 128, pos // 128 + 1


def check_selection_valid(gpu_sel_g, r, nbv, where=""):
    """What every selection must be, whatever the scores: min(nbv, 16) distinct
    ids in strictly ascending order, each a visible block (0 <= id < nbv), the
    recent block r among them, -1 only as trailing padding."""
    ids = np.asarray(gpu_sel_g)
    keep = min(nbv, 16)
    assert ids.shape == (16,), f"{where}: {ids.shape} ids"
    assert (ids[keep:] == -1).all(), f"{where}: ids past the first {keep} must be -1 padding: {ids}"
    kept = ids[:keep]
    assert (kept >= 0).all() and (kept < nbv).all(), f"{where}: id outside the visible blocks 0..{nbv - 1}: {ids}"
    assert (np.diff(kept) > 0).all(), f"{where}: ids not strictly ascending (duplicate or out of order): {ids}"
    assert keep == 0 or r in kept.tolist(), f"{where}: the recent block {r} is missing: {ids}"


def check_row(P, row, gpu_out, gpu_sel, gpu_bs=None, *, atol=ATOL, rtol=RTOL, tie_rel=TIE_REL, oracle_row=None,
              bound=None):
    """Compares one query row; returns a dict of findings (raises on failure).
    oracle_row: this row's (bs, sel, out) from a batched oracle call, each with
    a leading axis of 1; bound: its block-score bound, from score_abs_bounds."""
    bs_o, sel_o, out_o = oracle_row if oracle_row is not None else P.decode(row, row + 1)
    bs_o, sel_o, out_o = bs_o[0], sel_o[0], out_o[0]
    G = sel_o.shape[0]
    hpg = out_o.shape[0] // G
    pos, r, nbv = _row_position(P, row)
    info = dict(row=row, near_ties=0, max_abs_err=0.0)
    if gpu_bs is not None:
        bound = score_abs_bound(P, row) if bound is None else bound
        fin = np.isfinite(bs_o)
        assert np.array_equal(np.isneginf(gpu_bs), np.isneginf(bs_o)), f"row {row}: -inf pattern of block scores"
        err = np.abs(gpu_bs[fin].astype(np.float64) - bs_o[fin])
        assert (err <= bound[fin]).all(), f"row {row}: block score error {err.max()} > bound"
    for g in range(G):
        ref_out = out_o[g * hpg:(g + 1) * hpg]
        if not np.array_equal(gpu_sel[g], sel_o[g]):
            where = f"row {row} g {g}"
            check_selection_valid(gpu_sel[g], r, nbv, where)
            # near tie (R20): with the non-recent blocks in oracle order, the
            # 15th and 16th are within tie_rel; the GPU may then swap blocks
            # of that band only, as many in as out
            order = _order(bs_o[g], r)
            assert len(order) >= 16, f"{where}: sets differ with <= 16 candidates"
            c, c2 = bs_o[g][order[14]], bs_o[g][order[15]]
            near = abs(c - c2) < tie_rel * max(abs(c), abs(c2))
            assert near, f"{where}: selection differs without a near tie: gpu {gpu_sel[g]} oracle {sel_o[g]}"
            got, want = set(gpu_sel[g].tolist()) - {-1}, set(sel_o[g].tolist()) - {-1}
            added, dropped = got - want, want - got
            assert len(added) == len(dropped), f"{where}: {len(added)} blocks added, {len(dropped)} dropped"
            assert all(abs(bs_o[g][j] - c) <= tie_rel * abs(c) for j in added | dropped), \
                f"{where}: differing block not within the tie band"
            info["near_ties"] += 1
            ref_out = P.attend(row, g, gpu_sel[g])
        got = gpu_out[g * hpg:(g + 1) * hpg].astype(np.float64)
        err = np.abs(got - ref_out)
        bad = err > atol + rtol * np.abs(ref_out)
        assert not bad.any(), f"row {row} g {g}: output error {err.max()} (ref {ref_out.flat[np.argmax(err)]})"
        info["max_abs_err"] = max(info["max_abs_err"], float(err.max()))
    return info


def check_rows(P, gpu_out, gpu_sel, gpu_bs=None, rows=None, **kw):
    """Every given row (default: all) against one batched oracle call over the
    row range they span (OpenMP over (row, group) pairs), block-score bounds
    taken per sequence.  Returns (near ties, worst abs output error)."""
    rows = list(range(P.rows)) if rows is None else sorted(int(x) for x in rows)
    if not rows:
        return 0, 0.0
    lo, hi = rows[0], rows[-1] + 1
    bs_o, sel_o, out_o = P.decode(lo, hi, want_scores=True)
    bounds = score_abs_bounds(P, rows) if gpu_bs is not None else {}
    ties, worst = 0, 0.0
    for row in rows:
        k = row - lo
        info = check_row(P, row, gpu_out[row], gpu_sel[row], None if gpu_bs is None else gpu_bs[row],
                         oracle_row=(bs_o[k:k + 1], sel_o[k:k + 1], out_o[k:k + 1]), bound=bounds.get(row), **kw)
        ties += info["near_ties"]
        worst = max(worst, info["max_abs_err"])
    return ties, worst
