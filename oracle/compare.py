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
    """[G][mbps] bound on |gpu - oracle| block scores of one decode row."""
    b = row // P.q_len
    ik, L, nb = _ik_dense(P, b)
    iq = torch.from_numpy(P.arrays["iq"][row].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    G = iq.shape[0]
    out = np.zeros((G, P.max_blocks_per_seq))
    if L == 0:
        return out
    A = (ik[:L].abs() @ iq.abs().T) * P.idx_scale              # [L, G]
    if P.arrays.get("idx_sf") is not None and 1 < P.q_len <= 8:  # the f16 column scan
        A = A * (2.0 * 130.0 * 2.0 ** -24) + (ik[:L].abs() @ f16_query_rounding(iq).T) * P.idx_scale
    else:
        A = A * (2.0 * 130.0 * 2.0 ** -24)
    pad = torch.zeros(nb * 128, G, dtype=torch.float64)
    pad[:L] = A
    Ab = pad.reshape(nb, 128, G).amax(dim=1).T.numpy()         # [G, nb]
    out[:, :nb] = Ab + 1e-30
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


def check_row(P, row, gpu_out, gpu_sel, gpu_bs=None, *, atol=ATOL, rtol=RTOL, tie_rel=TIE_REL, oracle_row=None):
    """Compares one query row; returns a dict of findings (raises on failure)."""
    bs_o, sel_o, out_o = oracle_row if oracle_row is not None else P.decode(row, row + 1)
    bs_o, sel_o, out_o = bs_o[0], sel_o[0], out_o[0]
    G = sel_o.shape[0]
    hpg = out_o.shape[0] // G
    info = dict(row=row, near_ties=0, max_abs_err=0.0)
    if gpu_bs is not None:
        bound = score_abs_bound(P, row)
        fin = np.isfinite(bs_o)
        assert np.array_equal(np.isneginf(gpu_bs), np.isneginf(bs_o)), f"row {row}: -inf pattern of block scores"
        err = np.abs(gpu_bs[fin].astype(np.float64) - bs_o[fin])
        assert (err <= bound[fin]).all(), f"row {row}: block score error {err.max()} > bound"
    for g in range(G):
        ref_out = out_o[g * hpg:(g + 1) * hpg]
        if not np.array_equal(gpu_sel[g], sel_o[g]):
            kept_o = sel_o[g][sel_o[g] >= 0]
            r = int(kept_o.max())
            order = _order(bs_o[g], r)
            assert len(order) >= 16, f"row {row} g {g}: sets differ with <= 16 candidates"
            c, c2 = bs_o[g][order[14]], bs_o[g][order[15]]
            near = abs(c - c2) < tie_rel * max(abs(c), abs(c2))
            diff = set(gpu_sel[g].tolist()) ^ set(sel_o[g].tolist())
            assert near, f"row {row} g {g}: selection differs without a near tie: gpu {gpu_sel[g]} oracle {sel_o[g]}"
            assert all(abs(bs_o[g][j] - c) <= tie_rel * abs(c) for j in diff if j >= 0), \
                f"row {row} g {g}: differing block not within the tie band"
            info["near_ties"] += 1
            ref_out = P.attend(row, g, gpu_sel[g])
        got = gpu_out[g * hpg:(g + 1) * hpg].astype(np.float64)
        err = np.abs(got - ref_out)
        bad = err > atol + rtol * np.abs(ref_out)
        assert not bad.any(), f"row {row} g {g}: output error {err.max()} (ref {ref_out.flat[np.argmax(err)]})"
        info["max_abs_err"] = max(info["max_abs_err"], float(err.max()))
    return info
