"""Seeded synthetic inputs for the MSA decode path.

This module only *makes* inputs: random tensors, the quantisers that pack them
into the stored formats, and the paged layout.  It contains none of the
method's arithmetic (no decoding, scoring, pooling, selection or attention),
so both the HIP path and the CPU oracle can consume its bytes without sharing
any of the computation under test.

Stored formats (the layouts the library reads):
  q      bf16  [rows][Hq][128]          rows = num_seqs * q_len, request-major
  iq     bf16  [rows][Hkv][128]         one index query per GQA group
  idx_k  FP8 E4M3 (uint8) or bf16  [P][128 tokens][128], or NVFP4 uint8
         [P][128 tokens][64] + E4M3 scales idx_sf uint8 [P][128 tokens][8]
         (one shared index head; its fp32 tensor scale is idx_scale)
  k      NVFP4: uint8 [P][Hkv][128 tokens][64]   (element 2i in the low nibble)
         + E4M3 scales uint8 [P][Hkv][128 tokens][8]  (one per 16 elements)
         + one fp32 tensor scale;
  v      NVFP4: uint8 [P][Hkv][128 dims][64], each page's V transposed: row d
         holds dim d of the page's 128 tokens, token 2i in the low nibble of
         byte i; E4M3 scales as K's, [P][Hkv][128 tokens][8] (one per token and
         16 dims), + one fp32 tensor scale;
  k, v   bf16: [P][Hkv][128 tokens][128]
  block_table int32 [num_seqs][max_blocks_per_seq]; seq_lens int32 [num_seqs]

NVFP4 quantiser (harness only; results do not depend on it because both sides
decode the stored bytes): tensor scale gs = amax / (6 * 448); per group of 16,
s = E4M3(amax16 / (6 * gs)) round-to-nearest-even; code = the E2M1 value
nearest to x / (s * gs), ties to even, saturating at +-6.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK = 128
DIM = 128
# stored bytes of one token's index key: FP8 128, bf16 256, NVFP4 64 + 8 scales
IDX_BYTES_PER_TOKEN = {"fp8": DIM, "bf16": 2 * DIM, "nvfp4": DIM // 2 + DIM // 16}
E4M3_MAX = 448.0
# E2M1 magnitude grid, code index == magnitude code (OCP FP4)
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def quant_e4m3(x: torch.Tensor) -> torch.Tensor:
    """float -> OCP E4M3 bytes, round-to-nearest-even; clamps to +-448 first
    because torch turns out-of-range values into NaN instead of saturating."""
    return x.float().clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def quant_e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """float (already divided by its scale) -> 4-bit E2M1 codes (uint8, one per
    element), nearest value with ties to the even code, saturating at +-6."""
    mids = torch.tensor(_E2M1_MIDS, device=y.device, dtype=torch.float32)
    a = y.abs().float().clamp(max=6.0)
    idx = torch.bucketize(a, mids, right=False)  # mids[idx-1] < a <= mids[idx]
    # a tie sits exactly on mids[idx]; bucketize put it low, which is right when
    # the lower neighbour has the even code (idx even) and wrong otherwise.
    on_mid = (idx < len(_E2M1_MIDS)) & (a == mids[idx.clamp(max=len(_E2M1_MIDS) - 1)])
    idx = idx + (on_mid & (idx % 2 == 1)).to(idx.dtype)
    sign = ((y < 0) & (idx > 0)).to(torch.uint8)
    return (sign << 3) | idx.to(torch.uint8)


def nvfp4_tensor_scale(amax: float) -> float:
    return float(amax) / (6.0 * E4M3_MAX) if amax > 0 else 1.0


def quant_nvfp4_codes(x: torch.Tensor, gs: float):
    """x [..., 128] float -> (E2M1 codes uint8 [..., 128], scales uint8 [..., 8])."""
    shp = x.shape
    xg = x.float().reshape(*shp[:-1], DIM // 16, 16)
    amax16 = xg.abs().amax(dim=-1)
    sc = quant_e4m3(amax16 / (6.0 * gs))                       # [..., 8] bytes
    sc_val = sc.view(torch.float8_e4m3fn).float()              # exact decode of the stored scale
    denom = (sc_val * gs).unsqueeze(-1)
    y = torch.where(denom > 0, xg / torch.where(denom > 0, denom, torch.ones_like(denom)), torch.zeros_like(xg))
    return quant_e2m1_codes(y).reshape(*shp[:-1], DIM), sc.contiguous()


def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """[..., 2n] codes -> [..., n] bytes, element 2i in the low nibble of byte i."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).contiguous()


def quant_nvfp4(x: torch.Tensor, gs: float):
    """x [..., 128] float -> (packed uint8 [..., 64], scales uint8 [..., 8])."""
    codes, sc = quant_nvfp4_codes(x, gs)
    return pack_nibbles(codes), sc


def quant_nvfp4_v(x: torch.Tensor, gs: float):
    """V of whole pages, x [..., 128 tokens, 128 dims] float -> (packed uint8
    [..., 128 dims, 64]: row d holds dim d of the tokens, token 2i in the low
    nibble of byte i; scales uint8 [..., 128 tokens, 8])."""
    codes, sc = quant_nvfp4_codes(x, gs)
    return pack_nibbles(codes.transpose(-1, -2)), sc


@dataclass
class Workload:
    """One batch of synthetic inputs, resident on `device`."""
    name: str
    num_seqs: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    max_blocks_per_seq: int
    num_pages: int
    kv_dtype: str            # "bf16" | "nvfp4"
    idx_dtype: str           # "bf16" | "fp8" | "nvfp4"
    sm_scale: float
    k_scale: float
    v_scale: float
    idx_scale: float
    q: torch.Tensor
    iq: torch.Tensor
    idx_k: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    k_sf: Optional[torch.Tensor]
    v_sf: Optional[torch.Tensor]
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    meta: dict = field(default_factory=dict)
    idx_sf: Optional[torch.Tensor] = None   # NVFP4 index keys: E4M3 group scales [P][128][8]
    # prefix sharing (None without): int32 [groups][8] member sequence ids
    # (-1 padded, the first is the leader whose pages the members share),
    # int32 [groups] shared leading blocks, int32 [S] per-sequence shared blocks
    share_members: Optional[torch.Tensor] = None
    share_blocks: Optional[torch.Tensor] = None
    seq_shared_blocks: Optional[torch.Tensor] = None

    @property
    def rows(self) -> int:
        return self.num_seqs * self.q_len

    def host_arrays(self) -> dict:
        """numpy copies of exactly the bytes the device path reads."""
        def u16(t):
            return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        def raw(t):
            if t is None:
                return None
            if t.dtype == torch.bfloat16:
                return u16(t)
            return t.detach().contiguous().cpu().numpy()

        return dict(q=u16(self.q), iq=u16(self.iq), idx_k=raw(self.idx_k), k=raw(self.k), v=raw(self.v),
                    k_sf=raw(self.k_sf), v_sf=raw(self.v_sf), idx_sf=raw(self.idx_sf),
                    block_table=self.block_table.cpu().numpy().astype(np.int32),
                    seq_lens=self.seq_lens.cpu().numpy().astype(np.int32))

    def nbytes_algorithmic(self, sel=None) -> dict:
        """Bytes the method must move per layer-step: every visible token's
        index key, K+V of the selected tokens only, the used block-table
        entries, q, iq and the fp32 output.  K/V is counted once per (sequence,
        group, selected block): with q_len > 1 the union of the rows' selections
        (needs the step's `sel` [rows][groups][16]); without `sel`, 16 blocks
        per group (exact for q_len 1)."""
        lens = [int(x) for x in self.seq_lens.cpu().tolist()]
        b_idx = IDX_BYTES_PER_TOKEN[self.idx_dtype]
        b_kv_tok = DIM * (0.5 + 1.0 / 16) if self.kv_dtype == "nvfp4" else DIM * 2.0
        scan = sum(lens) * b_idx
        if self.seq_shared_blocks is not None:  # a shared page's keys are read once for its group
            ssb = [int(x) for x in self.seq_shared_blocks.cpu().tolist()]
            leaders = set(int(m[0]) for m in self.share_members.cpu().tolist())
            scan -= sum(ssb[b] * BLOCK * b_idx for b in range(len(lens)) if b not in leaders)
        gather = 0.0
        table = 0
        if sel is not None:
            sel = sel.cpu().reshape(self.num_seqs, self.q_len, self.num_kv_heads, 16)
        for b, L in enumerate(lens):
            if L <= 0:
                continue
            nb = (L - 1) // BLOCK + 1
            if sel is None:
                kept = self.num_kv_heads * min(nb, 16)
            else:
                kept = sum(int(torch.unique(sel[b, :, g][sel[b, :, g] >= 0]).numel())
                           for g in range(self.num_kv_heads))
            gather += kept * BLOCK * b_kv_tok * 2   # K and V
            table += nb * 4
        qio = self.rows * (self.num_q_heads + self.num_kv_heads) * DIM * 2
        out = self.rows * self.num_q_heads * DIM * 4
        return dict(scan=scan, gather=gather, table=table, q_iq=qio, out=out,
                    total=scan + gather + table + qio + out)


def make_workload(*, name: str = "custom", seq_lens, q_len: int = 1, kv_dtype: str = "nvfp4",
                  idx_dtype: str = "fp8", max_blocks_per_seq: Optional[int] = None, layout: str = "identity",
                  spare_pages: int = 0, plant: int = 0, zipf: Optional[float] = None, zipf_amp: float = 4.0,
                  idx_dist: str = "normal", shared_bias_iq: bool = False, iq_noise: float = 1.0, seed: int = 0,
                  device="cpu", num_q_heads: int = 16, num_kv_heads: int = 4,
                  sm_scale: Optional[float] = None, idx_scale: float = 1.0,
                  kv_chunk_pages: int = 1024, share: Optional[tuple] = None) -> Workload:
    """Seeded synthetic workload.

    seq_lens: visible tokens per sequence (including the q_len new tokens);
    0 marks a padded row.  layout "identity" gives sequence b the consecutive
    pages of its blocks; "paged" scatters all pages through the pool with one
    random permutation (the block table is then a random int32 map).
    plant n: for each (sequence, group), n distinct non-recent blocks get
    2.0 * (unit index-query direction) added to every index key.
    zipf s: for each (sequence, group) a random permutation ranks the
    non-recent blocks 1..nb-1 and block of rank k gets zipf_amp * k^-s times the
    unit direction added.  idx_dist: "normal" N(0,1) or "uniform" U(-1,1).
    shared_bias_iq: (q_len > 1) index queries are u_{b,g} + iq_noise N(0,1),
    with u the bias direction shared by the chunk (a small iq_noise: queries
    of a chunk that select mostly the same blocks).
    share (group_size, shared_blocks): consecutive sequences form groups of
    group_size (at most 64 / q_len) whose first shared_blocks logical blocks map to the
    leader's (the group's first sequence's) pages: a shared prefix, keys and
    K/V included.  Every member must see all shared tokens.
    Index-key rows past a sequence's end are filled with a poison value that
    scores high, so an unmasked tail would show up in the selection.
    """
    dev = torch.device(device)
    seq_lens = [int(x) for x in seq_lens]
    S = len(seq_lens)
    G, Hq = num_kv_heads, num_q_heads
    nbs = [((L - 1) // BLOCK + 1) if L > 0 else 0 for L in seq_lens]
    mbps = max_blocks_per_seq if max_blocks_per_seq is not None else max([1] + nbs)
    assert all(nb <= mbps for nb in nbs)
    assert all(L == 0 or L >= q_len for L in seq_lens)
    # ---- prefix sharing: owned[b] = first logical block with a page of b's own
    owned = [0] * S
    groups = []
    if share is not None:
        gsize, sblocks = int(share[0]), int(share[1])
        assert 1 <= gsize and gsize * q_len <= 64 and sblocks >= 0
        for g0 in range(0, S, gsize):
            members = list(range(g0, min(S, g0 + gsize)))
            if len(members) < 2:  # a group of one shares nothing
                continue
            for b in members:
                assert seq_lens[b] == 0 or sblocks * BLOCK <= seq_lens[b] - q_len + 1, "shared tokens must be visible"
                assert seq_lens[b] > 0, "padded rows cannot share"
            groups.append(members)
            for b in members[1:]:
                owned[b] = sblocks
    P = sum(nb - o for nb, o in zip(nbs, owned)) + spare_pages
    P = max(P, 1)
    rows = S * q_len

    # ---- page map
    perm = torch.arange(P, dtype=torch.int64)
    if layout == "paged":
        perm = torch.randperm(P, generator=_gen("cpu", seed * 7919 + 1))
    elif layout != "identity":
        raise ValueError(layout)
    bt = torch.zeros(S, mbps, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nbs):
        n_own = nb - owned[b]
        bt[b, owned[b]:nb] = perm[off:off + n_own].to(torch.int32)
        off += n_own
    for members in groups:
        for b in members[1:]:
            bt[b, :owned[b]] = bt[members[0], :owned[b]]

    # ---- queries
    gq = _gen(dev, seed * 7919 + 2)
    q = torch.randn(rows, Hq, DIM, generator=gq, device=dev).to(torch.bfloat16)
    if shared_bias_iq:
        u = torch.randn(S, 1, G, DIM, generator=gq, device=dev)
        iqf = u + float(iq_noise) * torch.randn(S, q_len, G, DIM, generator=gq, device=dev)
        iq = iqf.reshape(rows, G, DIM).to(torch.bfloat16)
        direction = (u[:, 0] / u[:, 0].norm(dim=-1, keepdim=True))            # [S][G][D]
    else:
        iq = torch.randn(rows, G, DIM, generator=gq, device=dev).to(torch.bfloat16)
        iq_last = iq.view(S, q_len, G, DIM)[:, -1].float().double()
        direction = (iq_last / iq_last.norm(dim=-1, keepdim=True)).float()     # [S][G][D]

    # ---- index keys, per sequence in logical order, scattered to pages
    planted = {}

    def index_keys():
        """(b, float keys [nb][128][128]) per sequence, from fresh generators
        (NVFP4 walks the stream twice: amax first, then the same keys)."""
        gi = _gen(dev, seed * 7919 + 3)
        gsel = _gen("cpu", seed * 7919 + 4)
        for b in range(S):
            nb, L = nbs[b], seq_lens[b]
            if nb == 0:
                continue
            if idx_dist == "normal":
                keys = torch.randn(nb, BLOCK, DIM, generator=gi, device=dev)
            elif idx_dist == "uniform":
                keys = torch.rand(nb, BLOCK, DIM, generator=gi, device=dev) * 2.0 - 1.0
            else:
                raise ValueError(idx_dist)
            r_last = nb - 1
            bias = torch.zeros(nb, DIM, device=dev)
            for g in range(G):
                dvec = direction[b, g].to(dev)
                if plant and r_last > 0:
                    n = min(plant, r_last)
                    picks = torch.randperm(r_last, generator=gsel)[:n]
                    planted[(b, g)] = sorted(int(x) for x in picks)
                    bias[picks.to(dev)] += 2.0 * dvec
                if zipf is not None and r_last > 0:
                    ranks = torch.randperm(r_last, generator=gsel).to(torch.float64) + 1.0  # block j -> rank
                    w = (zipf_amp * ranks.pow(-zipf)).to(torch.float32).to(dev)
                    bias[:r_last] += w[:, None] * dvec[None, :]
            keys += bias[:, None, :]
            tail = L - (nb - 1) * BLOCK
            if tail < BLOCK:
                keys[nb - 1, tail:] = 3.0 * direction[b].sum(dim=0).to(dev)  # poison past the end
            yield b, keys

    idx_sf = None
    if idx_dtype == "nvfp4":
        amax = 0.0
        for _, keys in index_keys():
            amax = max(amax, float(keys.abs().max()))
        idx_gs = nvfp4_tensor_scale(amax)
        idx_pool = torch.zeros(P, BLOCK, DIM // 2, dtype=torch.uint8, device=dev)
        idx_sf = torch.zeros(P, BLOCK, DIM // 16, dtype=torch.uint8, device=dev)
        for b, keys in index_keys():
            o = owned[b]
            pages = bt[b, o:nbs[b]].long().to(dev)
            idx_pool[pages], idx_sf[pages] = quant_nvfp4(keys[o:], idx_gs)
        idx_scale = idx_scale * idx_gs
    elif idx_dtype in ("fp8", "bf16"):
        bidx = 1 if idx_dtype == "fp8" else 2
        idx_pool = torch.zeros(P, BLOCK, DIM * bidx, dtype=torch.uint8, device=dev)
        for b, keys in index_keys():
            o = owned[b]
            keys = keys[o:]
            if idx_dtype == "fp8":
                kb = quant_e4m3(keys)
            else:
                kb = keys.to(torch.bfloat16).contiguous().view(torch.uint8).reshape(nbs[b] - o, BLOCK, DIM * 2)
            idx_pool[bt[b, o:nbs[b]].long().to(dev)] = kb
        if idx_dtype == "bf16":
            idx_pool = idx_pool.view(torch.bfloat16).reshape(P, BLOCK, DIM)
    else:
        raise ValueError(idx_dtype)

    # ---- K / V pools (i.i.d. N(0,1), generated page-chunk by page-chunk)
    def kv_pool(seed_k, is_v):
        if kv_dtype == "bf16":
            gk = _gen(dev, seed_k)
            out = torch.empty(P, G, BLOCK, DIM, dtype=torch.bfloat16, device=dev)
            for c0 in range(0, P, kv_chunk_pages):
                c1 = min(P, c0 + kv_chunk_pages)
                out[c0:c1] = torch.randn(c1 - c0, G, BLOCK, DIM, generator=gk, device=dev).to(torch.bfloat16)
            return out, None, 1.0
        # pass 1: amax, pass 2: quantise the same stream
        amax = 0.0
        gk = _gen(dev, seed_k)
        for c0 in range(0, P, kv_chunk_pages):
            c1 = min(P, c0 + kv_chunk_pages)
            amax = max(amax, float(torch.randn(c1 - c0, G, BLOCK, DIM, generator=gk, device=dev).abs().max()))
        gs = nvfp4_tensor_scale(amax)
        packed = torch.empty(P, G, BLOCK, DIM // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(P, G, BLOCK, DIM // 16, dtype=torch.uint8, device=dev)
        gk = _gen(dev, seed_k)
        for c0 in range(0, P, kv_chunk_pages):
            c1 = min(P, c0 + kv_chunk_pages)
            x = torch.randn(c1 - c0, G, BLOCK, DIM, generator=gk, device=dev)
            packed[c0:c1], scales[c0:c1] = quant_nvfp4_v(x, gs) if is_v else quant_nvfp4(x, gs)
        return packed, scales, gs

    k, k_sf, k_scale = kv_pool(seed * 7919 + 5, False)
    v, v_sf, v_scale = kv_pool(seed * 7919 + 6, True)

    return Workload(name=name, num_seqs=S, q_len=q_len, num_q_heads=Hq, num_kv_heads=G,
                    max_blocks_per_seq=mbps, num_pages=P, kv_dtype=kv_dtype, idx_dtype=idx_dtype,
                    sm_scale=sm_scale if sm_scale is not None else 1.0 / math.sqrt(DIM),
                    k_scale=float(k_scale), v_scale=float(v_scale), idx_scale=float(idx_scale),
                    q=q, iq=iq, idx_k=idx_pool, k=k, v=v, k_sf=k_sf, v_sf=v_sf,
                    block_table=bt.to(dev), seq_lens=torch.tensor(seq_lens, dtype=torch.int32, device=dev),
                    meta=dict(seed=seed, layout=layout, plant=plant, zipf=zipf, idx_dist=idx_dist,
                              planted=planted, share=share,
                              # lower bound of every sequence's shared blocks (0 unless all share)
                              min_shared_blocks=(int(share[1]) if share is not None and
                                                 sum(len(m) for m in groups) == S else 0)),
                    idx_sf=idx_sf, **_share_tensors(groups, share, S, dev))


def _share_tensors(groups, share, S, dev) -> dict:
    """The prefix-sharing descriptors of make_workload(share=...)."""
    if share is None:
        return {}
    members = torch.full((len(groups), int(share[0])), -1, dtype=torch.int32)   # rows of group_size slots
    for gi, mem in enumerate(groups):
        members[gi, :len(mem)] = torch.tensor(mem, dtype=torch.int32)
    sblocks = int(share[1])
    per_seq = torch.zeros(S, dtype=torch.int32)
    for mem in groups:
        per_seq[mem] = sblocks
    return dict(share_members=members.to(dev),
                share_blocks=torch.full((len(groups),), sblocks, dtype=torch.int32, device=dev),
                seq_shared_blocks=per_seq.to(dev))


# The five workloads the method is evaluated on.  Every config uses 4 KV heads
# (= 4 GQA groups = 4 index queries per token), 16 query heads, head and index
# dim 128 and 128-token blocks.
CONFIGS = {
    # batch 1, 4,096 tokens, everything bf16, 3 planted blocks per group
    "tiny_b1_4k_bf16": dict(seq_lens=[4096], kv_dtype="bf16", idx_dtype="bf16", plant=3,
                            layout="identity", seed=0),
    # batch 8, 32K tokens, NVFP4 K/V, FP8 index keys, 6 planted blocks per group
    "decode_b8_32k": dict(seq_lens=[32768] * 8, plant=6, layout="identity", seed=1),
    # batch 32, 128K tokens each, paged pool with a random block table,
    # Zipf(1.1) block-score bias
    "paged_b32_128k": dict(seq_lens=[131072] * 32, zipf=1.1, layout="paged", seed=2),
    # batch 4, 512K tokens, U(-1,1) index keys, 8 planted blocks per group, paged
    "paged_b4_512k": dict(seq_lens=[524288] * 4, idx_dist="uniform", plant=8, layout="paged", seed=3),
    # batch 2 x 256 new query tokens appended causally to a 128K paged context
    "verify_b2_q256_128k": dict(seq_lens=[131072 + 256] * 2, q_len=256, zipf=1.1, layout="paged",
                                shared_bias_iq=True, seed=4),
    # the 2 x 256-token chunk with strongly correlated index queries
    # (u + 0.25 N(0,1)): neighbouring queries select mostly the same blocks,
    # the case the KV-block-major attention is built for; not one of the five
    "verify_b2_q256_128k_corr": dict(seq_lens=[131072 + 256] * 2, q_len=256, zipf=1.1, layout="paged",
                                     shared_bias_iq=True, iq_noise=0.25, seed=4),
    # speculative verify on the decode path: batch 32, each sequence a 128K
    # context plus 4 new query tokens (1 + 3 draft tokens, the draft length of
    # the AMD serving recipe); not one of the five above
    "spec_b32_q4_128k": dict(seq_lens=[131072 + 4] * 32, q_len=4, zipf=1.1, layout="paged", seed=5),
    # batch 32 x 128K in groups of 8 sequences sharing a 96K-token prefix
    # (768 blocks: system prompt and agent context), own 32K each; not one of
    # the five above
    "shared_b32_128k": dict(seq_lens=[131072] * 32, zipf=1.1, layout="paged", share=(8, 768), seed=6),
    # the same with the index cache in NVFP4
    # 64 requests sharing one 96K-token prompt prefix in a single group: each
    # shared page read and converted once for all 64 (256 (request, group)
    # index queries)
    "shared_b64_128k": dict(seq_lens=[131072] * 64, zipf=1.1, layout="paged", share=(64, 768), seed=7),
    "shared_b64_128k_nvfp4_idx": dict(seq_lens=[131072] * 64, zipf=1.1, layout="paged", share=(64, 768),
                                      idx_dtype="nvfp4", seed=7),
    "shared_b32_128k_nvfp4_idx": dict(seq_lens=[131072] * 32, zipf=1.1, layout="paged", share=(8, 768),
                                      idx_dtype="nvfp4", seed=6),
    # the same with the index cache in NVFP4: the AMD serving setting of the
    # pages (NVFP4 indexer cache and 3 draft tokens)
    "spec_b32_q4_128k_nvfp4_idx": dict(seq_lens=[131072 + 4] * 32, q_len=4, zipf=1.1, layout="paged",
                                       idx_dtype="nvfp4", seed=5),
    # the multi-query verify chunk with the index cache in NVFP4; not one of
    # the five above
    "verify_b2_q256_128k_nvfp4_idx": dict(seq_lens=[131072 + 256] * 2, q_len=256, zipf=1.1, layout="paged",
                                          shared_bias_iq=True, idx_dtype="nvfp4", seed=4),
    # the batch-32 x 128K shape with the index cache in NVFP4 (72 B per token
    # instead of 128 B), the M3.1 production setting; not one of the five above
    "paged_b32_128k_nvfp4_idx": dict(seq_lens=[131072] * 32, zipf=1.1, layout="paged", idx_dtype="nvfp4",
                                     seed=2),
}


def make_config(name: str, device="cpu", **over) -> Workload:
    kw = dict(CONFIGS[name])
    kw.update(over)
    return make_workload(name=name, device=device, **kw)
