"""Test-side helpers that rebuild dense fp64 tensors from the stored bytes with
*library* routines (torch's FP8 cast, the OCP E2M1 table from tests/golden),
independently of the oracle's C decoders, so oracle results can be compared
with torch's SDPA / amax / matmul."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
E2M1_TABLE = torch.tensor(json.load(open(os.path.join(GOLDEN, "e2m1_ocp.json")))["codes_to_value"],
                          dtype=torch.float64)
BYTE_MODEL = json.load(open(os.path.join(GOLDEN, "byte_model.json")))


def e4m3_t(u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u8)).view(torch.float8_e4m3fn).to(torch.float64)


def bf16_t(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def nvfp4_t(packed: np.ndarray, scales: np.ndarray, tensor_scale: float) -> torch.Tensor:
    """[..., 64] packed + [..., 8] E4M3 scales -> fp64 [..., 128]."""
    p = torch.from_numpy(np.ascontiguousarray(packed)).to(torch.int64)
    lo, hi = p & 15, p >> 4
    codes = torch.stack([lo, hi], dim=-1).reshape(*p.shape[:-1], 128)
    vals = E2M1_TABLE[codes]
    sc = e4m3_t(scales).repeat_interleave(16, dim=-1)
    return vals * sc * tensor_scale


def nvfp4_v_t(packed_t: np.ndarray, scales: np.ndarray, tensor_scale: float) -> torch.Tensor:
    """V pages as stored, [..., 128 dims, 64] (row d: the 128 tokens' dim d,
    token 2i in the low nibble of byte i) + [..., 128 tokens, 8] E4M3 scales
    -> fp64 [..., 128 tokens, 128 dims]."""
    p = torch.from_numpy(np.ascontiguousarray(packed_t)).to(torch.int64)
    lo, hi = p & 15, p >> 4
    codes = torch.stack([lo, hi], dim=-1).reshape(*p.shape[:-1], 128).transpose(-1, -2)   # [..., tok, dim]
    vals = E2M1_TABLE[codes]
    sc = e4m3_t(scales).repeat_interleave(16, dim=-1)
    return vals * sc * tensor_scale


def dense_seq(P, b: int):
    """Logical-order fp64 tensors of sequence b: idx [L,128], K [G,L,128], V [G,L,128]."""
    a = P.arrays
    L = int(a["seq_lens"][b])
    nb = (L - 1) // 128 + 1 if L > 0 else 0
    pages = a["block_table"][b, :nb].astype(np.int64)
    if a.get("idx_sf") is not None:
        idx = nvfp4_t(a["idx_k"][pages], a["idx_sf"][pages], P.idx_scale)
    elif a["idx_k"].dtype == np.uint8:
        idx = e4m3_t(a["idx_k"][pages]) * P.idx_scale
    else:
        idx = bf16_t(a["idx_k"][pages]) * P.idx_scale
    idx = idx.reshape(nb * 128, 128)[:L]
    if a["k_sf"] is not None:
        K = nvfp4_t(a["k"][pages], a["k_sf"][pages], P.k_scale)
        V = nvfp4_v_t(a["v"][pages], a["v_sf"][pages], P.v_scale)
    else:
        K = bf16_t(a["k"][pages]) * P.k_scale
        V = bf16_t(a["v"][pages]) * P.v_scale
    G = K.shape[1]
    K = K.permute(1, 0, 2, 3).reshape(G, nb * 128, 128)[:, :L]
    V = V.permute(1, 0, 2, 3).reshape(G, nb * 128, 128)[:, :L]
    return idx, K, V


def row_queries(P, row: int):
    a = P.arrays
    return bf16_t(a["q"][row]), bf16_t(a["iq"][row])


def make_problem(w):
    import oracle
    return oracle.Problem.from_workload(w)
