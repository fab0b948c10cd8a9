"""Thin ctypes binding of the C ABI in include/msa.h (libmsa.so).

Argument marshalling only: torch tensors are passed as raw device pointers and
torch's current HIP stream as the stream; every step of the path runs in the
HIP kernels.  Importing this module fails loudly if the library is missing —
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MSA_LIB_PATH names another build of the same sources (the
# sanitizer run's instrumented copy)
LIB_PATH = os.environ.get("MSA_LIB_PATH") or os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARGUMENT, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE_TOO_SMALL, MSA_ERR_HIP = range(5)
MSA_KV_BF16, MSA_KV_NVFP4 = 0, 1
MSA_IDX_BF16, MSA_IDX_FP8_E4M3, MSA_IDX_NVFP4 = 0, 1, 2
MSA_SHARE_MAX = 64  # most (member x query token) per prefix-sharing group
_IDX = {"bf16": MSA_IDX_BF16, "fp8": MSA_IDX_FP8_E4M3, "nvfp4": MSA_IDX_NVFP4}
EXPORTED = ("msa_workspace_size", "msa_attn_workspace_size", "msa_indexer_score", "msa_block_topk",
            "msa_sparse_attn_decode", "msa_decode", "msa_kv_insert", "msa_indexer_score_shared", "msa_decode_shared",
            "msa_status_string", "msa_last_error", "msa_decode_noalloc", "msa_block_major_workspace_size",
            "msa_decode_block_major")
MSA_NOALLOC_SCRATCH_BYTES = 32 << 20  # static scratch of msa_decode_noalloc


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)}: {detail}")
        self.status = status


class MsaShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("idx_dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("idx_scale", ctypes.c_float)]

    @classmethod
    def from_workload(cls, w) -> "MsaShape":
        return cls(w.num_seqs, w.q_len, w.num_q_heads, w.num_kv_heads, w.max_blocks_per_seq, w.num_pages,
                   MSA_KV_NVFP4 if w.kv_dtype == "nvfp4" else MSA_KV_BF16,
                   _IDX[w.idx_dtype],
                   w.sm_scale, w.k_scale, w.v_scale, w.idx_scale)


class MsaCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_sf", ctypes.c_void_p), ("v_sf", ctypes.c_void_p),
                ("idx_k", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("idx_sf", ctypes.c_void_p)]

    @classmethod
    def from_tensors(cls, *, k, v, k_sf, v_sf, idx_k, block_table, seq_lens, idx_sf=None) -> "MsaCache":
        for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
            if t.dtype != torch.int32:
                raise TypeError(f"{name} must be int32")
        c = cls(_ptr(k), _ptr(v), _ptr(k_sf), _ptr(v_sf), _ptr(idx_k), _ptr(block_table), _ptr(seq_lens),
                _ptr(idx_sf))
        c._keep = (k, v, k_sf, v_sf, idx_k, block_table, seq_lens, idx_sf)
        return c

    @classmethod
    def from_workload(cls, w) -> "MsaCache":
        return cls.from_tensors(k=w.k, v=w.v, k_sf=w.k_sf, v_sf=w.v_sf, idx_k=w.idx_k, block_table=w.block_table,
                                seq_lens=w.seq_lens, idx_sf=w.idx_sf)


class MsaPrefixShare(ctypes.Structure):
    """Prefix-sharing groups (msa_prefix_share): device int32 arrays; members
    [groups][max_members], its row length is max_members."""
    _fields_ = [("num_groups", ctypes.c_int32), ("max_members", ctypes.c_int32),
                ("min_shared_blocks", ctypes.c_int32), ("members", ctypes.c_void_p),
                ("shared_blocks", ctypes.c_void_p), ("seq_shared_blocks", ctypes.c_void_p)]

    @classmethod
    def from_tensors(cls, *, members, shared_blocks, seq_shared_blocks, min_shared_blocks=0) -> "MsaPrefixShare":
        """min_shared_blocks: a lower bound of seq_shared_blocks over all
        sequences (host-side; 0 is always valid)."""
        for name, t in (("members", members), ("shared_blocks", shared_blocks),
                        ("seq_shared_blocks", seq_shared_blocks)):
            if t.dtype != torch.int32:
                raise TypeError(f"{name} must be int32")
        if members.dim() != 2 or members.shape[0] != shared_blocks.numel():
            raise ValueError("members must be [num_groups][max_members]")
        c = cls(int(shared_blocks.numel()), int(members.shape[1]), int(min_shared_blocks), _ptr(members),
                _ptr(shared_blocks), _ptr(seq_shared_blocks))
        c._keep = (members, shared_blocks, seq_shared_blocks)
        return c

    @classmethod
    def from_workload(cls, w) -> "MsaPrefixShare":
        if w.share_members is None:
            return cls(0, 1, 0, None, None, None)
        return cls.from_tensors(members=w.share_members, shared_blocks=w.share_blocks,
                                seq_shared_blocks=w.seq_shared_blocks,
                                min_shared_blocks=w.meta.get("min_shared_blocks", 0))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_msa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.msa_workspace_size.argtypes = [P(MsaShape)]
        L.msa_workspace_size.restype = ctypes.c_size_t
        L.msa_attn_workspace_size.argtypes = [P(MsaShape)]
        L.msa_attn_workspace_size.restype = ctypes.c_size_t
        L.msa_indexer_score.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp]
        L.msa_block_topk.argtypes = [P(MsaShape), vp, vp, vp, vp]
        L.msa_sparse_attn_decode.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_decode.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_kv_insert.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp, vp]
        L.msa_decode_noalloc.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp, vp, vp]
        L.msa_block_major_workspace_size.argtypes = [P(MsaShape)]
        L.msa_block_major_workspace_size.restype = ctypes.c_size_t
        L.msa_decode_block_major.argtypes = [P(MsaShape), P(MsaCache), vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_indexer_score_shared.argtypes = [P(MsaShape), P(MsaCache), P(MsaPrefixShare), vp, vp, vp]
        L.msa_decode_shared.argtypes = [P(MsaShape), P(MsaCache), P(MsaPrefixShare), vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        for f in ("msa_indexer_score", "msa_block_topk", "msa_sparse_attn_decode", "msa_decode", "msa_kv_insert",
                  "msa_indexer_score_shared", "msa_decode_shared", "msa_decode_noalloc", "msa_decode_block_major"):
            getattr(L, f).restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        L.msa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().msa_status_string(int(st)).decode()


def last_error() -> str:
    return lib().msa_last_error().decode()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(st: int, where: str):
    if st != MSA_OK:
        raise MsaError(st, where, last_error())


def msa_workspace_size(shape: MsaShape) -> int:
    return int(lib().msa_workspace_size(ctypes.byref(shape)))


def msa_attn_workspace_size(shape: MsaShape) -> int:
    return int(lib().msa_attn_workspace_size(ctypes.byref(shape)))


def msa_indexer_score(shape, cache, idx_q, block_scores, stream=None):
    _check(lib().msa_indexer_score(ctypes.byref(shape), ctypes.byref(cache), _ptr(idx_q), _ptr(block_scores),
                                   _stream(stream)), "msa_indexer_score")


def msa_block_topk(shape, seq_lens, block_scores, sel_blocks, stream=None):
    _check(lib().msa_block_topk(ctypes.byref(shape), _ptr(seq_lens), _ptr(block_scores), _ptr(sel_blocks),
                                _stream(stream)), "msa_block_topk")


def msa_sparse_attn_decode(shape, cache, q, sel_blocks, out, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_sparse_attn_decode(ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(sel_blocks),
                                        _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "msa_sparse_attn_decode")


def msa_decode(shape, cache, q, idx_q, out, sel_blocks, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_decode(ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(idx_q), _ptr(out),
                            _ptr(sel_blocks), _ptr(workspace), nbytes, _stream(stream)), "msa_decode")


def msa_block_major_workspace_size(shape: MsaShape) -> int:
    return int(lib().msa_block_major_workspace_size(ctypes.byref(shape)))


def msa_decode_block_major(shape, cache, q, idx_q, out, sel_blocks, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_decode_block_major(ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(idx_q), _ptr(out),
                                        _ptr(sel_blocks), _ptr(workspace), nbytes, _stream(stream)),
           "msa_decode_block_major")


def msa_decode_noalloc(shape, cache, q, idx_q, out, sel_blocks, stream=None):
    """msa_decode with the library's static scratch as its workspace."""
    _check(lib().msa_decode_noalloc(ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(idx_q), _ptr(out),
                                    _ptr(sel_blocks), _stream(stream)), "msa_decode_noalloc")


def msa_indexer_score_shared(shape, cache, share, idx_q, block_scores, stream=None):
    _check(lib().msa_indexer_score_shared(ctypes.byref(shape), ctypes.byref(cache), ctypes.byref(share), _ptr(idx_q),
                                          _ptr(block_scores), _stream(stream)), "msa_indexer_score_shared")


def msa_decode_shared(shape, cache, share, q, idx_q, out, sel_blocks, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().msa_decode_shared(ctypes.byref(shape), ctypes.byref(cache), ctypes.byref(share), _ptr(q),
                                   _ptr(idx_q), _ptr(out), _ptr(sel_blocks), _ptr(workspace), nbytes,
                                   _stream(stream)), "msa_decode_shared")


def msa_kv_insert(shape, cache, k_new, v_new, idx_new, stream=None):
    """Quantises the new tokens into the pools that `cache` points at (written)."""
    _check(lib().msa_kv_insert(ctypes.byref(shape), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(idx_new),
                               _stream(stream)), "msa_kv_insert")


# ---- small conveniences over a synth.Workload (allocation via torch) -------

def alloc_outputs(w):
    dev = w.q.device
    out = torch.empty(w.rows, w.num_q_heads, 128, dtype=torch.float32, device=dev)
    sel = torch.empty(w.rows, w.num_kv_heads, 16, dtype=torch.int32, device=dev)
    return out, sel


def alloc_workspace(shape: MsaShape, device, attn_only: bool = False):
    """Workspace for msa_decode (the fp32 block scores, ...) or, with
    attn_only, for the stand-alone attention (None where it needs none)."""
    n = msa_attn_workspace_size(shape) if attn_only else msa_workspace_size(shape)
    if n == 0:
        if shape.num_seqs > 0 and not attn_only:
            raise MsaError(MSA_ERR_INVALID_ARGUMENT, "workspace size", last_error())
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(w, out=None, sel=None, workspace=None, stream=None):
    """Fused path over a synth.Workload; returns (out, sel)."""
    shape, cache = MsaShape.from_workload(w), MsaCache.from_workload(w)
    if out is None or sel is None:
        out, sel = alloc_outputs(w)
    if workspace is None:
        workspace = alloc_workspace(shape, w.q.device)
    msa_decode(shape, cache, w.q, w.iq, out, sel, workspace, stream)
    return out, sel
