"""ctypes wrapper of the fp64 CPU oracle (oracle/msa_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package; the HIP library never does, and the
two share no code.  The shared object is built by gcc from the one C file
(`build()`), on demand if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_LIB_OVERRIDE = os.environ.get("MSA_ORACLE_LIB")  # another build of msa_oracle.c (the sanitizer run's)
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


IDX_FORMATS = {"bf16": 0, "fp8": 1, "nvfp4": 2}


class _Problem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_nvfp4", ctypes.c_int32), ("idx_fmt", ctypes.c_int32),
                ("sm_scale", ctypes.c_double), ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double),
                ("idx_scale", ctypes.c_double),
                ("q", ctypes.c_void_p), ("iq", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_sf", ctypes.c_void_p), ("v_sf", ctypes.c_void_p), ("idx_k", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("idx_sf", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        lib.msa_oracle_bf16.restype = ctypes.c_double
        lib.msa_oracle_bf16.argtypes = [ctypes.c_uint16]
        lib.msa_oracle_e4m3.restype = ctypes.c_double
        lib.msa_oracle_e4m3.argtypes = [ctypes.c_uint8]
        lib.msa_oracle_e2m1.restype = ctypes.c_double
        lib.msa_oracle_e2m1.argtypes = [ctypes.c_uint8]
        lib.msa_oracle_block_scores.restype = ctypes.c_int
        lib.msa_oracle_block_scores.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.msa_oracle_select.restype = ctypes.c_int
        lib.msa_oracle_select.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.msa_oracle_attend.restype = ctypes.c_int
        lib.msa_oracle_attend.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.msa_oracle_e4m3_rne.restype = ctypes.c_uint8
        lib.msa_oracle_e4m3_rne.argtypes = [ctypes.c_float]
        lib.msa_oracle_e2m1_rne.restype = ctypes.c_uint8
        lib.msa_oracle_bf16_rne.restype = ctypes.c_uint16
        lib.msa_oracle_bf16_rne.argtypes = [ctypes.c_float]
        lib.msa_oracle_e2m1_rne.argtypes = [ctypes.c_float]
        lib.msa_oracle_quant_nvfp4_group.restype = None
        lib.msa_oracle_quant_nvfp4_group.argtypes = [ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        lib.msa_oracle_kv_insert.restype = ctypes.c_int
        lib.msa_oracle_kv_insert.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.msa_oracle_decode.restype = ctypes.c_int
        lib.msa_oracle_decode.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class Problem:
    """Host copy of one workload: numpy arrays of the exact stored bytes."""

    def __init__(self, *, num_seqs, q_len, num_q_heads, num_kv_heads, max_blocks_per_seq, num_pages, kv_dtype,
                 idx_dtype, sm_scale, k_scale, v_scale, idx_scale, q, iq, idx_k, k, v, k_sf, v_sf, block_table,
                 seq_lens, idx_sf=None):
        c = np.ascontiguousarray
        self.arrays = dict(q=c(q), iq=c(iq), idx_k=c(idx_k), k=c(k), v=c(v),
                           k_sf=None if k_sf is None else c(k_sf), v_sf=None if v_sf is None else c(v_sf),
                           idx_sf=None if idx_sf is None else c(idx_sf),
                           block_table=c(block_table, dtype=np.int32), seq_lens=c(seq_lens, dtype=np.int32))
        if idx_dtype == "nvfp4" and idx_sf is None:
            raise ValueError("NVFP4 index keys need their scales (idx_sf)")
        a = self.arrays
        self.num_seqs, self.q_len = int(num_seqs), int(q_len)
        self.num_q_heads, self.num_kv_heads = int(num_q_heads), int(num_kv_heads)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        self.rows = self.num_seqs * self.q_len
        self.sm_scale, self.k_scale = float(sm_scale), float(k_scale)
        self.v_scale, self.idx_scale = float(v_scale), float(idx_scale)
        self._s = _Problem(self.num_seqs, self.q_len, self.num_q_heads, self.num_kv_heads, self.max_blocks_per_seq,
                           int(num_pages), 1 if kv_dtype == "nvfp4" else 0, IDX_FORMATS[idx_dtype],
                           float(sm_scale), float(k_scale), float(v_scale), float(idx_scale),
                           _ptr(a["q"]), _ptr(a["iq"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["k_sf"]),
                           _ptr(a["v_sf"]), _ptr(a["idx_k"]), _ptr(a["block_table"]), _ptr(a["seq_lens"]),
                           _ptr(a["idx_sf"]))

    @classmethod
    def from_workload(cls, w):
        h = w.host_arrays()
        return cls(num_seqs=w.num_seqs, q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                   max_blocks_per_seq=w.max_blocks_per_seq, num_pages=w.num_pages, kv_dtype=w.kv_dtype,
                   idx_dtype=w.idx_dtype, sm_scale=w.sm_scale, k_scale=w.k_scale, v_scale=w.v_scale,
                   idx_scale=w.idx_scale, **h)

    # -- per-step entry points ---------------------------------------------
    def block_scores(self, row: int, g: int):
        """(bs [max_blocks_per_seq] fp64, number of visible blocks)."""
        bs = np.empty(self.max_blocks_per_seq, dtype=np.float64)
        nbv = _load().msa_oracle_block_scores(ctypes.byref(self._s), int(row), int(g), bs.ctypes.data)
        return bs, nbv

    def attend(self, row: int, g: int, sel):
        """out [heads_per_group][128] fp64 over the given selected block ids."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        assert sel.shape == (16,)
        out = np.empty((self.num_q_heads // self.num_kv_heads, 128), dtype=np.float64)
        _load().msa_oracle_attend(ctypes.byref(self._s), int(row), int(g), sel.ctypes.data, out.ctypes.data)
        return out

    def kv_insert(self, k_new, v_new, idx_new):
        """Quantises the new tokens of every query row into this problem's own
        copies of the pools (self.arrays), in place.  k_new, v_new: bf16 bits
        (uint16) [rows][Hkv][128]; idx_new: bf16 bits [rows][128]."""
        def f32(bits):
            return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        kf, vf, xf = f32(k_new), f32(v_new), f32(idx_new)
        assert kf.shape == (self.rows, self.num_kv_heads, 128) and xf.shape == (self.rows, 128)
        _load().msa_oracle_kv_insert(ctypes.byref(self._s), kf.ctypes.data, vf.ctypes.data, xf.ctypes.data)

    def decode(self, row_begin: int = 0, row_end=None, nthreads: int = 0, want_scores: bool = True):
        """Whole path for rows [row_begin, row_end): (bs, sel, out)."""
        row_end = self.rows if row_end is None else int(row_end)
        n = row_end - row_begin
        G, Hq, mb = self.num_kv_heads, self.num_q_heads, self.max_blocks_per_seq
        bs = np.empty((n, G, mb), dtype=np.float64) if want_scores else None
        sel = np.empty((n, G, 16), dtype=np.int32)
        out = np.empty((n, Hq, 128), dtype=np.float64)
        nthreads = nthreads or len(os.sched_getaffinity(0))
        _load().msa_oracle_decode(ctypes.byref(self._s), int(row_begin), int(row_end), _ptr(bs), sel.ctypes.data,
                                  out.ctypes.data, int(nthreads))
        return bs, sel, out


def select(bs, nbv: int):
    """16 selected block ids (ascending, -1 padded) from fp64 block scores."""
    bs = np.ascontiguousarray(bs, dtype=np.float64)
    sel = np.empty(16, dtype=np.int32)
    _load().msa_oracle_select(bs.ctypes.data, int(nbv), sel.ctypes.data)
    return sel


def e4m3_rne(y: float) -> int:
    return int(_load().msa_oracle_e4m3_rne(float(y)))


def e2m1_rne(y: float) -> int:
    return int(_load().msa_oracle_e2m1_rne(float(y)))


def bf16_rne(y: float) -> int:
    """bf16 bits of the float32 value y rounded to nearest, ties to even."""
    return int(_load().msa_oracle_bf16_rne(float(y)))


def quant_nvfp4_group(x16, gs: float):
    """16 float32 values -> (8 packed bytes, scale byte)."""
    x = np.ascontiguousarray(x16, dtype=np.float32)
    assert x.shape == (16,)
    packed = np.zeros(8, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    _load().msa_oracle_quant_nvfp4_group(x.ctypes.data, float(gs), packed.ctypes.data, sc.ctypes.data)
    return packed, int(sc[0])


def e4m3(byte: int) -> float:
    return _load().msa_oracle_e4m3(int(byte))


def e2m1(nibble: int) -> float:
    return _load().msa_oracle_e2m1(int(nibble))


def bf16(bits: int) -> float:
    return _load().msa_oracle_bf16(int(bits))
