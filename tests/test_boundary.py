"""The C-ABI boundary on the CPU: the library loads without a GPU, exports
every function include/msa.h declares, and host-side validation returns its
documented status codes before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_msa_amd import msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(msa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def _shape(**kw):
    d = dict(num_seqs=2, q_len=1, num_q_heads=16, num_kv_heads=4, max_blocks_per_seq=8, num_pages=16,
             kv_dtype=msa.MSA_KV_NVFP4, idx_dtype=msa.MSA_IDX_FP8_E4M3, sm_scale=0.088, k_scale=1.0, v_scale=1.0,
             idx_scale=1.0)
    d.update(kw)
    return msa.MsaShape(*[d[f] for f, _ in msa.MsaShape._fields_])


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def _cache(**kw):
    d = dict(k=FAKE, v=FAKE, k_sf=FAKE, v_sf=FAKE, idx_k=FAKE, block_table=FAKE, seq_lens=FAKE, idx_sf=FAKE)
    d.update(kw)
    return msa.MsaCache(*[d[f] for f, _ in msa.MsaCache._fields_])


def _decode(shape, cache=None, q=FAKE, iq=FAKE, out=FAKE, sel=FAKE, ws=FAKE, nbytes=1 << 30):
    L = msa.lib()
    cache = cache or _cache()
    return L.msa_decode(ctypes.byref(shape) if shape is not None else None, ctypes.byref(cache), q, iq, out, sel, ws,
                        nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=8), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_kv_heads=2), msa.MSA_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), msa.MSA_ERR_UNSUPPORTED),
    (dict(idx_dtype=5), msa.MSA_ERR_UNSUPPORTED),
    (dict(q_len=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_seqs=-1), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(max_blocks_per_seq=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(max_blocks_per_seq=16385), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(sm_scale=0.0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(k_scale=float("nan")), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(idx_scale=-1.0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(q_len=2000, max_blocks_per_seq=8), msa.MSA_ERR_INVALID_ARGUMENT),
])
def test_shape_validation(kw, code):
    assert _decode(_shape(**kw)) == code
    assert msa.last_error() != ""
    assert msa.lib().msa_workspace_size(ctypes.byref(_shape(**kw))) == 0  # invalid shapes have no size


def test_null_and_pointer_validation():
    L = msa.lib()
    assert L.msa_decode(None, ctypes.byref(_cache()), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == \
        msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), q=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), iq=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), out=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), cache=_cache(k_sf=None)) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), cache=_cache(idx_k=None)) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), cache=_cache(block_table=None)) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), ws=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert _decode(_shape(), q=FAKE + 2) == msa.MSA_ERR_INVALID_ARGUMENT        # misaligned
    assert _decode(_shape(), ws=FAKE + 16) == msa.MSA_ERR_INVALID_ARGUMENT      # workspace not 256-B aligned
    # bf16 K/V needs no scale arrays; validation then proceeds to the workspace check
    assert _decode(_shape(kv_dtype=msa.MSA_KV_BF16), cache=_cache(k_sf=None, v_sf=None), nbytes=0) == \
        msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_scale_arrays_must_be_16_byte_aligned():
    """The E4M3 group-scale arrays are read with 16-byte loads: a misaligned
    k_sf / v_sf (NVFP4 K/V) or idx_sf (NVFP4 index keys) is rejected by every
    entry point that reads or writes it, before any HIP call; with bf16 K/V or
    FP8 index keys the arrays are not used and their alignment is free."""
    L = msa.lib()
    nv_idx = _shape(idx_dtype=msa.MSA_IDX_NVFP4)
    cases = [(_shape(), dict(k_sf=FAKE + 4), "k_sf"), (_shape(), dict(v_sf=FAKE + 1), "v_sf"),
             (nv_idx, dict(idx_sf=FAKE + 8), "idx_sf")]
    for s, kw, name in cases:
        c = _cache(**kw)
        assert _decode(s, cache=c) == msa.MSA_ERR_INVALID_ARGUMENT and name in msa.last_error()
        assert L.msa_kv_insert(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, None) == \
            msa.MSA_ERR_INVALID_ARGUMENT and name in msa.last_error()
        if name == "idx_sf":
            assert L.msa_indexer_score(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, None) == \
                msa.MSA_ERR_INVALID_ARGUMENT and name in msa.last_error()
        else:
            assert L.msa_sparse_attn_decode(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, FAKE, None, 0, None) == \
                msa.MSA_ERR_INVALID_ARGUMENT and name in msa.last_error()
    # unused arrays: validation proceeds to the workspace check
    assert _decode(_shape(kv_dtype=msa.MSA_KV_BF16), cache=_cache(k_sf=FAKE + 4, v_sf=FAKE + 2, idx_sf=FAKE + 1),
                   nbytes=0) == msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_nvfp4_index_keys_validation():
    """NVFP4 index keys need their scale array; every q_len takes them."""
    s = _shape(idx_dtype=msa.MSA_IDX_NVFP4)
    assert _decode(s, cache=_cache(idx_sf=None)) == msa.MSA_ERR_INVALID_ARGUMENT
    assert "idx_sf" in msa.last_error()
    assert msa.lib().msa_workspace_size(ctypes.byref(_shape(idx_dtype=msa.MSA_IDX_NVFP4, q_len=9))) > 0
    assert msa.lib().msa_workspace_size(ctypes.byref(_shape(idx_dtype=msa.MSA_IDX_NVFP4, q_len=256))) > 0
    assert msa.lib().msa_workspace_size(ctypes.byref(_shape(idx_dtype=msa.MSA_IDX_NVFP4, q_len=8))) > 0


def test_prefix_share_validation():
    """The shared entry points: a NULL descriptor, a negative group count, a
    missing array or a member row length outside 1..64 is INVALID_ARGUMENT;
    sharing beyond q_len 8, with bf16 index keys, or with more than 64 (member
    x query token) columns per group is UNSUPPORTED; FP8 and NVFP4 keys at
    q_len 1..8 within the limit pass on to the next check (here the short
    workspace), and so do zero groups (the unshared call)."""
    L = msa.lib()
    s = _shape()
    sh = msa.MsaPrefixShare(2, 8, 0, FAKE, FAKE, FAKE)

    def dec(shape, share, nbytes=1 << 30):
        return L.msa_decode_shared(ctypes.byref(shape), ctypes.byref(_cache()), share, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   nbytes, None)

    assert dec(s, None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert dec(s, ctypes.byref(msa.MsaPrefixShare(-1, 8, 0, FAKE, FAKE, FAKE))) == msa.MSA_ERR_INVALID_ARGUMENT
    assert dec(s, ctypes.byref(msa.MsaPrefixShare(2, 8, 0, None, FAKE, FAKE))) == msa.MSA_ERR_INVALID_ARGUMENT
    assert "members" in msa.last_error()
    for bad in (0, -3, 65):
        assert dec(s, ctypes.byref(msa.MsaPrefixShare(2, bad, 0, FAKE, FAKE, FAKE))) == msa.MSA_ERR_INVALID_ARGUMENT
        assert "max_members" in msa.last_error()
    assert dec(_shape(q_len=9, max_blocks_per_seq=8), ctypes.byref(sh)) == msa.MSA_ERR_UNSUPPORTED
    assert dec(_shape(q_len=9), ctypes.byref(msa.MsaPrefixShare(2, 1, 0, FAKE, FAKE, FAKE))) == msa.MSA_ERR_UNSUPPORTED
    assert dec(_shape(q_len=4), ctypes.byref(msa.MsaPrefixShare(2, 17, 0, FAKE, FAKE, FAKE))) == msa.MSA_ERR_UNSUPPORTED
    assert dec(_shape(idx_dtype=msa.MSA_IDX_BF16), ctypes.byref(sh)) == msa.MSA_ERR_UNSUPPORTED
    for idx in (msa.MSA_IDX_FP8_E4M3, msa.MSA_IDX_NVFP4):
        assert dec(_shape(idx_dtype=idx), ctypes.byref(sh), nbytes=16) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
        for q_len, mm in ((1, 64), (2, 32), (4, 16), (8, 8)):
            share = msa.MsaPrefixShare(2, mm, 0, FAKE, FAKE, FAKE)
            assert dec(_shape(idx_dtype=idx, q_len=q_len), ctypes.byref(share), nbytes=16) == \
                msa.MSA_ERR_WORKSPACE_TOO_SMALL, (idx, q_len, mm, msa.last_error())
    for bad in (-1, 8):  # min_shared_blocks outside [0, max_blocks_per_seq)
        assert dec(s, ctypes.byref(msa.MsaPrefixShare(2, 8, bad, FAKE, FAKE, FAKE))) == msa.MSA_ERR_INVALID_ARGUMENT
        assert "min_shared_blocks" in msa.last_error()
    assert dec(s, ctypes.byref(msa.MsaPrefixShare(0, 1, 0, None, None, None)), nbytes=16) == \
        msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert L.msa_indexer_score_shared(ctypes.byref(s), ctypes.byref(_cache()), None, FAKE, FAKE, None) == \
        msa.MSA_ERR_INVALID_ARGUMENT


def test_kv_insert_validation():
    """msa_kv_insert validates like the other entry points, before any HIP call."""
    L = msa.lib()
    ins = lambda s, c=None, k=FAKE, v=FAKE, x=FAKE: L.msa_kv_insert(ctypes.byref(s), ctypes.byref(c or _cache()), k, v,
                                                                     x, None)
    assert ins(_shape(), k=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert ins(_shape(), x=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert ins(_shape(), k=FAKE + 4) == msa.MSA_ERR_INVALID_ARGUMENT          # misaligned
    assert ins(_shape(), c=_cache(v_sf=None)) == msa.MSA_ERR_INVALID_ARGUMENT
    assert ins(_shape(num_kv_heads=2)) == msa.MSA_ERR_UNSUPPORTED
    assert ins(_shape(num_seqs=0)) == msa.MSA_OK


def test_workspace_size_and_too_small():
    L = msa.lib()
    s = _shape(num_seqs=32, max_blocks_per_seq=1024)
    need = L.msa_workspace_size(ctypes.byref(s))
    scores = 32 * 4 * 1024 * 4
    assert need >= scores and need % 256 == 0
    assert _decode(s, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in msa.last_error()
    ids = 32 * 4 * 16 * 4
    assert need == scores + ids  # the block scores, then the selected ids (256-B aligned each)
    assert L.msa_attn_workspace_size(ctypes.byref(s)) == 0


def test_empty_batch_is_a_no_op():
    """num_seqs == 0 returns MSA_OK without launching anything."""
    L = msa.lib()
    s = _shape(num_seqs=0)
    assert _decode(s, ws=None, nbytes=0) == msa.MSA_OK
    assert L.msa_indexer_score(ctypes.byref(s), ctypes.byref(_cache()), FAKE, FAKE, None) == msa.MSA_OK
    assert L.msa_block_topk(ctypes.byref(s), FAKE, FAKE, FAKE, None) == msa.MSA_OK
    assert msa.last_error() == ""


def test_other_entry_points_validate():
    L = msa.lib()
    s = _shape()
    assert L.msa_indexer_score(ctypes.byref(s), ctypes.byref(_cache()), None, FAKE, None) == \
        msa.MSA_ERR_INVALID_ARGUMENT
    rows = 2 * 256  # multi-query rows: scores [rows][4][8 blocks] + ids [rows][4][16]
    assert L.msa_workspace_size(ctypes.byref(_shape(q_len=256))) == rows * 4 * 8 * 4 + rows * 4 * 16 * 4
    assert L.msa_block_topk(ctypes.byref(s), None, FAKE, FAKE, None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert L.msa_sparse_attn_decode(ctypes.byref(s), ctypes.byref(_cache(v=None)), FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == msa.MSA_ERR_INVALID_ARGUMENT
    for st in range(5):
        assert msa.status_string(st).startswith("MSA_")


def test_kept_block_split_workspace():
    """bf16 K/V and at most 64 (row, group) pairs: msa_decode's workspace adds
    the split's partials (2,080 B per (pair, kept block)) and one int32
    arrival counter per pair after the scores and ids, 256-B aligned, and the
    stand-alone attention then needs the same region as its workspace.  NVFP4
    K/V merge on chip: no partials."""
    L = msa.lib()

    def split_region(pairs):
        return -(-(pairs * 16 * 2080 + pairs * 4) // 256) * 256

    nv = _shape(num_seqs=2, max_blocks_per_seq=8)  # NVFP4 K/V, 8 pairs
    assert L.msa_attn_workspace_size(ctypes.byref(nv)) == 0
    assert L.msa_workspace_size(ctypes.byref(nv)) == 256 + 512
    s = _shape(num_seqs=2, max_blocks_per_seq=8, kv_dtype=msa.MSA_KV_BF16)  # 8 pairs
    parts = split_region(8)
    assert parts == 266496
    assert L.msa_attn_workspace_size(ctypes.byref(s)) == parts
    assert L.msa_workspace_size(ctypes.byref(s)) == 256 + 512 + parts
    s16 = _shape(num_seqs=16, max_blocks_per_seq=8, kv_dtype=msa.MSA_KV_BF16)  # 64 pairs: the largest split batch
    assert L.msa_attn_workspace_size(ctypes.byref(s16)) == split_region(64)
    s17 = _shape(num_seqs=17, max_blocks_per_seq=8, kv_dtype=msa.MSA_KV_BF16)
    assert L.msa_attn_workspace_size(ctypes.byref(s17)) == 0

    def attn(ws, nbytes, out=FAKE):
        return L.msa_sparse_attn_decode(ctypes.byref(s), ctypes.byref(_cache()), FAKE, FAKE, out, ws, nbytes, None)

    assert attn(None, 0) == msa.MSA_ERR_INVALID_ARGUMENT and "workspace" in msa.last_error()
    assert attn(FAKE, parts - 1) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert attn(FAKE + 64, parts) == msa.MSA_ERR_INVALID_ARGUMENT
    assert attn(FAKE, parts, out=FAKE + 4) == msa.MSA_ERR_INVALID_ARGUMENT and "out" in msa.last_error()
    assert _decode(s, out=FAKE + 4) == msa.MSA_ERR_INVALID_ARGUMENT and "out" in msa.last_error()


def test_block_major_validation():
    """msa_decode_block_major: NVFP4 K/V, q_len <= 256 and tables of at most
    8,192 blocks only; 16-B aligned out; a workspace of
    msa_block_major_workspace_size() bytes (0 for an unsupported shape)."""
    L = msa.lib()

    def dec(shape, out=FAKE, ws=FAKE, nbytes=1 << 30):
        return L.msa_decode_block_major(ctypes.byref(shape), ctypes.byref(_cache()), FAKE, FAKE, out, FAKE, ws,
                                        nbytes, None)

    for kw in (dict(kv_dtype=msa.MSA_KV_BF16), dict(q_len=257), dict(max_blocks_per_seq=8193)):
        s = _shape(**kw)
        assert dec(s) == msa.MSA_ERR_UNSUPPORTED, kw
        assert L.msa_block_major_workspace_size(ctypes.byref(s)) == 0
    s = _shape(q_len=256, max_blocks_per_seq=1024)
    need = L.msa_block_major_workspace_size(ctypes.byref(s))
    assert need > L.msa_workspace_size(ctypes.byref(s)) and need % 256 == 0
    assert dec(s, out=FAKE + 8) == msa.MSA_ERR_INVALID_ARGUMENT and "out" in msa.last_error()
    assert dec(s, ws=None) == msa.MSA_ERR_INVALID_ARGUMENT
    assert dec(s, ws=FAKE + 16) == msa.MSA_ERR_INVALID_ARGUMENT
    assert dec(s, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert dec(_shape(num_seqs=0), ws=None, nbytes=0) == msa.MSA_OK


def test_read_ceiling_library_exports_and_validates():
    """The benchmark's read-ceiling kernel library (not part of the MSA path)
    loads, exports its entry point and rejects bad arguments before any HIP
    call."""
    path = os.path.join(os.path.dirname(msa.LIB_PATH), "libmsa_ceiling.so")
    lib = ctypes.CDLL(path)
    fn = lib.msa_ceiling_read_pages
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    assert fn(None, 16, None, 0, fake, fake, None, 1, 1, fake, None) == -1       # no pool
    assert fn(fake, 16, fake, 0, fake, fake, None, 1, 1, fake, None) == -1       # pool1 without kb1
    assert fn(fake, 8, None, 1, fake, fake, None, 1, 1, fake, None) == -1        # kb1 without pool1
    assert fn(fake, 12, None, 0, fake, fake, None, 1, 1, fake, None) == -1       # unsupported page size
    assert fn(fake, 16, None, 0, fake, fake, None, 0, 1, fake, None) == -1       # no sequences
    assert fn(fake, 16, None, 0, fake, fake, None, 70000, 1, fake, None) == -1   # grid rows past 65535


def test_binding_constants_match_header():
    """The binding's enum values and limits are the header's."""
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "msa.h")).read()
    defines = dict(re.findall(r"#define (MSA_[A-Z_]+) (\d+)", hdr))
    assert int(defines["MSA_SHARE_MAX"]) == msa.MSA_SHARE_MAX
    for name in ("MSA_KV_BF16", "MSA_KV_NVFP4", "MSA_IDX_BF16", "MSA_IDX_FP8_E4M3", "MSA_IDX_NVFP4", "MSA_OK",
                 "MSA_ERR_INVALID_ARGUMENT", "MSA_ERR_UNSUPPORTED", "MSA_ERR_WORKSPACE_TOO_SMALL", "MSA_ERR_HIP"):
        m = re.search(name + r" = (\d+)", hdr)
        assert m and int(m.group(1)) == getattr(msa, name), name


def test_header_compiles_as_c_and_links(tmp_path):
    """include/msa.h as a C99 caller sees it: a C program that includes it
    compiles with warnings as errors, links against libmsa.so and gets the
    same workspace size as the binding for the headline shape (host-only
    entry points: no GPU is touched)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "msa.h"
int main(void) {
  msa_shape s = {32, 1, MSA_NUM_Q_HEADS, MSA_NUM_KV_HEADS, 1024, 32768, MSA_KV_NVFP4, MSA_IDX_FP8_E4M3,
                 0.08838834764831845f, 1.0f, 1.0f, 1.0f};
  size_t ws = msa_workspace_size(&s);
  msa_shape bad = s;
  bad.num_q_heads = 3;
  size_t none = msa_workspace_size(&bad);
  printf("%zu %zu %s %s\n", ws, none, msa_status_string(MSA_OK), msa_status_string(MSA_ERR_INVALID_ARGUMENT));
  return ws > 0 && none == 0 ? 0 : 1;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(msa.LIB_PATH)
    include = os.path.join(os.path.dirname(libdir), "include")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    # the header takes hipStream_t from the HIP runtime API header, which a C
    # compiler reads with the platform macro set
    subprocess.check_call([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", include,
                           "-I", os.path.join(rocm, "include"), str(src), "-o", str(exe), msa.LIB_PATH,
                           f"-Wl,-rpath,{libdir}"])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    shape = msa.MsaShape(32, 1, 16, 4, 1024, 32768, msa.MSA_KV_NVFP4, msa.MSA_IDX_FP8_E4M3, 0.08838834764831845,
                         1.0, 1.0, 1.0)
    assert int(out[0]) == msa.msa_workspace_size(shape)
    assert out[1:] == ["0", "MSA_OK", "MSA_ERR_INVALID_ARGUMENT"]
