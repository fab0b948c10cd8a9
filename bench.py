#!/usr/bin/env python3
"""Bench of the fused MSA decode step on one MI355X.

One step = one call of msa_decode (index scan + block max-pool, top-16 with
the recent block, sparse GQA attention over NVFP4 K/V) for the whole batch:
batch 32, 128K-token contexts, paged pool with a random block table, FP8 index
keys (the headline workload).  Inputs are resident in HBM before timing; the
steps rotate through copies of the inputs, enough of them that more than
1.25 x the 256 MB Infinity Cache of other inputs is read between two uses of
one copy, so that no step reads what an earlier one left in that cache.

Prints ONE JSON line.  Extra detail goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "MSA decode µs/layer-step + achieved HBM GB/s (%peak), 128K ctx, batch 32"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def scan_bytes(w) -> float:
    """Algorithmic bytes of one index-scan launch: every visible token's index
    key, the used block-table entries, the index queries, the block scores."""
    lens = [int(x) for x in w.seq_lens.cpu().tolist()]
    nbs = [((L - 1) // 128 + 1) if L > 0 else 0 for L in lens]
    # index keys: every visible token's, a shared-prefix page once for its group
    return (w.nbytes_algorithmic()["scan"] + sum(nbs) * 4 + w.rows * w.num_kv_heads * 128 * 2
            + w.rows * w.num_kv_heads * w.max_blocks_per_seq * 4)


def scan_flops(w) -> float:
    """Algorithmic flops of one multi-query index scan: 2 x 128 per (row,
    group, visible key) pair; row i of sequence b sees its tokens at or before
    position seq_lens[b] - q_len + i."""
    total = 0
    for L in [int(x) for x in w.seq_lens.cpu().tolist()]:
        if L <= 0:
            continue
        first = L - w.q_len + 1                      # keys visible to query 0
        total += w.num_kv_heads * (w.q_len * first + w.q_len * (w.q_len - 1) // 2)
    return 2.0 * 128 * total


CEILING_LIB = os.path.join(ROOT, "block_sparse_attention_msa_amd", "libmsa_ceiling.so")


def read_ceiling(w, copies, stream, steps: int, warmup: int):
    """The practical HBM ceiling of the index scan on this machine: a read-only
    kernel (libmsa_ceiling.so) walks the same index-key pages through the same
    block table with the scan's load pattern and computes nothing.  Returns
    (us per launch, bytes read per launch), or None where the scan is not a
    page stream (more than 8 query rows per sequence: the multi-query scan)."""
    import ctypes
    import torch
    if w.q_len > 8:
        return None
    kb0, kb1 = {"fp8": (16, 0), "bf16": (32, 0), "nvfp4": (8, 1)}[w.idx_dtype]
    lib = ctypes.CDLL(CEILING_LIB)
    fn = lib.msa_ceiling_read_pages
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lens = [int(x) for x in w.seq_lens.cpu().tolist()]
    first = [0] * w.num_seqs
    if w.seq_shared_blocks is not None:  # a shared page once, by its group's leader
        leaders = set(int(m[0]) for m in w.share_members.cpu().tolist())
        first = [0 if b in leaders else int(x) for b, x in enumerate(w.seq_shared_blocks.cpu().tolist())]
    first_t = torch.tensor(first, dtype=torch.int32, device=w.seq_lens.device)
    pages = sum(max(0, min((L + 127) // 128, w.max_blocks_per_seq) - f) for L, f in zip(lens, first))
    sink = torch.zeros(1, dtype=torch.int32, device=w.seq_lens.device)
    for c in copies:  # the pools hold exactly kb0 (kb1) KiB per page
        assert c.idx_k.is_contiguous() and c.idx_k.numel() * c.idx_k.element_size() == w.num_pages * kb0 * 1024
        assert kb1 == 0 or c.idx_sf.numel() * c.idx_sf.element_size() == w.num_pages * kb1 * 1024
        assert tuple(c.block_table.shape) == (w.num_seqs, w.max_blocks_per_seq) and c.block_table.is_contiguous()

    def launch(i):
        c = copies[i % len(copies)]
        rc = fn(c.idx_k.data_ptr(), kb0, c.idx_sf.data_ptr() if kb1 else None, kb1, c.block_table.data_ptr(),
                c.seq_lens.data_ptr(), first_t.data_ptr(), w.num_seqs, w.max_blocks_per_seq, sink.data_ptr(),
                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"msa_ceiling_read_pages failed: {rc}")

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3, pages * (kb0 + kb1) * 1024


MALL_BYTES = 256 << 20   # MI355X Infinity Cache


def auto_copies(w) -> int:
    """Input copies for the step rotation: between two uses of one copy the
    other copies' step bytes (at least 1.25 x the Infinity Cache) pass
    through, so a step never finds its inputs there; 2 to 64."""
    import math
    step = w.nbytes_algorithmic()["total"]
    return max(2, min(64, 1 + math.ceil(1.25 * MALL_BYTES / step)))


def clone_workload(w):
    import copy
    w2 = copy.copy(w)
    for name in ("q", "iq", "idx_k", "idx_sf", "k", "v", "k_sf", "v_sf", "block_table", "seq_lens",
                 "share_members", "share_blocks", "seq_shared_blocks"):
        t = getattr(w, name)
        setattr(w2, name, None if t is None else t.clone())
    return w2


def cpu_baseline(w, sample_seqs: int, t_gpu_us: float):
    import oracle
    P = oracle.Problem.from_workload(w)
    cores = len(os.sched_getaffinity(0))
    if w.q_len == 1:
        n = min(sample_seqs, w.num_seqs)
        rows, what = n, f"{n} of {w.num_seqs} sequences (rows 0-{n - 1})"
    else:  # multi-query rows each scan the whole context: a few rows bound the CPU time
        rows = min(16, w.rows)
        what = f"{rows} of {w.rows} query rows (rows 0-{rows - 1})"
    t0 = time.perf_counter()
    P.decode(0, rows, nthreads=cores, want_scores=False)
    dt = time.perf_counter() - t0
    scaled_us = dt * 1e6 * (w.rows / rows)
    return {"value": round(scaled_us, 1), "unit": "us/layer-step", "cores": cores, "kind": "oracle",
            "sample": f"{what}, full {int(w.seq_lens[0])}-token context each, fp64 C oracle with OpenMP over "
                      f"(row, group); wall {dt:.2f} s scaled by {w.rows / rows:g} to the whole step; "
                      f"CPU: {cpu_model()}",
            "gpu_speedup": round(scaled_us / t_gpu_us, 1)}


COPY_BYTES = 512 << 20
SCAN_SOURCES = ("indexer_scan.hip", "scan_device.hpp", "msa_device.hpp", "msa_kernels.hpp")


def traffic_file(config: str) -> str:
    return os.path.join(ROOT, "profiles", f"scan_{config}_traffic.json")


def scan_source_hash() -> str:
    """Hash of the scan kernels' sources and of the compiler flags they are
    built with: a traffic record stays valid only for the same code."""
    import hashlib
    from block_sparse_attention_msa_amd import build as hip_build
    h = hashlib.sha256()
    for name in SCAN_SOURCES:
        h.update(open(os.path.join(ROOT, "block_sparse_attention_msa_amd", "csrc", name), "rb").read())
        if name.endswith(".hip"):
            # flags as written, with the checkout's own path taken out (the
            # include directory is absolute and differs between machines)
            flags = [f.replace(hip_build.ROOT, "<root>") for f in hip_build.FLAGS + hip_build.FILE_FLAGS.get(name, [])]
            h.update(" ".join(flags).encode())
    return h.hexdigest()


def scan_traffic(config: str):
    """HBM bytes per scan launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (each scaled by what the counter read for a plain copy of
    known size), or None if there are none or the scan's sources changed since."""
    try:
        rec = json.load(open(traffic_file(config)))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != scan_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _counter_means(run_dir: str, counter: str):
    """{kernel name: (mean counter value per dispatch, dispatches)} from a
    rocprofv3 --pmc CSV run directory."""
    import csv
    import glob
    sums = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            k = r["Kernel_Name"]
            v, n = sums.get(k, (0.0, 0))
            sums[k] = (v + float(r["Counter_Value"]), n + 1)
    return {k: (v / n, n) for k, (v, n) in sums.items()}


def write_traffic(config: str, fetch_dir: str, write_dir: str):
    """Turns the FETCH_SIZE and WRITE_SIZE runs of `--mode counters` into the
    traffic record of the config's scan: each counter is scaled by what it
    read for the plain copy of COPY_BYTES in the same runs."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    # the scan's kernels (two with prefix sharing: the sequences' own blocks,
    # then the shared ones), each dispatched once per scan call
    scans = sorted(k for k in fetch if re.search(r"scan_(decode|cols|shared)", k))
    if not scans or len({fetch[k][1] for k in scans}) != 1 or any(k not in write for k in scans):
        raise SystemExit(f"expected the scan kernels once per call in {fetch_dir}, found {scans}")
    n = fetch[scans[0]][1]
    # the calibration kernel: torch's negation of COPY_BYTES, once per scan call
    copy = [k for k in write if "neg" in k.lower() and k in fetch and write[k][1] == n]
    if len(copy) != 1:
        raise SystemExit(f"expected one calibration kernel in {write_dir}, found {copy}")
    copy = copy[0]
    fs, ws = COPY_BYTES / (fetch[copy][0] * 1024.0), COPY_BYTES / (write[copy][0] * 1024.0)
    fraw, wraw = sum(fetch[k][0] for k in scans), sum(write[k][0] for k in scans)
    fb, wb = fraw * 1024.0 * fs, wraw * 1024.0 * ws
    names = [re.search(r"scan_(?:decode|cols|shared)\w*(?:<[^>]*>)?", k).group(0) for k in scans]
    rec = {"kernel": " + ".join(names), "workload": config, "source_sha256": scan_source_hash(),
           "fetch_kib_per_dispatch_raw": fraw, "write_kib_per_dispatch_raw": wraw,
           "copy_fetch_kib_raw": fetch[copy][0], "copy_write_kib_raw": write[copy][0], "copy_bytes": COPY_BYTES,
           "fetch_scale": fs, "write_scale": ws, "fetch_bytes": fb, "write_bytes": wb,
           "bytes_per_launch": int(round(fb + wb)), "dispatches": n}
    with open(traffic_file(config), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def scan_call(msa, shape, cache, c, bs, stream):
    """The index scan of workload copy c (the shared-prefix call when it has groups)."""
    if c.share_members is not None:
        msa.msa_indexer_score_shared(shape, cache, msa.MsaPrefixShare.from_workload(c), c.iq, bs, stream)
    else:
        msa.msa_indexer_score(shape, cache, c.iq, bs, stream)


def decode_call(msa, shape, cache, c, out, sel, ws, stream, block_major: bool = False):
    """One msa_decode step of workload copy c (msa_decode_shared when it has
    groups, msa_decode_block_major when asked for)."""
    if block_major:
        msa.msa_decode_block_major(shape, cache, c.q, c.iq, out, sel, ws, stream)
    elif c.share_members is not None:
        msa.msa_decode_shared(shape, cache, msa.MsaPrefixShare.from_workload(c), c.q, c.iq, out, sel, ws, stream)
    else:
        msa.msa_decode(shape, cache, c.q, c.iq, out, sel, ws, stream)


def run_counter_pass(args, w, copies, shape, caches):
    """Launches for hardware-counter runs: the index scan (steps x) and a plain
    streaming kernel over COPY_BYTES (torch's negation: reads and writes
    COPY_BYTES, steps x) whose FETCH_SIZE / WRITE_SIZE per dispatch calibrate
    the counters against a known byte count."""
    import torch
    from block_sparse_attention_msa_amd import msa
    dev = w.q.device
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for i in range(args.steps):
        c = copies[i % len(copies)]
        scan_call(msa, shape, caches[i % len(copies)], c, bs, None)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] counters pass: {args.steps} scan launches ({scan_bytes(w)} algorithmic B each), "
        f"{args.steps} copies of {COPY_BYTES} B")


OTHER_CONFIGS = ("tiny_b1_4k_bf16", "decode_b8_32k", "paged_b4_512k", "verify_b2_q256_128k")


def time_steps(step, steps: int, warmup: int, stream):
    """(mean us over `steps` back-to-back steps between one event pair, sorted
    us of single steps each between its own event pair, host wall us per step)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) / steps * 1e6
    mean_us = e0.elapsed_time(e1) / steps * 1e3
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    return mean_us, sorted(a.elapsed_time(b) * 1e3 for a, b in pairs), wall


def pct(xs, p):
    return round(xs[min(len(xs) - 1, int(p / 100.0 * len(xs)))], 2)


def median(xs):
    n = len(xs)
    return round(xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2]), 2)


def setup(name: str, dev, ncopies: int = 0):
    """The workload, its input copies (see auto_copies), shape and caches."""
    import torch
    from block_sparse_attention_msa_amd import msa, synth
    t0 = time.perf_counter()
    w = synth.make_config(name, device=dev)
    ncopies = ncopies or auto_copies(w)
    copies = [w] + [clone_workload(w) for _ in range(max(0, ncopies - 1))]
    torch.cuda.synchronize()
    log(f"[bench] generated {name} x{len(copies)} in {time.perf_counter() - t0:.1f} s")
    return w, copies, msa.MsaShape.from_workload(w), [msa.MsaCache.from_workload(c) for c in copies]


def measure_step_and_scan(w, copies, shape, caches, steps: int, warmup: int, stream, block_major: bool = False):
    """Times the fused step (with the block-major attention when asked for)
    and the index scan alone (same rotation of input copies); returns a dict
    of the figures and the step's selected ids."""
    import torch
    from block_sparse_attention_msa_amd import msa
    dev = w.q.device
    if block_major:
        ws = torch.empty(msa.msa_block_major_workspace_size(shape), dtype=torch.uint8, device=dev)
    else:
        ws = msa.alloc_workspace(shape, dev)
    out, sel = msa.alloc_outputs(w)

    def step(i):
        decode_call(msa, shape, caches[i % len(copies)], copies[i % len(copies)], out, sel, ws, stream, block_major)

    us_step, per_step, wall = time_steps(step, steps, warmup, stream)
    bs = torch.empty(w.rows, 4, w.max_blocks_per_seq, dtype=torch.float32, device=dev)

    def scan(i):
        scan_call(msa, shape, caches[i % len(copies)], copies[i % len(copies)], bs, stream)

    scan_us, _, _ = time_steps(scan, steps, warmup, stream)
    return dict(us_step=us_step, per_step=per_step, wall=wall, scan_us=scan_us), sel


def scan_roofline(w, scan_us: float):
    """(bound, achieved, peak, unit, frac, algorithmic amount) of the index scan:
    the bound with the longer ideal time at the published peaks."""
    sb = scan_bytes(w)
    fl = scan_flops(w) if w.q_len > 1 else 0.0
    if fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) > sb / (HBM_PEAK_GBPS * 1e9):
        tf = fl / (scan_us * 1e-6) / 1e12
        return "mfma", tf, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", tf / MFMA_BF16_PEAK_TFLOPS, fl
    gb = sb / (scan_us * 1e-6) / 1e9
    return "hbm", gb, HBM_PEAK_GBPS, "GB/s", gb / HBM_PEAK_GBPS, sb


def config_summary(name: str, dev, steps: int, warmup: int, stream) -> dict:
    """The compact record of one more workload: us per step (K-step mean and
    single-step median), algorithmic GB/s and % of HBM peak, the index scan's
    us and roofline fraction (MFMA for the long multi-query chunk)."""
    import torch
    w, copies, shape, caches = setup(name, dev)
    m, sel = measure_step_and_scan(w, copies, shape, caches, steps, warmup, stream)
    nb = w.nbytes_algorithmic(sel if w.q_len > 1 else None)
    bound, ach, peak, unit, frac, amount = scan_roofline(w, m["scan_us"])
    rec = {"us": round(m["us_step"], 2), "us_p50": median(m["per_step"]),
           "us_p10_p90": [pct(m["per_step"], 10), pct(m["per_step"], 90)],
           "bytes": int(nb["total"]), "GBps": round(nb["total"] / (m["us_step"] * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100.0 * nb["total"] / (m["us_step"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
           "scan_us": round(m["scan_us"], 2), "scan_bound": bound, "scan_achieved": round(ach, 1),
           "scan_unit": unit, "scan_frac": round(frac, 4), "scan_share_of_step": round(m["scan_us"] / m["us_step"], 3),
           "input_copies": len(copies)}
    log(f"[bench] {name}: step {rec['us']} us (p50 {rec['us_p50']}), {rec['GBps']} GB/s algorithmic "
        f"({rec['pct_hbm_peak']} %), scan {rec['scan_us']} us = {rec['scan_achieved']} {unit} ({100 * frac:.1f} % of "
        f"{bound} peak)")
    del w, copies, caches, sel
    torch.cuda.empty_cache()
    return rec


BLOCK_MAJOR_CONFIGS = ("verify_b2_q256_128k", "verify_b2_q256_128k_corr")


def block_major_summary(name: str, dev, steps: int, warmup: int, stream) -> dict:
    """us per step of msa_decode (per-row attention) and msa_decode_block_major
    on one multi-query chunk, timed in alternation (4 rounds each, median of
    the rounds' K-step means), with the distinct blocks its rows select per
    (sequence, group)."""
    import torch
    from block_sparse_attention_msa_amd import msa
    w, copies, shape, caches = setup(name, dev)
    ws = msa.alloc_workspace(shape, dev)
    wsb = torch.empty(msa.msa_block_major_workspace_size(shape), dtype=torch.uint8, device=dev)
    out, sel = msa.alloc_outputs(w)

    def per_row(i):
        c = copies[i % len(copies)]
        msa.msa_decode(shape, caches[i % len(copies)], c.q, c.iq, out, sel, ws, stream)

    def block_major(i):
        c = copies[i % len(copies)]
        msa.msa_decode_block_major(shape, caches[i % len(copies)], c.q, c.iq, out, sel, wsb, stream)

    runs = {"per_row": [], "block_major": []}
    for _ in range(4):
        for key, f in (("per_row", per_row), ("block_major", block_major)):
            runs[key].append(time_steps(f, steps, warmup, stream)[0])
    s4 = sel.view(w.num_seqs, w.q_len, 4, 16).cpu()
    distinct = [len(set(x for x in s4[b, :, g].flatten().tolist() if x >= 0))
                for b in range(w.num_seqs) for g in range(4)]
    rec = {"per_row_us": median(sorted(runs["per_row"])),
           "block_major_us": median(sorted(runs["block_major"])),
           "distinct_blocks_per_seq_group_mean": round(sum(distinct) / len(distinct), 1),
           "selections_per_seq_group": w.q_len * 16}
    log(f"[bench] {name}: per-row attention step {rec['per_row_us']} us, block-major step {rec['block_major_us']} us "
        f"({rec['distinct_blocks_per_seq_group_mean']} distinct blocks of {rec['selections_per_seq_group']} "
        f"selections per (sequence, group))")
    del w, copies, caches, sel, wsb
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="paged_b32_128k")
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies the steps rotate through (0: enough that more than 1.25 x the 256 MB "
                         "Infinity Cache of other inputs is read between two uses of one copy)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attention", choices=["per-row", "block-major"], default="per-row",
                    help="block-major: the step runs msa_decode_block_major (NVFP4 K/V, q_len <= 256)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the compact records of the other workloads (tiny, batch-8 32K, batch-4 512K, "
                         "2 x 256-token chunk)")
    ap.add_argument("--mode", choices=["bench", "counters"], default="bench",
                    help="counters: only the scan kernel and a plain 512 MiB copy of known size, for rocprofv3 --pmc")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/scan_<config>_traffic.json from the rocprofv3 FETCH_SIZE and WRITE_SIZE "
                         "runs of --mode counters (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.config, *args.write_traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the MSA decode step; runs on more than one GPU are not "
              "supported (decode context parallelism across GPUs is design-only)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_attention_msa_amd import msa

    dev = torch.device("cuda:0")
    log(f"[bench] device {torch.cuda.get_device_name(0)}")
    w, copies, shape, caches = setup(args.config, dev, args.copies)
    ncopies = len(copies)
    if args.mode == "counters":
        run_counter_pass(args, w, copies, shape, caches)
        return
    stream = torch.cuda.current_stream()
    m, sel = measure_step_and_scan(w, copies, shape, caches, args.steps, args.warmup, stream,
                                   args.attention == "block-major")
    us_step, per_step, scan_us = m["us_step"], m["per_step"], m["scan_us"]
    ms_per_step = us_step / 1e3

    ceiling = read_ceiling(w, copies, stream, args.steps, args.warmup)

    # the write side of the step, timed apart: the new tokens' K/V/index keys
    # quantised into the pools (msa_kv_insert; not part of `value`)
    gi = torch.Generator(device=dev).manual_seed(11)
    k_new = torch.randn(w.rows, w.num_kv_heads, 128, generator=gi, device=dev).to(torch.bfloat16)
    v_new = torch.randn(w.rows, w.num_kv_heads, 128, generator=gi, device=dev).to(torch.bfloat16)
    x_new = torch.randn(w.rows, 128, generator=gi, device=dev).to(torch.bfloat16)
    insert_us, _, _ = time_steps(lambda i: msa.msa_kv_insert(shape, caches[i % len(copies)], k_new, v_new, x_new,
                                                             stream), args.steps, args.warmup, stream)

    nb = w.nbytes_algorithmic(sel if w.q_len > 1 else None)
    step_gbps = nb["total"] / (us_step * 1e-6) / 1e9
    sb = scan_bytes(w)
    ctx_tokens = int(w.seq_lens.sum())
    per_tok = nb["total"] / ctx_tokens
    log(f"[bench] step {us_step:.1f} us, single-step median {median(per_step)} us ({step_gbps:.0f} GB/s "
        f"algorithmic, {nb['total'] / 1e6:.1f} MB), scan {scan_us:.1f} us ({sb / 1e6:.1f} MB), "
        f"host wall {m['wall']:.1f} us, kv insert {insert_us:.1f} us")

    if w.share_members is not None:
        kname = (f"index scan + block max-pool, each shared-prefix page read once per group "
                 f"({w.idx_dtype.upper()} keys, bf16 MFMA)")
    elif w.q_len == 1:
        kname = {"fp8": "index scan + block max-pool (FP8 keys, bf16 MFMA)",
                 "nvfp4": "index scan + block max-pool (NVFP4 keys, bf16 MFMA)",
                 "bf16": "index scan + block max-pool (bf16 keys, VALU dot2)"}[w.idx_dtype]
    elif w.idx_dtype in ("fp8", "nvfp4") and w.q_len <= 8:
        kname = (f"index scan + causal block max-pool ({w.idx_dtype.upper()} keys), {4 * w.q_len} (query, group) "
                 f"columns per sequence (bf16 MFMA)")
    else:
        kname = "multi-query index scan + causal block max-pool (bf16 MFMA)"
    bound, ach, peak, unit, frac, amount = scan_roofline(w, scan_us)
    roofline = {"bound": bound, "kernel": kname, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(frac, 4), "traffic": scan_traffic(args.config) if bound == "hbm" else None,
                "launch_us": round(scan_us, 2)}
    roofline["algorithmic_bytes" if bound == "hbm" else "algorithmic_flops"] = int(amount)
    read_ceil = None
    if ceiling is not None:
        c_us, c_bytes = ceiling
        read_ceil = {"kernel": "read-only walk of the scan's index pages, same block table and load pattern",
                     "us": round(c_us, 2), "bytes": int(c_bytes), "GBps": round(c_bytes / (c_us * 1e-6) / 1e9, 1),
                     "scan_us_over_ceiling_us": round(scan_us / c_us, 4)}
        log(f"[bench] read ceiling {c_us:.1f} us ({read_ceil['GBps']:.0f} GB/s, {c_bytes / 1e6:.1f} MB): "
            f"the scan takes {scan_us / c_us:.3f}x the pure read of its pages")
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        cpu = cpu_baseline(w, args.cpu_sample_seqs, us_step)
        log(f"[bench] cpu baseline {cpu['value'] / 1e6:.2f} s/step on {cpu['cores']} cores "
            f"({time.perf_counter() - t0:.1f} s)")
    del copies, caches
    torch.cuda.empty_cache()

    others = bmaj = None
    if not args.no_other_configs and args.config == "paged_b32_128k":
        # the other workloads, compactly (fewer steps: each is a short run)
        n, wu = max(5, min(args.steps, 30)), max(2, min(args.warmup, 10))
        others = {name: config_summary(name, dev, n, wu, stream) for name in OTHER_CONFIGS}
        bmaj = {name: block_major_summary(name, dev, n, wu, stream) for name in BLOCK_MAJOR_CONFIGS}

    rec = {
        "metric": METRIC,
        "value": round(us_step, 2),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{w.idx_dtype}-idx/{w.kv_dtype}-kv, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": args.config, "num_seqs": w.num_seqs, "context_tokens": int(w.seq_lens[0]),
                   "q_len": w.q_len, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": 128,
                   "block": 128, "top_blocks": 16, "layout": w.meta.get("layout"), "input_copies": ncopies,
                   "attention": args.attention},
        "achieved_GBps": round(step_gbps, 1),
        "pct_hbm_peak": round(100.0 * step_gbps / HBM_PEAK_GBPS, 2),
        "bytes_per_step": int(nb["total"]),
        "bytes_per_ctx_token": round(per_tok, 1),
        "vs_dense_fp8_kv_per_token": round(per_tok / 1024.0, 4),
        "step_us_median": median(per_step),
        "pct_hbm_peak_at_median": round(100.0 * nb["total"] / (median(per_step) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
        "step_us_p10_p50_p90": [pct(per_step, 10), median(per_step), pct(per_step, 90)],
        "timing": "value: mean over the K back-to-back steps between one event pair; step_us_median: median of "
                  "K single steps, each between its own event pair (includes the event overhead)",
        "roofline": roofline,
        "read_ceiling": read_ceil,
        "cpu_baseline": cpu,
        "kv_insert_us": round(insert_us, 2),
        "other_configs": others,
        "block_major_vs_per_row": bmaj,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
