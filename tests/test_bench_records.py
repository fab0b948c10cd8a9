"""CPU checks of the benchmark: its committed measurement records (the
traffic records match the scan sources as checked out, on any machine) and
its refusal of runs on several GPUs."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_attention_msa_amd import build as hip_build  # noqa: E402


def test_source_hash_independent_of_checkout_path(monkeypatch):
    """The records' hash covers the scan sources and their compiler flags, but
    not the directory the repository sits in (the include path is absolute)."""
    h0 = bench.scan_source_hash()
    other = "/some/other/checkout"
    monkeypatch.setattr(hip_build, "FLAGS", [f.replace(hip_build.ROOT, other) for f in hip_build.FLAGS])
    monkeypatch.setattr(hip_build, "ROOT", other)
    assert bench.scan_source_hash() == h0


def test_committed_traffic_records():
    """A committed traffic record is reported by the bench exactly when it was
    taken on the scan code as it stands (otherwise the bench reports null)."""
    import pytest
    recs = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_traffic.json")]
    assert recs
    stale = []
    for f in recs:
        rec = json.load(open(os.path.join(ROOT, "profiles", f)))
        current = rec["source_sha256"] == bench.scan_source_hash()
        assert bench.scan_traffic(rec["workload"]) == (rec["bytes_per_launch"] if current else None), f
        if not current:
            stale.append(f)
    if stale:
        pytest.skip(f"records taken before the last scan change (bench reports traffic null): {stale}")


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: asked for several it exits with status 2 and
    says why, before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "more than one GPU" in (r.stdout + r.stderr)
