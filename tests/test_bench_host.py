"""Host-side contract of bench.py (no GPU): one GPU only, the committed
profile's traffic is used only while the kernel sources are unchanged, the
timings are medians, and the oracle leg runs on a bounded sample in
single-threaded processes."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profiled_traffic_requires_matching_source(tmp_path, monkeypatch):
    src = tmp_path / "e8_lattice_vector_amd" / "csrc"
    src.mkdir(parents=True)
    for f in bench.SOURCES:
        (src / f).write_bytes(b"v1 " + f.encode())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = hashlib.sha256(b"".join(b"v1 " + f.encode() for f in bench.SOURCES)).hexdigest()
    assert bench.source_sha() == sha
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k.md").write_text(f"kernel sources sha256: {sha}\n\ntraffic_bytes_per_launch: 12345\n")
    (prof / "v.md").write_text(f"kernel sources sha256: {sha}\n\ntraffic_bytes_per_launch: 10001\n")
    assert bench.profiled_traffic(["k.md"]) == 12345
    # one launch per summary: the step's per-launch traffic is their mean
    assert bench.profiled_traffic(["k.md", "v.md"]) == 11173
    assert bench.profiled_traffic(["k.md", "missing.md"]) is None
    # any of the sources changing invalidates the counters
    (src / bench.SOURCES[-1]).write_bytes(b"v2")
    assert bench.profiled_traffic(["k.md"]) is None
    assert bench.profiled_traffic(["k.md", "v.md"]) is None


def test_median_of_event_times():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 3.0, 2.0]) == 2.5


def test_cpu_baseline_leg_runs_the_oracle():
    """The oracle leg on a tiny cache: spawned single-threaded workers, the
    cores and CPU model reported."""
    from e8_lattice_vector_amd import workloads

    w = workloads.Workload("tiny-bench", 4, 2, 64, 128, 5e5, 2, 2, 0, False)
    out = bench.cpu_baseline(w, 1, heads_per_job=1, max_procs=2)
    assert out["kind"] == "oracle" and out["cores"] == 2 and out["unit"] == "tokens/s"
    assert out["value"] > 0 and isinstance(out["cpu_model"], str)
    assert out["sample"].startswith("1 of 4 slabs")
    # 2 tensors x 1 slab x 2 heads = 4 jobs: never more processes than jobs
    out = bench.cpu_baseline(w, 1, heads_per_job=1, max_procs=16)
    assert out["cores"] == min(4, os.cpu_count())
