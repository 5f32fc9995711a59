"""Host-side contract of bench.py (no GPU): one GPU only, the committed
profile's traffic is used only while the kernel source is unchanged, and the
oracle leg runs on a bounded sample with one thread."""
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
    (src / "nq_kernels.hip").write_bytes(b"kernel v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = hashlib.sha256(b"kernel v1").hexdigest()
    (prof / "k.md").write_text(f"nq_kernels.hip sha256: {sha}\n\ntraffic_bytes_per_launch: 12345\n")
    (prof / "v.md").write_text(f"nq_kernels.hip sha256: {sha}\n\ntraffic_bytes_per_launch: 10001\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic(["k.md"]) == 12345
    # one launch per summary: the step's per-launch traffic is their mean
    assert bench.profiled_traffic(["k.md", "v.md"]) == 11173
    assert bench.profiled_traffic(["k.md", "missing.md"]) is None
    (src / "nq_kernels.hip").write_bytes(b"kernel v2")
    assert bench.profiled_traffic(["k.md"]) is None
    assert bench.profiled_traffic(["k.md", "v.md"]) is None


def test_cpu_baseline_leg_runs_the_oracle():
    from e8_lattice_vector_amd import workloads

    out = bench.cpu_baseline(workloads.LLAMA, 64, 1)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["unit"] == "tokens/s"
    assert out["value"] > 0
    assert out["sample"].startswith("1 of 32 slabs")
