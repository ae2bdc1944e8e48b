"""Host-side parts of bench.py (no GPU): the single-GPU guard, the kernel-source hash that keys the
stored byte counters, and the host CPU description of the CPU-oracle baseline."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() {\n  return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "t", ("k.hip",))
    h = bench.kernel_sha("t")
    src.write_text("/* a kernel */\nint f() {\n\n  return 1;  // the value\n}\n")
    assert bench.kernel_sha("t") == h
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_sha("t") != h


def test_stored_traffic_holds_only_for_the_measured_sources():
    for name, t in bench.TRAFFIC.items():
        path = {"c5": "prefill", "v4p-w4a8": "w4a8", "v4p-mx": "w4a8", "v3-int8": "int8"}.get(name, "decode")
        assert bench.measured_traffic(name, path) == (t["bytes"] if t["sha"] == bench.kernel_sha(path) else None)
    assert bench.measured_traffic("no-such-workload", "decode") is None


def test_host_cpu_names_the_model_and_counts_usable_threads():
    model, threads = bench.host_cpu()
    assert model
    assert 1 <= threads <= len(os.sched_getaffinity(0))


@pytest.mark.parametrize("name", bench.WORKLOADS)
def test_every_workload_has_a_bounded_cpu_sample(name):
    assert 1 <= bench.CPU_TOKENS[name] <= 256
