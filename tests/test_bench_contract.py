"""Host-side checks of bench.py: the one-GPU refusal, the algorithmic work
figures the rooflines divide by, the long-run schedule, and the rule that a
recorded HBM traffic figure is reported only for the kernel source it was
measured on.  No GPU is touched (bench.py imports torch only inside its
GPU paths)."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_work_per_launch_figures():
    # attention, every one of the 5,788 slots visible to each of the 757
    # queries: QK^T and PV are 2 d flops each per (query, slot, head)
    assert bench.ATTN_FLOP == 89_733_447_680
    # write of 757 tokens: bf16 K and V in (15,503,360) + FP8 codes out
    # (7,751,680) + float32 scales (242,240) + slot_pos and slot_block (6,056)
    assert bench.WRITE_BYTES == 23_503_336
    # re-rotation of a full ring: codes (29,634,560) and scales (926,080)
    # read and written, slot_block read, slot_pos read and written
    assert bench.REROT_BYTES == 61_190_736


def test_long_run_schedule():
    # positions: 757 per chunk until the first reset at chunk 300; a reset
    # rebases the cache to 0 .. 5,787, so the chunk after it starts at 5,788
    assert [bench.chunk_pos0(t) for t in (0, 1, 299)] == [0, 757, 299 * 757]
    assert [bench.chunk_pos0(t) for t in (300, 301, 599, 600)] == [5788, 5788 + 757, 5788 + 299 * 757, 5788]
    # ten transitions from chunk 150, every 200 chunks: 0, -2, -4, -2, 0
    assert [bench.bias_at(t) for t in range(149, 156)] == [0.0, 0.0, -2.0, -4.0, -2.0, 0.0, 0.0]
    assert bench.bias_at(150 + 9 * 200 + 2) == -4.0
    assert bench.bias_at(150 + 10 * 200 + 2) == 0.0
    # no transition overlaps a reset chunk
    assert all(bench.bias_at(t) == 0.0 for t in range(0, 4000, 300))


def _traffic_file(tmp_path, sha, value="78646221"):
    p = tmp_path / "traffic.txt"
    p.write_text("# header: not a field\n"
                 f"kernel_source_sha256: {sha}\n"
                 f"traffic_bytes_per_launch: {value}\n")
    return str(p)


def test_recorded_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"__global__ void k() {}\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, sha))
    assert bench.recorded_traffic() == 78646221.0
    # the kernel changed since the counters were taken: no figure
    src.write_bytes(b"__global__ void k() { /* changed */ }\n")
    assert bench.recorded_traffic() is None
    # no record, or a record without the figure
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None
    sha2 = hashlib.sha256(src.read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, sha2, value="n/a"))
    assert bench.recorded_traffic() is None


@pytest.mark.parametrize("flag", ["--joint-av-only", "--longrun", "--copy-calibration", "--no-cpu-baseline"])
def test_options_are_listed(flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0 and flag in r.stdout
