"""Host-side checks of bench.py (no GPU): the one-GPU guard, and that an
HBM-traffic record is reported only while it describes the kernel sources as
they are."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

RECORDS = [("bf16", "768p", None), ("fp8", "768p-fp8", None), ("linear", "768p", "linear"),
           ("linear", "768p", "fuse"), ("bwd", "768p", "bwd")]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("dtype,workload,kernel", RECORDS)
def test_traffic_records_match_the_sources(dtype, workload, kernel):
    path = bench.TRAFFIC_FILE.format(kernel=kernel or f"fwd_{dtype}", workload=workload)
    with open(path) as f:
        rec = json.load(f)
    # every record is stamped with the hash of the sources it was taken on;
    # its bytes are reported exactly while the sources still hash the same
    fresh = rec["kernel_source_sha256_16"] == bench.kernel_source_hash(dtype)
    assert bench.load_traffic(dtype, workload, kernel) == (rec["bytes_per_launch"] if fresh else None)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    # the measured bytes are at least the algorithmic ones (where recorded)
    if "algorithmic_bytes" in rec:
        assert rec["bytes_per_launch"] >= 0.9 * rec["algorithmic_bytes"]


def test_stale_traffic_record_is_not_reported(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda dtype: "0" * 16)
    for dtype, workload, kernel in RECORDS:
        assert bench.load_traffic(dtype, workload, kernel) is None
    assert bench.load_traffic("bf16", "no-such-workload") is None


def test_host_cpu_record():
    rec = bench.host_cpu()
    assert rec["nproc"] == os.cpu_count()
    assert 1 <= rec["affinity"] <= rec["nproc"]
    assert rec["cpu_model"] is None or isinstance(rec["cpu_model"], str)


def test_every_source_set_hashes():
    for dtype in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(dtype)) == 16
