"""bench.py end to end on the GPU: one short run, and the JSON line it prints
carries every field of its contract (the metric, throughput, the roofline of
the forward kernel with its traffic record, the CPU oracle baseline and the
vendor-GEMM context line)."""

import json
import os
import subprocess
import sys

import pytest

from .gpu_util import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_its_contract():
    sys.path.insert(0, ROOT)
    import bench

    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--also=", "--dense-steps", "2", "--cpu-seconds", "2", "--gemm", "2048"]
    run = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stderr[-2000:]
    rec = json.loads(run.stdout.strip().splitlines()[-1])
    assert rec["metric"] == bench.METRIC
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["dtype"] == "bf16" and rec["data"] == "synthetic" and rec["higher_is_better"] is True
    assert rec["config"]["workload"] == "768p" and rec["config"]["heads"] == 32
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    flop = 4.0 * 128 * rec["config"]["allowed_pairs_per_head"] * 32
    assert abs(rec["value"] - flop / (rec["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * rec["value"]
    roof = rec["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == bench.PEAK_TFLOPS["bf16"]
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # HBM traffic is reported exactly when the committed record matches the
    # kernel sources (null otherwise, as for a kernel changed since profiling)
    fresh = bench.load_traffic("bf16", "768p") is not None
    assert (roof["traffic"] is not None) == fresh
    assert roof["traffic"] is None or roof["traffic"] > 0
    assert rec["sparse_vs_dense_speedup"] > 1
    cpu = rec["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    gemm = rec["library_gemm"]
    assert gemm["tflops_at_median"] > 0 and gemm["forward_vs_gemm"] > 0
