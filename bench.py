#!/usr/bin/env python3
"""Benchmark of the local-window attention forward on one MI355X.

One step = one forward call over the whole workload (all samples and heads),
inputs already resident in HBM.  Prints one JSON line with effective TFLOP/s
(allowed (query, key) pairs only: 4*D flops per pair per head), ms per step,
the fraction of the dense MFMA peak, the speedup over the same kernel run
dense (block_frames = F), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload 768p]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s + ms/call, 768p-shaped local-window attn; % MFMA peak"
# Dense MFMA peaks of MI355X in TFLOP/s: 256 CUs x 2.4 GHz x 4096 (bf16) or
# 8192 (fp8) flop per clock per CU; AMD quotes them as 2.5 and 5.0 PFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}
KERNEL_SOURCES = {"bf16": "fwd_kernel.hip", "fp8": "fwd_fp8_kernel.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{kernel}_{workload}.json")


def kernel_source_hash(dtype: str) -> str:
    path = os.path.join(ROOT, "block_sparse_attention_31_amd", "csrc", KERNEL_SOURCES[dtype])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(dtype: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the kernel source as it is now; otherwise None."""
    path = TRAFFIC_FILE.format(kernel=f"fwd_{dtype}", workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(dtype):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inp, seconds: float):
    """Time the fp64 oracle on whole heads of sample 0 until `seconds` pass."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    allowed, _ = oracle.count_pairs(w.F, w.T, w.N, w.Bf)
    done = 0
    t_total = 0.0
    for h in range(w.H):
        idx = torch.tensor([h])
        q, k, v = (inp[n][:1].index_select(2, idx) for n in ("q", "k", "v"))
        if inp["scales"] is not None:
            s = inp["scales"][:, h:h + 1].numpy()
            q, k, v = (oracle.dequantize_fp8(x.to(torch.float64).numpy(), s[i])
                       for i, x in enumerate((q, k, v)))
        else:
            q, k, v = (x.to(torch.float64).numpy() for x in (q, k, v))
        g = None if inp["gate"] is None else inp["gate"][:1, :, h:h + 1].to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.attend(q, k, v, g, w.F, w.T, w.N, w.Bf)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= seconds:
            break
    flops = 4.0 * w.D * allowed * done
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{w.name}: sample 0, {done} of {w.H} heads, all {w.S} query rows "
                      f"({done * allowed} allowed pairs), fp64 NumPy, {t_total:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="768p")
    ap.add_argument("--dense-steps", type=int, default=20, help="0 skips the dense run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="0 skips the CPU baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device-to-device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch

    from block_sparse_attention_31_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    binding.lib()  # fail loudly if the HIP library is missing
    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    gate = None if inp["gate"] is None else inp["gate"].to(dev)
    scales = None if inp["scales"] is None else inp["scales"].to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(bf):
        binding.vdn_local_attn_fwd(q, k, v, gate, out, w.F, w.T, w.N, bf, qkv_scales=scales,
                                   stream=stream.cuda_stream)

    def timed(bf, steps, warmup):
        for _ in range(warmup):
            step(bf)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step(bf)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    ms, wall_ms = timed(w.Bf, args.steps, args.warmup)
    print(f"[bench] {w.name} sparse: {ms:.4f} ms/step over {args.steps} steps", file=sys.stderr, flush=True)
    dense_ms = None
    if args.dense_steps > 0:
        dense_ms, _ = timed(w.F, args.dense_steps, 2)
        print(f"[bench] {w.name} dense: {dense_ms:.4f} ms/step", file=sys.stderr, flush=True)

    import oracle  # closed-form pair counts only; no oracle compute on this path

    allowed, _ = oracle.count_pairs(w.F, w.T, w.N, w.Bf)
    flops = 4.0 * w.D * w.H * w.B * allowed
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = load_traffic(w.dtype, w.name)
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.D,
                   "frames": w.F, "tokens_per_frame": w.T, "text_tokens": w.N, "seq_len": w.S,
                   "block_frames": w.Bf, "gate": w.gate, "allowed_pairs_per_head": allowed},
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
        "wall_ms_per_step": round(wall_ms, 4),
        "dense_ms_per_step": None if dense_ms is None else round(dense_ms, 4),
        "sparse_vs_dense_speedup": None if dense_ms is None else round(dense_ms / ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
