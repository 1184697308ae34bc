#!/usr/bin/env python3
"""Benchmark of the local-window attention forward on one MI355X.

One step = one forward call over the whole workload (all samples and heads),
inputs already resident in HBM.  Prints one JSON line with effective TFLOP/s
(allowed (query, key) pairs only: 4*D flops per pair per head), ms per step,
the fraction of the dense MFMA peak, the speedup over the same kernel run
dense (block_frames = F), and the CPU oracle timed on a bounded sample.
Every timed line also carries the median of its per-call durations (one HIP
event before each call on the launch stream).  Extra workloads -- the medium,
long-video and fp8 forward configurations (each with its dense run and a CPU
oracle sample), the backward pass, the complement linear branch, the
two-branch fusion, the whole hybrid attention output and one GPU's 4-head
share -- are reported under "other_workloads".  For context, "library_gemm"
times the vendor's dense bf16 GEMM on the same GPU (a practical ceiling for
matrix-core work on the part) and gives the forward's rate as a fraction of it.

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
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
KERNEL_SOURCES = {"bf16": ["fwd_kernel.hip", "fwd_common.hpp", "fwd_params.hpp"],
                  "fp8": ["fwd_fp8_kernel.hip", "fwd_common.hpp", "fwd_params.hpp"],
                  "linear": ["linear_kernel.hip", "linear_params.hpp", "fwd_common.hpp"],
                  "bwd": ["bwd_kernel.hip", "fwd_common.hpp", "fwd_params.hpp"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{kernel}_{workload}.json")


def kernel_source_hash(dtype: str) -> str:
    """Hash of the sources the kernel is compiled from (traffic counters are
    only reported while they describe the kernel as it is)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, "block_sparse_attention_31_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(dtype: str, workload: str, kernel: str | None = None):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the kernel source as it is now; otherwise None.  `dtype` picks
    the source set ("bf16", "fp8", "linear"), `kernel` the file name part
    (default fwd_<dtype>)."""
    path = TRAFFIC_FILE.format(kernel=kernel or f"fwd_{dtype}", workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(dtype):
        return None
    return rec.get("bytes_per_launch")


def host_cpu() -> dict:
    """The host CPU the oracle runs on: model name, logical CPUs, and the CPUs
    this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity}


def cpu_baseline(w, inp, seconds: float):
    """Time the fp64 oracle on whole heads of sample 0 until `seconds` pass."""
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
    rec = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{w.name}: sample 0, {done} of {w.H} heads, all {w.S} query rows "
                     f"({done * allowed} allowed pairs), fp64 NumPy, {t_total:.1f} s",
           "ms_per_head": round(1e3 * t_total / done, 1)}
    rec.update(host_cpu())
    return rec


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="768p")
    ap.add_argument("--dense-steps", type=int, default=20, help="0 skips the dense runs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle budget for the headline workload (0 skips every CPU baseline)")
    ap.add_argument("--cpu-seconds-other", type=float, default=4.0,
                    help="CPU oracle budget for each other forward configuration")
    ap.add_argument("--also", default="768p-fp8,medium,long,768p-bwd,768p-linear,768p-fuse,768p-hybrid,768p-h4",
                    help="comma-separated extra workloads reported under 'other_workloads' "
                         "(suffixes: '-bwd' the backward pass, '-linear' the linear branch, "
                         "'-fuse' the fusion, '-hybrid' softmax + linear + fusion; '' for none)")
    ap.add_argument("--gemm", type=int, default=8192,
                    help="size n of the vendor bf16 GEMM (n^3) timed for context after the "
                         "workloads (0 skips it)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device-to-device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch

    from block_sparse_attention_31_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    binding.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    other_steps = max(args.steps, 20)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def time_calls(step, steps: int, warmup: int):
        """(mean ms, median ms, wall ms) per call over `steps` back-to-back
        calls: an event is recorded on the launch stream before every call and
        after the last, so the mean is the bracketed total over `steps`."""
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i].record(stream)
            step()
        ev[steps].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        mean = ev[0].elapsed_time(ev[steps]) / steps
        mid = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
        return mean, mid, wall

    def shape_config(w):
        return {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.D, "frames": w.F,
                "tokens_per_frame": w.T, "text_tokens": w.N, "seq_len": w.S, "block_frames": w.Bf}

    def measure(name: str, steps: int, warmup: int, dense_steps: int, cpu_seconds: float):
        """The forward pass of a configuration: sparse, dense (block_frames
        = F) on the same inputs, and the CPU oracle on a bounded sample."""
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        gate = None if inp["gate"] is None else inp["gate"].to(dev)
        scales = None if inp["scales"] is None else inp["scales"].to(dev)
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

        def run(bf):
            return lambda: binding.vdn_local_attn_fwd(q, k, v, gate, out, w.F, w.T, w.N, bf, qkv_scales=scales,
                                                      stream=stream.cuda_stream)

        ms, med, wall_ms = time_calls(run(w.Bf), steps, warmup)
        print(f"[bench] {w.name} sparse: {ms:.4f} ms/step (median {med:.4f}) over {steps} steps",
              file=sys.stderr, flush=True)
        dense_ms = dense_med = None
        if dense_steps > 0:
            dense_ms, dense_med, _ = time_calls(run(w.F), dense_steps, 2)
            print(f"[bench] {w.name} dense: {dense_ms:.4f} ms/step (median {dense_med:.4f})",
                  file=sys.stderr, flush=True)
        # closed-form count of attended (query, key) pairs, from the library
        allowed, _ = binding.vdn_local_attn_count_pairs(w.F, w.T, w.N, w.Bf)
        flop = 4.0 * w.D * w.H * w.B * allowed
        tflops = flop / (ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        cfg = shape_config(w)
        cfg.update({"gate": w.gate, "allowed_pairs_per_head": allowed, "outlier_frac": w.outlier_frac})
        rec = {
            "ms_per_step": round(ms, 4),
            "ms_per_call_median": round(med, 4),
            "tflops": round(tflops, 2),
            "tflops_at_median": round(flop / (med * 1e-3) / 1e12, 2),
            "wall_ms_per_step": round(wall_ms, 4),
            "steps": steps,
            "dtype": w.dtype,
            "config": cfg,
            "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
            "dense_ms_per_step": None if dense_ms is None else round(dense_ms, 4),
            "dense_ms_per_call_median": None if dense_med is None else round(dense_med, 4),
            "sparse_vs_dense_speedup": None if dense_ms is None else round(dense_ms / ms, 3),
            "ideal_sparse_vs_dense_speedup": round(float(w.S) * w.S / allowed, 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                         "traffic": load_traffic(w.dtype, w.name)},
        }
        if cpu_seconds > 0:
            rec["cpu_baseline"] = cpu_baseline(w, inp, cpu_seconds)
        return rec

    def measure_bwd(name: str, steps: int, warmup: int):
        """The backward pass of a workload (inputs, upstream gradient, and the
        forward's out and log-sum-exp prepared outside the timed region)."""
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        gate = None if inp["gate"] is None else inp["gate"].to(dev)
        dout = synth.make_dout(w).to(dev)
        out, lse = binding.local_attn_fwd(q, k, v, gate, F=w.F, tokens_per_frame=w.T, n_text=w.N,
                                          block_frames=w.Bf, return_lse=True)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        dgate = None if gate is None else torch.empty_like(gate)
        ws = torch.empty(2 * w.B * w.H * w.S, dtype=torch.float32, device=dev)

        def step():
            binding.vdn_local_attn_bwd(q, k, v, gate, out, dout, lse, dq, dk, dv, dgate, w.F, w.T, w.N,
                                       w.Bf, workspace=ws, stream=stream.cuda_stream)
        ms, med, _ = time_calls(step, steps, warmup)
        print(f"[bench] {w.name} backward: {ms:.4f} ms/step (median {med:.4f}) over {steps} steps",
              file=sys.stderr, flush=True)
        allowed, _ = binding.vdn_local_attn_count_pairs(w.F, w.T, w.N, w.Bf)
        # 2.5x the forward's work: S recomputed, dP, dS K, dS^T Q, P^T dO
        tflops = 10.0 * w.D * w.H * w.B * allowed / (ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        cfg = shape_config(w)
        cfg["gate"] = w.gate
        return {"ms_per_step": round(ms, 4), "ms_per_call_median": round(med, 4), "tflops": round(tflops, 2),
                "steps": steps, "dtype": w.dtype, "pass": "backward (dq, dk, dv, dgate)",
                "flop_convention": "10*D per attended pair per head (2.5x forward)",
                "config": cfg,
                "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
                "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                             "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                             "traffic": load_traffic("bwd", w.name, "bwd")}}

    def linear_bytes(w) -> int:
        """Compulsory HBM bytes of the linear branch: K and V of frames
        1..F-2 once, Q of the rows whose block has keys outside its window,
        and every output row (bf16)."""
        nb = -(-w.F // w.Bf)
        rows_with_keys = 0
        for beta in range(nb):
            lo, hi = w.Bf * max(0, beta - 1), min(w.F, w.Bf * (beta + 2))
            if any((f < lo or f >= hi) for f in range(1, w.F - 1)):
                rows_with_keys += (min(w.F, (beta + 1) * w.Bf) - beta * w.Bf) * w.T
        per_head = 2 * max(w.F - 2, 0) * w.T + rows_with_keys + w.S
        return per_head * w.B * w.H * w.D * 2

    def hbm_roofline(nbytes: int, ms: float, traffic=None) -> dict:
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}

    def measure_linear(name: str, steps: int, warmup: int):
        """The complement linear branch (three kernels per step)."""
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        nws = binding.vdn_linear_branch_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

        def step():
            binding.vdn_linear_branch_fwd(q, k, v, out, w.F, w.T, w.N, w.Bf, workspace=ws,
                                          stream=stream.cuda_stream)
        ms, med, _ = time_calls(step, steps, warmup)
        print(f"[bench] {w.name} linear branch: {ms:.4f} ms/step (median {med:.4f}) over {steps} steps",
              file=sys.stderr, flush=True)
        nbytes = linear_bytes(w)
        return {"ms_per_step": round(ms, 4), "ms_per_call_median": round(med, 4), "steps": steps,
                "dtype": "bf16", "pass": "complement linear branch (frame states, block states, apply)",
                "algorithmic_bytes": nbytes, "workspace_bytes": nws,
                "config": shape_config(w),
                "roofline": hbm_roofline(nbytes, ms, load_traffic("linear", w.name, "linear"))}

    def measure_fuse(name: str, steps: int, warmup: int):
        """The two-branch fusion over every token of the workload."""
        w = synth.WORKLOADS[name]
        fi = synth.make_fuse_inputs(w)
        soft, lin = fi["soft"].to(dev), fi["lin"].to(dev)
        gate, weight = fi["gate"].to(dev), fi["weight"].to(dev)
        out = torch.empty_like(soft)

        def step():
            binding.vdn_hybrid_fuse(soft, lin, gate, weight, out, 1e-6, stream=stream.cuda_stream)
        ms, med, _ = time_calls(step, steps, warmup)
        print(f"[bench] {w.name} fusion: {ms:.4f} ms/step (median {med:.4f}) over {steps} steps",
              file=sys.stderr, flush=True)
        tokens = w.B * w.S
        nbytes = 3 * tokens * w.H * w.D * 2 + tokens * w.H * 4 + w.H * w.D * 4
        return {"ms_per_step": round(ms, 4), "ms_per_call_median": round(med, 4), "steps": steps,
                "dtype": "bf16", "pass": "fusion: soft + sigmoid(g) * RMSNorm(lin) * w",
                "algorithmic_bytes": nbytes, "config": shape_config(w),
                "roofline": hbm_roofline(nbytes, ms, load_traffic("linear", w.name, "fuse"))}

    def measure_gemm(n: int, steps: int, warmup: int):
        """Context, not this library: the vendor's dense bf16 GEMM (torch.matmul,
        which dispatches to hipBLASLt) on n x n x n, the same GPU and the same
        peak, as a practical ceiling for matrix-core work on this part."""
        g = torch.Generator(device=dev).manual_seed(1)
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)

        def step():
            torch.matmul(a, b, out=c)
        ms, med, _ = time_calls(step, steps, warmup)
        tflops = 2.0 * n ** 3 / (med * 1e-3) / 1e12
        print(f"[bench] bf16 GEMM {n}^3 (torch.matmul): {ms:.4f} ms/step (median {med:.4f}), "
              f"{tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
        return {"what": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), same GPU; context only",
                "ms_per_step": round(ms, 4), "ms_per_call_median": round(med, 4), "steps": steps,
                "tflops_at_median": round(tflops, 2),
                "pct_of_mfma_peak": round(100.0 * tflops / PEAK_TFLOPS["bf16"], 2)}

    def measure_hybrid(name: str, steps: int, warmup: int):
        """The hybrid attention output of one layer before the output
        projections: gated softmax branch, linear branch, fusion."""
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        fi = synth.make_fuse_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        gate = inp["gate"].to(dev) if inp["gate"] is not None else None
        gl, weight = fi["gate"].to(dev), fi["weight"].to(dev)
        soft, lin = torch.empty_like(q), torch.empty_like(q)
        nws = binding.vdn_linear_branch_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        st = stream.cuda_stream

        def step():
            binding.vdn_local_attn_fwd(q, k, v, gate, soft, w.F, w.T, w.N, w.Bf, stream=st)
            binding.vdn_linear_branch_fwd(q, k, v, lin, w.F, w.T, w.N, w.Bf, workspace=ws, stream=st)
            binding.vdn_hybrid_fuse(soft, lin, gl, weight, soft, 1e-6, stream=st)
        ms, med, _ = time_calls(step, steps, warmup)
        print(f"[bench] {w.name} hybrid layer attention, three calls: {ms:.4f} ms/step (median {med:.4f})",
              file=sys.stderr, flush=True)
        # one call: the linear branch, then the softmax branch with the fusion
        # in its epilogue
        nws1 = binding.vdn_hybrid_attn_workspace_bytes(w.F, w.T, w.N, w.Bf, w.H, w.D, w.B)
        ws1 = torch.empty(nws1, dtype=torch.uint8, device=dev)

        def step1():
            binding.vdn_hybrid_attn_fwd(q, k, v, gate, gl, weight, soft, w.F, w.T, w.N, w.Bf,
                                        eps=1e-6, workspace=ws1, stream=st)
        ms1, med1, _ = time_calls(step1, steps, warmup)
        print(f"[bench] {w.name} hybrid layer attention, one call: {ms1:.4f} ms/step (median {med1:.4f})",
              file=sys.stderr, flush=True)
        return {"ms_per_step": round(ms1, 4), "ms_per_call_median": round(med1, 4),
                "ms_per_step_three_calls": round(ms, 4), "steps": steps, "dtype": "bf16",
                "pass": "hybrid attention output: linear branch, then the softmax branch with the "
                        "fusion in its epilogue (vdn_hybrid_attn_fwd); three_calls: softmax branch, "
                        "linear branch, fusion kernel",
                "config": shape_config(w),
                "context": "whole-layer figures on the pages (332.5 / 192.1 / 125.3 ms per layer on "
                           "one B200) include projections and other hardware; not a target"}

    main_rec = measure(args.workload, args.steps, args.warmup, args.dense_steps, args.cpu_seconds)
    result = {
        "metric": METRIC,
        "value": main_rec["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_rec["dtype"],
        "data": "synthetic",
        "config": main_rec["config"],
    }
    for key in ("ms_per_call_median", "tflops_at_median", "pct_of_mfma_peak", "wall_ms_per_step",
                "dense_ms_per_step", "dense_ms_per_call_median", "sparse_vs_dense_speedup",
                "ideal_sparse_vs_dense_speedup", "roofline"):
        result[key] = main_rec[key]
    others = {}
    cpu_other = args.cpu_seconds_other if args.cpu_seconds > 0 else 0.0
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        if name.endswith("-bwd"):
            others[name] = measure_bwd(name[:-4], other_steps, max(args.warmup // 2, 2))
        elif name.endswith("-linear"):
            others[name] = measure_linear(name[:-7], other_steps, args.warmup)
        elif name.endswith("-fuse"):
            others[name] = measure_fuse(name[:-5], other_steps, args.warmup)
        elif name.endswith("-hybrid"):
            others[name] = measure_hybrid(name[:-7], other_steps, max(args.warmup // 2, 2))
        else:
            dense = args.dense_steps if name != "768p-h4" else 0
            others[name] = measure(name, other_steps, max(args.warmup // 2, 2), dense,
                                   cpu_other if name != "768p-h4" else 0.0)
        torch.cuda.empty_cache()
    if others:
        result["other_workloads"] = others
    if args.gemm > 0:
        gemm = measure_gemm(args.gemm, other_steps, args.warmup)
        gemm["forward_vs_gemm"] = round(main_rec["tflops_at_median"] / gemm["tflops_at_median"], 4)
        result["library_gemm"] = gemm
    if "cpu_baseline" in main_rec:
        result["cpu_baseline"] = main_rec["cpu_baseline"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
