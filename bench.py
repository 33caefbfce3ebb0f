"""Benchmark: one decode token of a Qwen3-8B-shaped 1-bit model = 253 Q1_0
matrix-vector products (36 layers x q, k, v, o, gate, up, down + LM head,
about 1.06 GB of packed weights), on one MI355X.

A step is the whole hot path for one token: one launch quantizes the 253
activation vectors (laid end to end) and one launch runs the 253 products.
Weights are packed and copied to the GPU once, before timing; inputs are
seeded synthetic data with the workload's shapes and distributions.

Prints ONE JSON line.  python bench.py [--steps K] [--warmup W] [--fmt q1_0|q2_0]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PROFILE = os.path.join(ROOT, "profiles", "sweep_kernel_q1_0_decode_token.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(fmt_name: str):
    """HBM bytes per sweep launch from the committed rocprofv3 counter summary,
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        with open(PROFILE) as f:
            prof = json.load(f)
        h = hashlib.sha256()
        for p in prof["kernel_sources"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    if fmt_name != "Q1_0" or h.hexdigest() != prof.get("kernel_sources_sha256"):
        return None
    return prof.get("traffic_bytes_per_launch")


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(sw, y_gpu: np.ndarray, budget_s: float, threads: int):
    """The CPU oracle on a bounded sample of the same token: whole products,
    taken in sweep order until about budget_s seconds of work.  Also checks
    the GPU's outputs for those products bit for bit."""
    import oracle

    q_ref, d_ref, _ = oracle.quantize_q8(sw.x, sw.qa)
    done_bytes = 0
    secs = 0.0
    mismatched = 0
    n = 0
    for i, (name, rows, cols) in enumerate(sw.shapes):
        k0, k1 = int(sw.koff[i]), int(sw.koff[i + 1])
        t0 = time.perf_counter()
        y = oracle.matvec(sw.fmt, sw.canon[i], rows, cols, q_ref[k0:k1], d_ref[k0 // sw.qa:k1 // sw.qa], sw.qa,
                          threads=threads)[0]
        secs += time.perf_counter() - t0
        done_bytes += sw.canon[i].size + cols + 4 * (cols // sw.qa) + 4 * rows
        yg = y_gpu[int(sw.yoff[i]):int(sw.yoff[i + 1])]
        mismatched += int(np.count_nonzero(yg.view(np.uint32) != y.view(np.uint32)))
        n += 1
        if secs >= budget_s:
            break
    return {
        "value": round(done_bytes / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n} of {len(sw.shapes)} products of the token ({done_bytes / 1e9:.3f} GB, "
                  f"{secs:.1f} s); quantizer excluded",
        "ms_per_token_equiv": round(sw.sweep_bytes() / (done_bytes / secs) * 1e3, 1),
        "gpu_outputs_checked": int(sum(r for _, r, _ in sw.shapes[:n])),
        "gpu_outputs_mismatched": mismatched,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--fmt", choices=["q1_0", "q2_0"], default="q1_0")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the 253 products of a token are independent row "
              "blocks; rows would shard across GPUs with no exchange, but this benchmark measures "
              "one GPU. Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import ternary_quantized_gemv_amd as bq
    from ternary_quantized_gemv_amd.staging import StagedSweep

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    fmt = bq.BQ_Q1_0 if args.fmt == "q1_0" else bq.BQ_Q2_0
    shapes = synth.decode_sweep_shapes()
    t0 = time.time()
    canon = [synth.blocks(fmt, r, c, args.seed, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, args.seed, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
    sw = StagedSweep(fmt, canon, shapes, x, qa=128)
    log(f"staged {len(shapes)} products, {sw.weight_bytes / 1e9:.3f} GB of weights in {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        sw.run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        a, b, c = ev[k]
        a.record(stream)
        sw.quantize()
        b.record(stream)
        sw.sweep()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    quant_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    sweep_ms_all = np.array([b.elapsed_time(c) for _, b, c in ev])
    sweep_ms = float(np.mean(sweep_ms_all))
    ms_per_step = wall * 1e3 / K

    step_bytes = sw.sweep_bytes() + sw.quantize_bytes()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = sw.sweep_bytes() / (sweep_ms * 1e-3) / 1e9
    y_gpu = sw.y.cpu().numpy()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device-to-device copies done")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(sw, y_gpu, args.cpu_budget, cpu_threads())

    fmt_name = "Q1_0" if fmt == bq.BQ_Q1_0 else "Q2_0"
    out = {
        "metric": f"achieved HBM GB/s (% of peak) and ms/token for 253-matmul {fmt_name} sweep",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_token": round(ms_per_step, 5),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xQ1_0->f32" if fmt == bq.BQ_Q1_0 else "int8xQ2_0->f32",
        "data": "synthetic (seeded; uniform sign bits, f16 |N(0,0.02)| block scales, N(0,1) activations)",
        "config": {
            "workload": f"decode token, Qwen3-8B shapes, {fmt_name}: 36 x (q 4096x4096, k 1024x4096, "
                        "v 1024x4096, o 4096x4096, gate 12288x4096, up 12288x4096, down 4096x12288) "
                        "+ lm_head 151936x4096 = 253 GEMVs, one activation vector each, qa 128",
            "products": len(shapes),
            "weight_bytes": sw.weight_bytes,
            "step_bytes": step_bytes,
            "launches_per_step": 2,
        },
        "kernels": {
            "sweep_ms": round(sweep_ms, 5),
            "sweep_ms_min": round(float(sweep_ms_all.min()), 5),
            "quantize_ms": round(quant_ms, 5),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "bq::sweep_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(fmt_name),
            "algorithmic_bytes_per_launch": sw.sweep_bytes(),
        },
        "cpu_baseline": cpu,
    }
    sw.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
