"""Benchmark: one decode token of a Qwen3-8B-shaped 1-bit model = 253 Q1_0
matrix-vector products (36 layers x q, k, v, o, gate, up, down + LM head,
about 1.06 GB of packed weights), on one MI355X.

A step is the whole hot path for one token: one launch quantizes the 253
activation vectors (laid end to end) and one launch runs the 253 products.
Weights are packed and copied to the GPU once, before timing; inputs are
seeded synthetic data with the workload's shapes and distributions.

Prints ONE JSON line.  python bench.py [--steps K] [--warmup W] [--fmt q1_0|q2_0]
Beside GB/s it gives us per matmul and ms per token, each with its HBM
roofline time and fraction, the streaming-read floor measured live on the same
GPU (k_floor, bq_read_floor over 1 GiB) and every fraction against it, the
oracle on the host's cores with a bit-for-bit check of the GPU's outputs (and
their largest relative error), and the pages' laptop CPU figures as context.
The line also reports, as context, the same token in one launch that
quantizes the f32 activations itself (field one_launch_token), and run as a
dependency-ordered decode (field decode_chain; --no-chain skips it).
[--act q8_128|q8_0]: q8_0 quantizes with qa 32 and f16-valued scales (the
pages' activation flavour) instead of qa 128 with f32 scales.

Other workloads (each prints its own JSON line; not the headline):
  --workload gemv   single products at the configured shapes (Q1_0 4096x4096,
                    12288x4096, 4096x12288, 151936x4096; Q2_0 4096x4096,
                    1024x4096, 12288x4096, 4096x12288): us per product, GB/s,
                    fraction of HBM peak, ms per token-equivalent
  --workload batch  12288x4096 and 151936x4096 with N = 1, 4, 8, 16 (--fmt)
                    activation columns: us per call against the HBM and the
                    fp32 vector-ALU rooflines
  --workload chain  the token as 145 dependent groups (each group's
                    activation is the quantized output of the previous one),
                    one fused launch per group: ms per token launched eagerly
                    and replayed from a graph, beside the two-launch version
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
VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector
# algorithmic bytes of one decode token (weights + q + d + y of the 253 products)
TOKEN_BYTES = {"Q1_0": 1071847552, "Q2_0": 2136111232}
PROFILES = {"Q1_0": os.path.join(ROOT, "profiles", "sweep_kernel_q1_0_decode_token.json"),
            "Q2_0": os.path.join(ROOT, "profiles", "sweep_kernel_q2_0_decode_token.json")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(fmt_name: str):
    """HBM bytes per sweep launch from the committed rocprofv3 counter summary,
    or None when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        with open(PROFILES[fmt_name]) as f:
            prof = json.load(f)
        h = hashlib.sha256()
        for p in prof["kernel_sources"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest() != prof.get("kernel_sources_sha256"):
        return None
    return prof.get("traffic_bytes_per_launch")


def host_cpus() -> dict:
    """What the host offers: logical CPUs, the ones this process may run on,
    and the CPU model."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"logical_cpus": os.cpu_count(), "affinity_cpus": aff, "model": model}


# A GPU machine gives one GPU's job a share of 16 host threads, whatever the host
# has in all; the oracle's thread pool is sized to that share.
BOX_THREADS = 16


def cpu_threads() -> int:
    return max(1, min(host_cpus()["affinity_cpus"], BOX_THREADS))


def oracle_leg(sw, y_gpu: np.ndarray, budget_s: float, threads: int):
    """The CPU oracle on a bounded sample of the same token: whole products,
    taken in sweep order until about budget_s seconds of work, at `threads`
    threads.  Also checks the GPU's outputs for those products bit for bit."""
    import oracle

    q_ref, d_ref, _ = oracle.quantize_q8(sw.x, sw.qa, sw.f16_scale)
    done_bytes = 0
    secs = 0.0
    mismatched = 0
    max_rel = 0.0
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
        ref = np.abs(y.astype(np.float64))
        err = np.abs(yg.astype(np.float64) - y.astype(np.float64))
        max_rel = max(max_rel, float(np.max(np.where(ref > 0, err / np.where(ref > 0, ref, 1.0), err), initial=0.0)))
        n += 1
        if secs >= budget_s:
            break
    return {"threads": threads, "value": round(done_bytes / secs / 1e9, 4), "unit": "GB/s",
            "s_per_token_equiv": round(sw.sweep_bytes() / (done_bytes / secs), 3),
            "sample": f"first {n} of {len(sw.shapes)} products of the token ({done_bytes / 1e9:.3f} GB, "
                      f"{secs:.1f} s); quantizer excluded",
            "gpu_outputs_checked": int(sum(r for _, r, _ in sw.shapes[:n])),
            "gpu_outputs_mismatched": mismatched, "gpu_max_rel_err": max_rel}


def host_floor_leg(threads: int) -> dict:
    """The host's streaming-read floor over 768 MiB (the pages' buffer) and
    4 GiB, at 1, 2, 4, ... threads up to `threads` (median of 3 passes)."""
    import oracle

    counts = sorted({1, threads} | {t for t in (2, 4, 8, 16) if t < threads})
    out = {"threads": counts}
    for name, nbytes in (("768MiB", 768 << 20), ("4GiB", 4 << 30)):
        out[name + "_GB_s"] = [round(v, 2) for v in oracle.host_read_floor(nbytes, counts, 3)]
    return out


def cpu_baseline(sw, y_gpu: np.ndarray, budget_s: float):
    """The oracle timed on the host: at all the threads this job may use (the
    headline cpu_baseline figure) and at one thread, plus the host's memory
    floor; GPU outputs are checked bit for bit by both legs."""
    host = host_cpus()
    threads = cpu_threads()
    full = oracle_leg(sw, y_gpu, budget_s, threads)
    one = oracle_leg(sw, y_gpu, budget_s / 2, 1)
    try:
        floor = host_floor_leg(threads)
    except Exception as e:  # context only
        floor = {"error": f"{type(e).__name__}: {e}"}
    return {
        "value": full["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": full["sample"],
        "ms_per_token_equiv": round(full["s_per_token_equiv"] * 1e3, 1),
        # both legs take products in sweep order, so the larger sample holds the smaller
        "gpu_outputs_checked": max(full["gpu_outputs_checked"], one["gpu_outputs_checked"]),
        "gpu_outputs_mismatched": max(full["gpu_outputs_mismatched"], one["gpu_outputs_mismatched"]),
        "gpu_max_rel_err": max(full["gpu_max_rel_err"], one["gpu_max_rel_err"]),
        "one_thread": {k: one[k] for k in ("value", "unit", "s_per_token_equiv", "sample")},
        "host": dict(host, threads_used=threads,
                     why=f"a GPU job's share of the host is {BOX_THREADS} threads; the oracle's pool is "
                         "sized to min(affinity, that share)"),
        "host_memory_floor": floor,
    }


def timed_calls(fn, reps: int) -> float:
    """Mean microseconds per call of fn(i) over reps back-to-back calls on the
    current stream: the calls are captured once in a graph and the replay is
    timed with HIP events, so the figure is the GPU's time per call (kernel
    plus the launch gap between kernels), not the host's launch rate."""
    import torch

    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(reps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / reps


def read_floor(gib: float = 1.0, reps: int = 20) -> dict:
    """The streaming-read floor of this GPU, measured live: bq_read_floor over
    a buffer four times the last-level cache, median of reps event-timed
    launches after a warm-up."""
    import torch
    import ternary_quantized_gemv_amd as bq

    nbytes = int(gib * (1 << 30))
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(bq.BQ_FLOOR_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        bq.bq_read_floor(buf, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        bq.bq_read_floor(buf, sink)
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    del buf, sink
    torch.cuda.empty_cache()
    gbs = nbytes / us / 1e3
    return {"value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "how": f"bq_read_floor: one streaming read of {gib:g} GiB, median of {reps} launches"}


def weight_copies(bq, fmt, rows, cols, seed, total=1.1e9, cap=512):
    """Device copies of one packed matrix, enough to total about 1.1 GB, so a
    timed batch that cycles through them streams from HBM (the 256 MB
    last-level cache cannot hold them)."""
    import synth

    canon = synth.blocks(fmt, rows, cols, seed, rows)
    w0 = bq.Weights.upload(fmt, canon, rows, cols)
    n = max(1, min(cap, int(total // canon.size)))
    ws = [w0] + [bq.Weights(fmt, rows, cols, w0.bits.clone(), w0.scales.clone()) for _ in range(n - 1)]
    return ws, canon.size


def quantized_columns(bq, cols, ncols, seed):
    import torch
    import synth

    x = torch.from_numpy(np.stack([synth.activation(cols, seed, 500 + c) for c in range(ncols)])).to("cuda")
    q = torch.empty((ncols, cols), dtype=torch.int8, device="cuda")
    d = torch.empty((ncols, cols // 128), dtype=torch.float32, device="cuda")
    for c in range(ncols):
        bq.bq_quantize_act_q8(x[c], 128, q[c], d[c])
    return bq.Act(q, d, cols, 128, ncols)


def bench_gemv(args):
    import torch
    import ternary_quantized_gemv_amd as bq

    shapes = [(bq.BQ_Q1_0, 4096, 4096), (bq.BQ_Q1_0, 12288, 4096), (bq.BQ_Q1_0, 4096, 12288),
              (bq.BQ_Q1_0, 151936, 4096), (bq.BQ_Q2_0, 4096, 4096), (bq.BQ_Q2_0, 1024, 4096),
              (bq.BQ_Q2_0, 12288, 4096), (bq.BQ_Q2_0, 4096, 12288)]
    floor = read_floor()
    rows_out = []
    for fmt, rows, cols in shapes:
        ws, wbytes = weight_copies(bq, fmt, rows, cols, args.seed)
        a = quantized_columns(bq, cols, 1, args.seed)
        y = torch.empty(rows, device="cuda")
        f = bq.bq_q1_0_matvec if fmt == bq.BQ_Q1_0 else bq.bq_q2_0_matvec
        us = timed_calls(lambda i: f(ws[i % len(ws)], a, y), max(args.steps, 2 * len(ws)))
        nbytes = wbytes + cols + 4 * (cols // 128) + 4 * rows
        gbs = nbytes / us / 1e3
        name = "Q1_0" if fmt == bq.BQ_Q1_0 else "Q2_0"
        rows_out.append({"fmt": name, "shape": f"{rows}x{cols}", "us_per_product": round(us, 2),
                         "algorithmic_bytes": nbytes, "GB_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "frac_of_floor": round(gbs / floor["value"], 4),
                         "ms_per_token_equiv": round(TOKEN_BYTES[name] / (gbs * 1e9) * 1e3, 3),
                         "weight_copies": len(ws)})
        log(f"gemv {name} {rows}x{cols}: {us:.2f} us, {gbs:.0f} GB/s")
        del ws
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "single-product us and HBM GB/s (% of peak) at the configured shapes",
                      "unit": "us", "higher_is_better": False, "n_gpus": 1,
                      "dtype": "int8xQ->f32", "data": "synthetic (seeded)",
                      "config": {"workload": "single Q1_0 / Q2_0 products, one activation vector, qa 128; "
                                             "each timed batch cycles through ~1.1 GB of weight copies"},
                      "k_floor": floor, "results": rows_out}), flush=True)


def bench_batch(args):
    """Small batch: us per call of bq_q1_0_matvec / bq_q2_0_matvec with N
    activation columns, weights cycled from ~1.1 GB of copies; for N >= 2 the
    table and matrix-core paths are each timed beside the automatic choice."""
    import torch
    import ternary_quantized_gemv_amd as bq

    fmt = bq.BQ_Q1_0 if args.fmt == "q1_0" else bq.BQ_Q2_0
    name = "Q1_0" if fmt == bq.BQ_Q1_0 else "Q2_0"
    f = bq.bq_q1_0_matvec if fmt == bq.BQ_Q1_0 else bq.bq_q2_0_matvec
    rows_out = []
    for rows in (12288, 151936):
        cols = 4096
        ws, wbytes = weight_copies(bq, fmt, rows, cols, args.seed)
        for ncols in (1, 4, 8, 16):
            a = quantized_columns(bq, cols, ncols, args.seed)
            y = torch.empty(ncols * rows, device="cuda")
            reps = max(args.steps // 4, 2 * len(ws))
            paths = {}
            if ncols >= 2:
                paths.update({"tables": bq.BQ_BATCH_TABLES, "mfma": bq.BQ_BATCH_MFMA})
            paths["auto"] = bq.BQ_BATCH_AUTO  # timed last, after both forced paths
            times = {}
            for pname, path in paths.items():
                prev = bq.bq_set_batch_path(path)
                try:
                    times[pname] = timed_calls(lambda i: f(ws[i % len(ws)], a, y), reps)
                finally:
                    bq.bq_set_batch_path(prev)
            us = times["auto"]
            nbytes = wbytes + ncols * (cols + 4 * (cols // 128) + 4 * rows)
            # f32 chain operations per weight per column: Q1_0 0.3125 (5 per lane group of a
            # 128-weight block: d1*s, three fmas, the block's fma), Q2_0 0.375 (3 per 64 weights)
            flops = rows * cols * ncols * (0.625 if fmt == bq.BQ_Q1_0 else 0.75)
            hbm_us = nbytes / (HBM_PEAK_GBS * 1e3)
            valu_us = flops / (VALU_PEAK_TFLOPS * 1e6)
            bound = "hbm" if hbm_us >= valu_us else "alu"
            row = {"shape": f"{rows}x{cols}", "ncols": ncols, "us_per_call": round(us, 2),
                   "GB_s": round(nbytes / us / 1e3, 1), "TFLOP_s": round(flops / us / 1e6, 2),
                   "bound": bound, "roofline_us": round(max(hbm_us, valu_us), 2),
                   "frac": round(max(hbm_us, valu_us) / us, 4)}
            if ncols >= 2:
                row["us_tables"] = round(times["tables"], 2)
                row["us_mfma"] = round(times["mfma"], 2)
            rows_out.append(row)
            log(f"batch {name} {rows}x{cols} N={ncols}: " + ", ".join(f"{k} {v:.2f} us" for k, v in times.items()))
        del ws
        torch.cuda.empty_cache()
    print(json.dumps({"metric": f"small-batch {name} us per call against the HBM and fp32 vector rooflines",
                      "unit": "us", "higher_is_better": False, "n_gpus": 1,
                      "dtype": f"int8x{name}->f32", "data": "synthetic (seeded)",
                      "config": {"workload": f"{name} 12288x4096 and 151936x4096, N = 1, 4, 8, 16 activation "
                                             "columns, qa 128; peaks 8 TB/s and 157.3 TFLOP/s; us_tables / "
                                             "us_mfma: the lane-group sums from LDS tables or the matrix cores"},
                      "results": rows_out}), flush=True)


def chain_timing(fmt, canon, shapes, x0, fused: bool, K: int, W: int):
    """The dependency-ordered decode token (staging.StagedChain): ms per token
    launched eagerly and replayed from a captured graph, and the outputs."""
    import torch
    from ternary_quantized_gemv_amd.staging import StagedChain

    def per_token(fn):
        for _ in range(W):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ch = StagedChain(fmt, canon, shapes, x0, fused=fused)
    try:
        eager_ms = per_token(ch.run)
        ref = ch.y.cpu().numpy()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ch.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            ch.run()
        graph_ms = per_token(graph.replay)
        same = bool(np.array_equal(ch.y.cpu().numpy().view(np.uint32), ref.view(np.uint32)))
        out = {"launches_per_token": ch.launches(), "token_bytes": ch.token_bytes(),
               "eager_ms_per_token": round(eager_ms, 4), "graph_ms_per_token": round(graph_ms, 4),
               "graph_GB_s": round(ch.token_bytes() / (graph_ms * 1e-3) / 1e9, 1),
               "graph_replay_equals_eager": same}
        del graph
    finally:
        ch.close()
    return out, ref


def bench_chain(args):
    import synth
    import ternary_quantized_gemv_amd as bq

    fmt = bq.BQ_Q1_0 if args.fmt == "q1_0" else bq.BQ_Q2_0
    shapes = synth.decode_sweep_shapes()
    canon = [synth.blocks(fmt, r, c, args.seed, i) for i, (_, r, c) in enumerate(shapes)]
    x0 = synth.activation(shapes[0][2], args.seed, 999)
    K, W = max(20, args.steps // 4), max(5, args.warmup // 10)
    fused, y_fused = chain_timing(fmt, canon, shapes, x0, True, K, W)
    split, y_split = chain_timing(fmt, canon, shapes, x0, False, K, W)
    name = "Q1_0" if fmt == bq.BQ_Q1_0 else "Q2_0"
    print(json.dumps({"metric": f"ms per token for the {name} decode token as 145 dependent groups",
                      "value": fused["graph_ms_per_token"], "unit": "ms", "higher_is_better": False,
                      "n_gpus": 1, "dtype": f"int8x{name}->f32", "data": "synthetic (seeded)",
                      "config": {"workload": "36 layers x ({q,k,v}, {o}, {gate,up}, {down}) + {lm_head}; each "
                                             "group's activation is the quantized f32 output of the previous "
                                             "group; value = one fused launch per group, graph replay"},
                      "fused": fused, "quantize_then_sweep": split,
                      "fused_equals_quantize_then_sweep": bool(np.array_equal(y_fused.view(np.uint32),
                                                                              y_split.view(np.uint32)))}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--fmt", choices=["q1_0", "q2_0"], default="q1_0")
    ap.add_argument("--workload", choices=["sweep", "gemv", "batch", "chain"], default="sweep")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--act", choices=["q8_128", "q8_0"], default="q8_128",
                    help="sweep activations: qa 128 with f32 scales, or qa 32 with f16-valued scales")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of back-to-back steps before the W warm-up steps (untimed)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache sweep timing")
    ap.add_argument("--no-chain", action="store_true", help="skip the decode-chain context field")
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
    if args.workload == "gemv":
        return bench_gemv(args)
    if args.workload == "batch":
        return bench_batch(args)
    if args.workload == "chain":
        return bench_chain(args)
    fmt = bq.BQ_Q1_0 if args.fmt == "q1_0" else bq.BQ_Q2_0
    shapes = synth.decode_sweep_shapes()
    t0 = time.time()
    canon = [synth.blocks(fmt, r, c, args.seed, i) for i, (_, r, c) in enumerate(shapes)]
    x = [synth.activation(c, args.seed, 1000 + i) for i, (_, _, c) in enumerate(shapes)]
    q8_0 = args.act == "q8_0"
    sw = StagedSweep(fmt, canon, shapes, x, qa=32 if q8_0 else 128, f16_scale=q8_0)
    log(f"staged {len(shapes)} products, {sw.weight_bytes / 1e9:.3f} GB of weights in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    K = args.steps

    def event_pairs(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    # the step, back to back, for a fixed time: the GPU's clocks ramp over
    # the first ~100 launches, so every timed leg below starts settled
    def settle(seconds):
        t_settle, n = time.perf_counter(), 0
        while time.perf_counter() - t_settle < seconds:
            for _ in range(50):
                sw.run()
            n += 50
            torch.cuda.synchronize()
        return n

    # ---- context legs, run BEFORE the timed loop so that the headline is
    # taken on a GPU that has been busy for a while (clocks settled)
    floor = read_floor()
    log(f"streaming-read floor {floor['value']:.0f} GB/s")
    sw.run()
    torch.cuda.synchronize()
    y_ref = sw.y.cpu().numpy()
    settle_legs = settle(args.settle)

    # the sweep with the 256 MB last-level cache flushed before each launch (a
    # streaming read of 512 MB between launches, outside the events; a read
    # leaves no dirty lines to write back during the sweep)
    cold = None
    if not args.no_cold:
        try:
            scratch = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
            sink = torch.empty(bq.BQ_FLOOR_SINK_WORDS, dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            cev = event_pairs(20)
            for b, c in cev:
                bq.bq_read_floor(scratch, sink)
                b.record(stream)
                sw.sweep()
                c.record(stream)
            torch.cuda.synchronize()
            cms = np.array([b.elapsed_time(c) for b, c in cev])
            cold = {"mean": round(float(cms.mean()), 5), "median": round(float(np.median(cms)), 5)}
            del scratch, sink
            log(f"sweep after a 512 MB cache flush: {cold['median'] * 1e3:.1f} us (median of 20)")
        except Exception as e:  # context only; the headline line must print regardless
            log(f"cold-cache timing skipped: {type(e).__name__}: {e}")

    # the same token in ONE launch that quantizes the f32 activations itself
    # (bq_sweep_create_x), checked against the two-launch outputs bit for bit
    fused = None
    if not q8_0:
        try:
            sw.y.fill_(float("nan"))
            sw.sweep_fused()
            torch.cuda.synchronize()
            same = bool(np.array_equal(sw.y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)))
            nf = max(K, 20)
            fev = event_pairs(nf)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for b, c in fev:
                b.record(stream)
                sw.sweep_fused()
                c.record(stream)
            torch.cuda.synchronize()
            f_ms = (time.perf_counter() - t0) * 1e3 / nf
            fk = np.array([b.elapsed_time(c) for b, c in fev])
            fused = {"ms_per_step": round(f_ms, 5), "value": round(sw.fused_bytes() / (f_ms * 1e-3) / 1e9, 2),
                     "kernel_ms": round(float(fk.mean()), 5), "kernel_ms_median": round(float(np.median(fk)), 5),
                     "bytes_per_launch": sw.fused_bytes(),
                     "kernel_GB_s": round(sw.fused_bytes() / (float(fk.mean()) * 1e-3) / 1e9, 2),
                     "same_bits_as_two_launch": same,
                     "how": "one bq_token_sweep launch of a bq_sweep_create_x plan (f32 activations quantized "
                            "in the launch)"}
            log(f"one-launch token: {f_ms * 1e3:.1f} us per step, kernel {np.median(fk) * 1e3:.1f} us (median), "
                f"same bits: {same}")
        except Exception as e:  # the headline line must print regardless
            fused = {"error": f"{type(e).__name__}: {e}"}

    # settle again, then the W warm-up steps the command asks for
    settle_steps = settle(args.settle)
    for _ in range(args.warmup):
        sw.run()
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps.  Events bracket each sweep
    # launch only (a marker before the quantizer measured ~4 us more per
    # step); the quantizer's share is the time from one sweep's end to the
    # next one's start (its kernel and the two launch gaps).
    ev = event_pairs(K)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        b, c = ev[k]
        sw.quantize()
        b.record(stream)
        sw.sweep()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    quant_ms = float(np.mean([ev[k - 1][1].elapsed_time(ev[k][0]) for k in range(1, K)])) if K > 1 else 0.0
    sweep_ms_all = np.array([b.elapsed_time(c) for b, c in ev])
    sweep_ms = float(np.mean(sweep_ms_all))
    ms_per_step = wall * 1e3 / K
    y_gpu = sw.y.cpu().numpy()
    same_as_first = bool(np.array_equal(y_gpu.view(np.uint32), y_ref.view(np.uint32)))

    step_bytes = sw.sweep_bytes() + sw.quantize_bytes()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = sw.sweep_bytes() / (sweep_ms * 1e-3) / 1e9
    log(f"timed: {K} steps, {ms_per_step * 1e3:.1f} us per step; sweep events mean {sweep_ms * 1e3:.1f} us, "
        f"median {np.median(sweep_ms_all) * 1e3:.1f} us")

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device-to-device copies done")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(sw, y_gpu, args.cpu_budget)
        log(f"cpu oracle: {cpu['value']} GB/s at {cpu['cores']} threads, {cpu['one_thread']['value']} GB/s at 1")

    # context, not the headline: the same products as a dependency-ordered
    # decode (145 groups, each the quantized output of the one before)
    chain = None
    if not args.no_chain and not q8_0:
        try:
            out, _ = chain_timing(fmt, canon, shapes, x[0], True, 40, 10)
            chain = {"ms_per_token": out["graph_ms_per_token"], "eager_ms_per_token": out["eager_ms_per_token"],
                     "launches_per_token": out["launches_per_token"],
                     "how": "bench.py --workload chain: one fused quantize+product launch per group, graph replay"}
        except Exception as e:  # the headline line must print regardless
            chain = {"error": f"{type(e).__name__}: {e}"}

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
                        "+ lm_head 151936x4096 = 253 GEMVs, one activation vector each, "
                        + ("qa 32 with f16-valued scales (q8_0)" if q8_0 else "qa 128"),
            "products": len(shapes),
            "weight_bytes": sw.weight_bytes,
            "step_bytes": step_bytes,
            "launches_per_step": 2,
        },
        "kernels": {
            "sweep_ms": round(sweep_ms, 5),
            "sweep_ms_median": round(float(np.median(sweep_ms_all)), 5),
            "sweep_ms_min": round(float(sweep_ms_all.min()), 5),
            "quantize_with_gaps_ms": round(quant_ms, 5),
            "sweep_ms_cold_cache": cold,
        },
        "before_timing": {"settle_s": args.settle, "settle_steps": [settle_legs, settle_steps],
                          "how": "the floor read, the step back to back for settle_s, the context legs "
                                 "(cold-cache and one-launch sweeps), the step back to back for settle_s again, "
                                 "then the W warm-up steps; outputs of the timed steps equal the first step's "
                                 "bit for bit: " + str(same_as_first)},
        "roofline": {
            "bound": "hbm",
            "kernel": "bq::sweep_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_of_floor": round(achieved / floor["value"], 4),
            "traffic": None if q8_0 else measured_traffic(fmt_name),
            "algorithmic_bytes_per_launch": sw.sweep_bytes(),
        },
        "per_matmul": {
            "us": round(ms_per_step * 1e3 / len(shapes), 4),
            "roofline_us": round(step_bytes / len(shapes) / (HBM_PEAK_GBS * 1e3), 4),
            "frac": round(value / HBM_PEAK_GBS, 4),
        },
        "per_token": {
            "ms": round(ms_per_step, 5),
            "roofline_ms": round(step_bytes / (HBM_PEAK_GBS * 1e6), 5),
            "frac": round(value / HBM_PEAK_GBS, 4),
            "frac_of_floor": round(value / floor["value"], 4),
        },
        "k_floor": floor,
        "cpu_baseline": cpu,
        "pages_cpu_context": {
            "memory_floor_GB_s": [14.9, 17.2],
            "ternary_token_s_at_3_threads": [0.23, 0.25],
            "machine": "the pages' laptop CPU (other hardware; context, not the target)",
        },
        "one_launch_token": fused,
        "decode_chain": chain,
    }
    sw.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
