"""Benchmark of the W4A16 dequantize-matmul hot path on one MI355X.

One step = the seven dequantize-matmuls of a Llama-3-8B-shaped decoder layer at
decode batch M = 1 (q, k, v, o: 4096 -> 4096/1024; gate, up: 4096 -> 14336;
down: 14336 -> 4096), group 128, AWQ scale s, each launched through the C ABI on
torch's current stream.  Inputs are resident in HBM before timing starts; the
packed weights rotate over enough layer copies (>= 1 GiB) that each step reads
weights from HBM rather than from the 256 MB last-level cache.

Printed JSON line (rank 0):
  value      aggregate HBM throughput of the step: algorithmic bytes per step
             (packed codes + fp16 scales/zeros + s + X + Y) / wall time per step;
  roofline   the dominant kernel's achieved bandwidth: its algorithmic bytes per
             launch / its average launch duration from HIP events recorded on the
             launch stream around every launch of the timed region;
  prefill    the 70B-shaped layer at M = 4096 (compute-bound): TFLOP/s against
             the dense fp16 MFMA peak, same method;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, published
POOL_BYTES = 1 << 30         # rotate weight copies over at least this much memory
METRIC = "W4A16 dequant-GEMM: HBM TB/s @M=1, TFLOP/s @M=4096, % of roofline"


def alg_bytes(M, N, K, awq):
    """Bytes the method must move: packed codes, fp16 scale + zero per group, s, X, Y."""
    return N * K // 2 + 4 * N * K // 128 + (2 * K if awq else 0) + 2 * M * K + 2 * M * N


def prepare_layer(cfg, M, torch, w4, workloads, copies_min_bytes=POOL_BYTES):
    """Pack every matrix of a configuration once on the GPU; replicate the packed
    buffers into enough copies to cover `copies_min_bytes`."""
    mats = []
    for mi, mat in enumerate(cfg.matrices):
        W = workloads.weights(cfg.weight_key, mi, mat.N, mat.K, threads=16)
        s = workloads.awq_scales(cfg.weight_key, mi, mat.K) if cfg.awq else None
        Wd = torch.from_numpy(W).to("cuda")
        sd = None if s is None else torch.from_numpy(s).to("cuda")
        del W
        pw = w4.w4a16_quantize_pack(Wd, sd)
        del Wd
        X = torch.from_numpy(workloads.activations(cfg.weight_key, mi, M, mat.K,
                                                   outliers=cfg.act_outliers)).to("cuda")
        Y = torch.empty((M, mat.N), dtype=torch.float16, device="cuda")
        mats.append(dict(name=mat.name, N=mat.N, K=mat.K, pw=pw, s=sd, X=X, Y=Y,
                         bytes=alg_bytes(M, mat.N, mat.K, sd is not None),
                         flops=2 * M * mat.N * mat.K))
    layer_w = sum(m["pw"].wq.numel() + 2 * m["pw"].scales.numel() * 2 for m in mats)
    copies = max(1, -(-copies_min_bytes // layer_w))
    pool = []
    for _ in range(copies):
        pool.append([w4.PackedWeight(m["pw"].wq.clone(), m["pw"].scales.clone(),
                                     m["pw"].zeros.clone(), m["N"], m["K"]) for m in mats])
    torch.cuda.synchronize()
    return mats, pool, layer_w


def timed_steps(mats, pool, steps, warmup, torch, w4, per_launch_events=True):
    """Run warmup + steps; return (wall seconds, per-matrix list of launch ms)."""
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        layer = pool[i % len(pool)]
        for j, m in enumerate(mats):
            if evs is not None:
                evs[j][0].record(stream)
            w4.w4a16_gemm(m["X"], layer[j], m["s"], out=m["Y"])
            if evs is not None:
                evs[j][1].record(stream)

    for i in range(warmup):
        step(i)
    events = []
    if per_launch_events:
        events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                   for _ in mats] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, events[i] if per_launch_events else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [[ev[j][0].elapsed_time(ev[j][1]) for ev in events] for j in range(len(mats))]
    return wall, launch_ms


def kernel_groups(mats, M, w4):
    """Group the launches by the kernel instance they run (same kernel name in a trace)."""
    groups = {}
    for j, m in enumerate(mats):
        path = w4.w4a16_select_path(M, m["N"], m["K"])
        if path == w4.PATH_SKINNY:
            chunks = (m["K"] // 128 + 3) // 4
            waves = 2 if chunks <= 2 else 4 if chunks <= 4 else 8 if chunks <= 8 else 16
            name = f"skinny_kernel<{waves},4>"
        else:
            name = "tiled_kernel"
        groups.setdefault(name, []).append(j)
    return groups


def roofline_of(mats, launch_ms, groups, bound):
    """The dominant kernel instance (largest share of the step's launch time)."""
    best = None
    for name, idx in groups.items():
        tot_ms = sum(sum(launch_ms[j]) for j in idx)
        n_launch = sum(len(launch_ms[j]) for j in idx)
        if best is None or tot_ms > best[1]:
            best = (name, tot_ms, n_launch, idx)
    name, tot_ms, n_launch, idx = best
    avg_ms = tot_ms / n_launch
    per_launch = sum(mats[j]["bytes" if bound == "hbm" else "flops"] for j in idx) / len(idx)
    if bound == "hbm":
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        peak, unit = FP16_PEAK_TFLOPS, "TFLOP/s"
    return {"bound": bound, "kernel": name, "launches_per_step": len(idx),
            "avg_launch_us": round(avg_ms * 1e3, 3), "per_launch": per_launch,
            "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None}


def per_matrix(mats, launch_ms, bound):
    out = {}
    for j, m in enumerate(mats):
        ms = float(np.median(launch_ms[j]))
        if bound == "hbm":
            out[m["name"]] = {"us": round(ms * 1e3, 2), "TB/s": round(m["bytes"] / ms / 1e9, 3)}
        else:
            out[m["name"]] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(m["flops"] / ms / 1e9, 1)}
    return out


def cpu_baseline(cfg, M, workloads, rows=1024, budget_s=10.0):
    """The fp64 oracle (dequantize then matmul), timed on this host on a bounded
    sample of the workload: the first `rows` rows of every matrix, quantized by
    the oracle beforehand (untimed), then oracle.gemm repeated over the sample
    until about `budget_s` have passed.  Reported as TB/s of algorithmic bytes."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    parts = []
    for mi, mat in enumerate(cfg.matrices):
        n = min(rows, mat.N)
        Wr = workloads.weight_rows(cfg.weight_key, mi, mat.N, mat.K, 0, n)
        s = workloads.awq_scales(cfg.weight_key, mi, mat.K) if cfg.awq else None
        X = workloads.activations(cfg.weight_key, mi, M, mat.K, outliers=cfg.act_outliers)
        parts.append((X, oracle.quantize(Wr, s), s, n, mat.K))
    byts, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for X, ref, s, n, K in parts:
            oracle.gemm(X, ref.q, ref.scales, ref.zeros, s)
            byts += alg_bytes(M, n, K, s is not None)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    return {"value": byts / dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {rows} rows of each of the {len(cfg.matrices)} matrices of "
                      f"{cfg.name} at M={M}, oracle.gemm (fp64 dequantize + matmul) "
                      f"repeated {reps}x"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_int4_group_amd as w4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w4.lib()  # fail loudly if the HIP library is missing
    cfg = workloads.config_by_name(args.workload)
    M = cfg.Ms[0]
    print(f"[bench] preparing {cfg.name} M={M}", file=sys.stderr, flush=True)
    mats, pool, layer_w = prepare_layer(cfg, M, torch, w4, workloads)
    step_bytes = sum(m["bytes"] for m in mats)
    print(f"[bench] {len(pool)} layer copies, {layer_w * len(pool) / 2**30:.2f} GiB of packed "
          f"weights; timing {args.steps} steps", file=sys.stderr, flush=True)
    wall, launch_ms = timed_steps(mats, pool, args.steps, args.warmup, torch, w4)
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (ms_per_step * 1e-3) / 1e12
    roof = roofline_of(mats, launch_ms, kernel_groups(mats, M, w4), "hbm")

    out = {
        "metric": METRIC, "value": round(value, 4), "unit": "TB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Llama-3-8B-shaped decoder layer (7 matrices), "
                               f"M={M}, group 128, AWQ s, asym uint4 + fp16 scale/zero",
                   "M": M, "step_bytes": step_bytes, "weight_copies": len(pool),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "per_matrix": per_matrix(mats, launch_ms, "hbm"),
        "layer_kernel_TBps": round(step_bytes / (sum(sum(x) for x in launch_ms) /
                                                 args.steps * 1e-3) / 1e12, 4),
    }
    del pool, mats
    torch.cuda.empty_cache()

    if not args.no_prefill:
        pcfg = workloads.config_by_name("llama_70b_prefill")
        PM = pcfg.Ms[0]
        print(f"[bench] preparing {pcfg.name} M={PM}", file=sys.stderr, flush=True)
        pmats, ppool, _ = prepare_layer(pcfg, PM, torch, w4, workloads, copies_min_bytes=0)
        pwall, pms = timed_steps(pmats, ppool, args.prefill_steps, 2, torch, w4)
        flops = sum(m["flops"] for m in pmats)
        pstep = pwall / args.prefill_steps
        out["prefill"] = {
            "workload": f"{pcfg.name}: 70B-shaped layer (7 matrices), M={PM}, AWQ s, "
                        "1% activation channels x20",
            "TFLOP/s": round(flops / pstep / 1e12, 2), "ms_per_step": round(pstep * 1e3, 4),
            "frac_of_fp16_peak": round(flops / pstep / 1e12 / FP16_PEAK_TFLOPS, 4),
            "roofline": roofline_of(pmats, pms, kernel_groups(pmats, PM, w4), "mfma"),
            "per_matrix": per_matrix(pmats, pms, "mfma"),
        }
        del ppool, pmats
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, M, workloads)
        out["cpu_baseline"]["value"] = float(f"{out['cpu_baseline']['value']:.6g}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
