"""Benchmark of the W4A16 dequantize-matmul hot path on one MI355X.

One step = the seven dequantize-matmuls of a Llama-3-8B-shaped decoder layer at
decode batch M = 1 (q, k, v, o: 4096 -> 4096/1024; gate, up: 4096 -> 14336;
down: 14336 -> 4096), group 128, AWQ scale s, each with its own seeded input.
The seven problems are independent here, so the step is ONE grouped launch
through the C ABI (w4a16_gemm_grouped) on torch's current stream.  (Replaying
the step from a captured HIP graph was measured slower on this stack than a
direct launch.)  Inputs are resident in HBM before timing starts; the packed
weights rotate over enough layer copies (>= 1 GiB) that each step streams its
weights from HBM rather than from the 256 MB last-level cache.

Printed JSON line:
  value         algorithmic bytes per step (packed codes + fp16 scales/zeros + s
                + X + Y) / wall time per step, in TB/s;
  roofline      the step's kernel (one launch per step): its algorithmic bytes /
                its average duration, from HIP events recorded on the launch
                stream around each block of 10 back-to-back launches of the
                timed region (so a launch's own event overhead is amortised);
  layer_variants  the same layer as 4 launches in a real layer's dependency
                order ([q,k,v], [o], [gate,up], [down]) and as 7 separate
                launches, timed the same way (context for the headline);
  batched       the same 8B layer at speculative-verify batches M = 2, 5, 9 and a
                Qwen2-7B-shaped layer at batched-decode M = 16, 64, 256, one grouped
                call per step (streaming kernel for M <= 16, else the tiled GEMM);
  outliers      the headline layer with each matrix's top 0.1% |W/s| kept in fp16
                and added by the kernels (one grouped launch per step); the prefill
                line carries the same variant of the 70B layer;
  bf16          the headline layer (and, in the prefill line, the 70B layer) with bf16
                activations and outputs on the same packed weights;
  gptq          the GPTQ packer (offline) on an 8B q projection: seconds and fp64 rate;
  spec_verify   the accept / reject / draw step after a K = 4 verify pass over the
                Llama-3 vocabulary (V = 128256), for 1 and 64 sequences per call;
  prefill       the 70B-shaped layer at M = 4096 (compute-bound): TFLOP/s
                against the dense fp16 MFMA peak;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload;
  ceilings      measured context, not targets: a plain 1 GiB device-to-device
                copy (read + write GB/s) and torch's dense fp16 GEMM (the
                vendor library, dense fp16 weights) at the 70B prefill shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, published
POOL_BYTES = 1 << 30         # rotate weight copies over at least this much memory
METRIC = "W4A16 dequant-GEMM: HBM TB/s @M=1, TFLOP/s @M=4096, % of roofline"


def alg_bytes(M, N, K, awq, bits=4):
    """Bytes the method must move: packed codes, fp16 scale + zero per group, s, X, Y."""
    return N * K * bits // 8 + 4 * N * K // 128 + (2 * K if awq else 0) + 2 * M * K + 2 * M * N


KERNEL_HEADERS = ("w4a16_device.h", "w4a16_internal.h")


def kernel_source_sha(name):
    """SHA-256 of a kernel source file followed by the device headers it includes, to
    tie a counter profile to the code it measured."""
    import hashlib
    h = hashlib.sha256()
    for part in (name,) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "weight_only_int4_group_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(summary, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, calibrated against a plain copy), or None when the kernel source has
    changed since the counters were taken (or there is no summary)."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_sha(source):
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def profile_run(torch, w4, workloads):
    """A short, fixed sequence for counter collection under rocprofv3: one 256 MiB
    device-to-device copy (the calibration kernel: its bytes are known), then 20
    grouped decode steps of the 8B layer and one launch per 70B prefill matrix."""
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    cfg = workloads.config_by_name("llama3_8b_decode")
    mats, pool, _, copies = prepare_layer(cfg, 1, torch, w4, workloads)
    calls = make_calls(mats, pool, copies, [list(range(len(mats)))], w4, torch)
    for i in range(20):
        calls[i % copies][0]()
    torch.cuda.synchronize()
    del calls, pool, mats
    pcfg = workloads.config_by_name("llama_70b_prefill")
    pmats, ppool, _, pc = prepare_layer(pcfg, pcfg.Ms[0], torch, w4, workloads, copies_min_bytes=0)
    for c in make_calls(pmats, ppool, pc, [[j] for j in range(len(pmats))], w4, torch)[0]:
        c()
    torch.cuda.synchronize()
    print("profile run done", flush=True)


def profile_run_batches(torch, w4, workloads, name, Ms):
    """A short sequence for wave-level counters: ten grouped calls of one layer
    configuration at each batch size in Ms (one launch per call, plus the split-K
    reduction where the tiled kernel splits K)."""
    cfg = workloads.config_by_name(name)
    for M in Ms:
        mats, pool, _, copies = prepare_layer(cfg, M, torch, w4, workloads, copies_min_bytes=0)
        calls = make_calls(mats, pool, copies, [list(range(len(mats)))], w4, torch)
        for i in range(10):
            calls[i % copies][0]()
        torch.cuda.synchronize()
        del calls, pool, mats
        print(f"profile run: {name} M={M} done", flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def outlier_bytes(pw):
    """Bytes of a packed weight's fp16 outliers: row pointers, columns and values."""
    if pw.o_row_ptr is None:
        return 0
    return 4 * pw.o_row_ptr.numel() + 6 * pw.o_col.numel()


def prepare_layer(cfg, M, torch, w4, workloads, copies_min_bytes=POOL_BYTES, outliers=False,
                  int8=False):
    """Pack every matrix of a configuration once on the GPU (with the 0.1% fp16 outliers
    when asked, or as INT8 codes), and replicate the packed buffers into enough copies to
    cover `copies_min_bytes`."""
    mats = []
    for mi, mat in enumerate(cfg.matrices):
        W = workloads.weights(cfg.weight_key, mi, mat.N, mat.K, threads=16)
        s = workloads.awq_scales(cfg.weight_key, mi, mat.K) if cfg.awq else None
        Wd = torch.from_numpy(W).to("cuda")
        sd = None if s is None else torch.from_numpy(s).to("cuda")
        del W
        if outliers:
            pw = w4.w4a16_quantize_pack_outliers(Wd, sd)
        else:
            pw = w4.w4a16_quantize_pack(Wd, sd, mode=w4.QUANT_ASYM8 if int8 else w4.QUANT_ASYM)
        del Wd
        X = torch.from_numpy(workloads.activations(cfg.weight_key, mi, M, mat.K,
                                                   outliers=cfg.act_outliers)).to("cuda")
        Y = torch.empty((M, mat.N), dtype=torch.float16, device="cuda")
        mats.append(dict(name=mat.name, N=mat.N, K=mat.K, pw=pw, s=sd, X=X, Y=Y,
                         bytes=alg_bytes(M, mat.N, mat.K, sd is not None, pw.wbits)
                         + outlier_bytes(pw),
                         flops=2 * M * mat.N * mat.K))
    layer_w = sum(m["pw"].wq.numel() + 4 * m["pw"].scales.numel() + outlier_bytes(m["pw"])
                  for m in mats)
    copies = max(1, -(-copies_min_bytes // layer_w))
    pool = [[m["pw"]] for m in mats] if copies == 1 else None
    if copies > 1:
        def clone(t):
            return None if t is None else t.clone()
        pool = [[w4.PackedWeight(m["pw"].wq.clone(), m["pw"].scales.clone(),
                                 m["pw"].zeros.clone(), m["N"], m["K"], clone(m["pw"].o_row_ptr),
                                 clone(m["pw"].o_col), clone(m["pw"].o_val), m["pw"].wbits)
                 for _ in range(copies)]
                for m in mats]
    torch.cuda.synchronize()
    return mats, pool, layer_w, copies


def make_calls(mats, pool, copies, groups, w4, torch):
    """For every layer copy, one prepared grouped call per group of matrix indices,
    bound to torch's current stream.  The copies of a group share one workspace (the
    calls run one after the other on that stream), as a serving loop would reuse it."""
    st = torch.cuda.current_stream().cuda_stream
    first = [w4.GroupedCall([(mats[j]["X"], pool[j][0], mats[j]["s"], mats[j]["Y"]) for j in grp],
                            stream=st) for grp in groups]
    return [first] + [[w4.GroupedCall([(mats[j]["X"], pool[j][c], mats[j]["s"], mats[j]["Y"])
                                       for j in grp], stream=st,
                                      workspace=f.ws if f.ws is not None else True)
                       for grp, f in zip(groups, first)] for c in range(1, copies)]


def timed(calls, steps, warmup, torch, per=10, min_warm_s=0.2):
    """Warm up (`warmup` steps, and on until the GPU has run them for at least
    `min_warm_s` seconds: after the host-side preparation of a workload the clocks
    need that long to settle), then run exactly `steps` steps (step i uses copy
    i % copies).  HIP events on the launch stream bracket every block of up to `per`
    consecutive launches of each kind.  Returns (wall seconds, per-launch ms [launch
    kind][block]) where a block's per-launch ms is its duration divided by its number
    of launches."""
    stream = torch.cuda.current_stream()
    nl = len(calls[0])
    t_w = time.perf_counter()
    done = 0
    while True:
        if done >= warmup and done % 64 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t_w >= min_warm_s:
                break
        for u in calls[done % len(calls)]:
            u()
        done += 1
    warmup = done
    blocks = [(b0, min(per, steps - b0)) for b0 in range(0, steps, per)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nl)] for _ in blocks]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (b0, n), evb in zip(blocks, ev):
        for j in range(nl):
            evb[j][0].record(stream)
            for i in range(n):
                calls[(warmup + b0 + i) % len(calls)][j]()
            evb[j][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [[evb[j][0].elapsed_time(evb[j][1]) / n for (_, n), evb in zip(blocks, ev)]
                  for j in range(nl)]


def with_batch(mats, cfg, M, torch, workloads):
    """The same packed matrices with new seeded activations of batch M."""
    out = []
    for mi, m in enumerate(mats):
        X = torch.from_numpy(workloads.activations(cfg.weight_key, mi, M, m["K"],
                                                   outliers=cfg.act_outliers)).to("cuda")
        Y = torch.empty((M, m["N"]), dtype=torch.float16, device="cuda")
        out.append(dict(m, X=X, Y=Y, bytes=alg_bytes(M, m["N"], m["K"], m["s"] is not None,
                                                     m["pw"].wbits),
                        flops=2 * M * m["N"] * m["K"]))
    return out


def with_bf16(mats, cfg, M, torch, workloads):
    """The same packed matrices with bf16 activations and outputs (the same draws as the
    fp16 activations, rounded to bf16)."""
    out = []
    for mi, m in enumerate(mats):
        bits = workloads.activations_bf16(cfg.weight_key, mi, M, m["K"], outliers=cfg.act_outliers)
        X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
        Y = torch.empty((M, m["N"]), dtype=torch.bfloat16, device="cuda")
        out.append(dict(m, X=X, Y=Y))
    return out


def batched_line(cfg, M, mats, pool, copies, w4, torch, workloads, steps=200, warmup=20):
    """One grouped call over the whole layer per step at batch M."""
    bm = with_batch(mats, cfg, M, torch, workloads)
    calls = make_calls(bm, pool, copies, [list(range(len(bm)))], w4, torch)
    split = calls[0][0].ws_bytes > 0  # K split across workgroups: + one reduction launch
    wall, lms = timed(calls, steps, warmup, torch)
    byts, fl = sum(m["bytes"] for m in bm), sum(m["flops"] for m in bm)
    kern = float(np.mean(lms[0])) * 1e-3
    path = "streaming" if w4.w4a16_select_path(M, mats[0]["N"], mats[0]["K"]) == w4.PATH_SKINNY \
        else "tiled"
    line = {"workload": cfg.name, "M": M, "kernel": path,
            "launches_per_step": 1 + int(split), "split_k": split,
            "us_per_step": round(wall / steps * 1e6, 2), "kernel_us_per_step": round(kern * 1e6, 2),
            "TB/s": round(byts / (wall / steps) / 1e12, 4),
            "kernel_TB/s": round(byts / kern / 1e12, 4),
            "TFLOP/s": round(fl / (wall / steps) / 1e12, 2)}
    if split:
        # the same layer through w4a16_gemm_grouped, the entry point without a workspace
        # argument (the library's shared scratch takes the split-K partials)
        st = torch.cuda.current_stream().cuda_stream
        ncalls = [[w4.GroupedCall([(m["X"], pool[j][c], m["s"], m["Y"]) for j, m in enumerate(bm)],
                                  stream=st, workspace=False)] for c in range(copies)]
        _, nms = timed(ncalls, steps, warmup, torch)
        nk = float(np.mean(nms[0])) * 1e-3
        line["no_workspace_arg"] = {"entry": "w4a16_gemm_grouped (library's shared scratch)",
                                    "kernel_us_per_step": round(nk * 1e6, 2),
                                    "vs_workspace_call": round(nk / kern, 4)}
    return line


SWEEP_MS = (17, 24, 32, 48, 64, 96, 128, 256)


def dispatch_sweep(torch, w4, workloads, steps=50, warmup=5):
    """The M-dispatch crossover, measured: for the 8B, Qwen2-7B and 70B layers and every
    M in SWEEP_MS, one layer step through the tiled GEMM (the grouped call with its
    workspace: what the dispatch picks above 16 rows) against the streaming kernel fed
    16-row pieces (each piece of every matrix one problem of the grouped call, so the
    weights are streamed once per 16 rows).  HIP events per layer step, weights rotated
    over copies like the decode benchmark."""
    rows = []
    for name in ("llama3_8b_decode", "qwen2_7b_batched_decode", "llama_70b_prefill"):
        cfg = workloads.config_by_name(name)
        log(f"dispatch sweep: preparing {cfg.name}")
        mats, pool, _, copies = prepare_layer(cfg, 1, torch, w4, workloads,
                                              copies_min_bytes=POOL_BYTES // 2)
        st = torch.cuda.current_stream().cuda_stream
        for M in SWEEP_MS:
            bm = with_batch(mats, cfg, M, torch, workloads)
            tiled = make_calls(bm, pool, copies, [list(range(len(bm)))], w4, torch)
            pieces = [[w4.GroupedCall([(m["X"][m0:m0 + 16], pool[j][c], m["s"], m["Y"][m0:m0 + 16])
                                       for j, m in enumerate(bm) for m0 in range(0, M, 16)],
                                      stream=st)] for c in range(copies)]
            _, tms = timed(tiled, steps, warmup, torch)
            _, sms = timed(pieces, steps, warmup, torch)
            t_us, s_us = float(np.mean(tms[0])) * 1e3, float(np.mean(sms[0])) * 1e3
            rows.append({"layer": cfg.name, "M": M, "tiled_us": round(t_us, 2),
                         "streaming_pieces_us": round(s_us, 2),
                         "faster": "tiled" if t_us <= s_us else "streaming"})
            log(f"  M={M}: tiled {t_us:.1f} us, streaming pieces {s_us:.1f} us")
            del bm, tiled, pieces
        del mats, pool
        torch.cuda.empty_cache()
    return rows


def gemv_line(torch, w4, workloads, steps=400, warmup=40):
    """The single 1024 x 1024 matrix at M = 1: 0.56 MB per call, far below what
    keeps HBM busy, so the time is launch latency, not bandwidth."""
    cfg = workloads.config_by_name("gemv_1024")
    mats, pool, _, copies = prepare_layer(cfg, 1, torch, w4, workloads)
    byts = sum(m["bytes"] for m in mats)
    wall, lms = timed(make_calls(mats, pool, copies, [[0]], w4, torch), steps, warmup, torch)
    kern = float(np.mean(lms[0])) * 1e-3
    return {"workload": f"{cfg.name}: one 1024x1024 matrix, M=1, no AWQ s, {copies} rotating "
                        "copies", "bytes": byts,
            "us_per_call": round(wall / steps * 1e6, 2), "kernel_us": round(kern * 1e6, 2),
            "kernel_TB/s": round(byts / kern / 1e12, 4),
            "frac_of_hbm_peak": round(byts / kern / 1e9 / HBM_PEAK_GBS, 4),
            "note": "launch-latency bound: the roofline time at 8 TB/s is 0.07 us"}


def variant(mats, groups, launch_ms, steps, wall, unit_key):
    step_units = sum(m[unit_key] for m in mats)
    kern = sum(float(np.mean(x)) for x in launch_ms)  # ms of kernel time per step
    out = {"launches_per_step": len(groups), "ms_per_step": round(wall / steps * 1e3, 5),
           "kernel_ms_per_step": round(kern, 5)}
    if unit_key == "bytes":
        out["TB/s"] = round(step_units / (wall / steps) / 1e12, 4)
        out["kernel_TB/s"] = round(step_units / (kern * 1e-3) / 1e12, 4)
    else:
        out["TFLOP/s"] = round(step_units / (wall / steps) / 1e12, 2)
    out["launches"] = [{"matrices": [mats[j]["name"] for j in grp],
                        "us": round(float(np.median(launch_ms[i])) * 1e3, 2),
                        "us_p10": round(float(np.percentile(launch_ms[i], 10)) * 1e3, 2),
                        "us_p90": round(float(np.percentile(launch_ms[i], 90)) * 1e3, 2)}
                       for i, grp in enumerate(groups)]
    return out


def spec_verify_line(torch, w4, B, K, V, steps=200, warmup=20, per=10):
    """Speculative-sampling verification (w4a16_spec_verify) of B sequences with K drafts
    over a V-token vocabulary.  The inputs are cloned into enough copies that the rows
    the calls touch exceed 1 GiB, so every call reads them from HBM.  Algorithmic bytes
    per call: the rows the outcome needs, read once (target and draft rows at a
    rejection, the target row after K acceptances), plus the K probes and the outputs."""
    from workloads import verify as wv
    host = wv.batch(7, B, K, V)
    base = [torch.from_numpy(a).to("cuda") for a in host]
    n, _ = w4.w4a16_spec_verify(*base)
    n = n.cpu().numpy()
    rows = int(np.sum(np.where(n < K, 2, 1)))
    call_bytes = rows * V * 4 + B * K * (4 + 4 + 4 + 4) + B * (4 + 8)
    copies = max(1, -(-(1 << 30) // call_bytes))
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    outs = [(torch.empty(B, dtype=torch.int32, device="cuda"),
             torch.empty(B, dtype=torch.int32, device="cuda")) for _ in range(copies)]
    ws = torch.empty(max(1, w4.w4a16_spec_verify_workspace_size(B, K, V)), dtype=torch.uint8,
                     device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    calls = [[w4.SpecVerifyCall(*sets[c], out=outs[c], workspace=ws, stream=st)]
             for c in range(copies)]
    wall, lms = timed(calls, steps, warmup, torch, per=per)
    kern = float(np.mean(lms[0])) * 1e-3
    return {"workload": f"spec_verify: B={B} sequences, K={K} drafts, V={V}, fp32 "
                        "probabilities, synthetic target/draft distributions",
            "B": B, "K": K, "V": V, "accepted_mean": round(float(n.mean()), 3),
            "copies": copies, "us_per_call": round(wall / steps * 1e6, 2),
            "kernel_us_per_call": round(kern * 1e6, 2), "call_bytes": call_bytes,
            "kernel_GB/s": round(call_bytes / kern / 1e9, 1),
            "frac_of_hbm_peak": round(call_bytes / kern / 1e9 / HBM_PEAK_GBS, 4)}


def gptq_line(torch, w4, N=4096, K=4096, n=4096, reps=3):
    """GPTQ quantize-and-pack of an 8B q projection (N x K, AWQ s) with n seeded
    calibration rows: wall seconds per call (blocking, offline) and the fp64 work it
    amounts to -- H = 2 X^T X (2 n K^2) and the compensation (about 2 N K^2: the
    in-group sweeps plus the trailing products) -- against the fp64 peak."""
    rng = np.random.default_rng(0)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float16)).to("cuda")
    s = torch.from_numpy(rng.lognormal(0.0, 0.5, K).astype(np.float16)).to("cuda")
    X = torch.from_numpy(rng.standard_normal((n, K)).astype(np.float16)).to("cuda")
    w4.w4a16_quantize_pack_gptq(W, s, X)  # loads the solver libraries
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        w4.w4a16_quantize_pack_gptq(W, s, X)
    sec = (time.perf_counter() - t0) / reps
    flops = 2.0 * n * K * K + 2.0 * N * K * K
    return {"workload": f"GPTQ pack of a {N}x{K} projection (AWQ s), {n} calibration rows",
            "seconds_per_matrix": round(sec, 4), "fp64_TFLOP/s": round(flops / sec / 1e12, 2),
            "frac_of_fp64_peak": round(flops / sec / 1e12 / 78.6, 4)}


def read_ceiling(torch, nbytes, launches=100, per=10):
    """The measured read-bandwidth ceiling for `nbytes` per launch: a plain HIP
    streaming-read kernel (libw4a16_ceiling.so, built with the library) reading one
    buffer of nbytes per launch, rotating over enough copies (>= 1 GiB) that every
    launch reads HBM, timed like the decode kernel (HIP events around blocks of `per`
    back-to-back launches on the launch stream).  Its variants (16-byte loads, 4, 8 or
    16 in flight per thread, 256 or 512 threads, with or without the non-temporal bit)
    and grid sizes are swept and the fastest is the ceiling.  Also the same kernel over
    one buffer (which then largely stays in the 256 MB last-level cache), for context."""
    import ctypes
    from weight_only_int4_group_amd.build import CEILING_LIB_PATH
    if not os.path.exists(CEILING_LIB_PATH):
        raise RuntimeError(f"{CEILING_LIB_PATH} is missing: build the library first")
    L = ctypes.CDLL(CEILING_LIB_PATH)
    L.stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p, ctypes.c_void_p]
    L.stream_read.restype = ctypes.c_int
    nbytes = -(-nbytes // 16) * 16
    copies = max(1, -(-POOL_BYTES // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 256)
            for _ in range(copies)]
    grids = (512, 1024, 2048, 4096)
    sink = torch.empty(max(grids) * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    def run(variant, blocks, pool):
        def go(i):
            rc = L.stream_read(pool[i % len(pool)].data_ptr(), nbytes, variant, blocks,
                               sink.data_ptr(), st)
            if rc:
                raise RuntimeError(f"stream_read failed: {rc}")
        for i in range(10):
            go(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(0, launches, per)]
        torch.cuda.synchronize()
        for b, (e0, e1) in enumerate(evs):
            e0.record(stream)
            for i in range(per):
                go(10 + b * per + i)
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) / per for e0, e1 in evs]))  # ms per launch

    table = []
    for variant in (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13):
        for blocks in grids:
            ms = run(variant, blocks, bufs)
            table.append({"variant": variant, "nt": bool(variant & 1),
                          "loads_in_flight": 4 << ((variant >> 1) & 3),
                          "threads": 512 if variant & 8 else 256, "workgroups": blocks,
                          "us": round(ms * 1e3, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    best = min(table, key=lambda r: r["us"])
    warm_ms = run(best["variant"], best["workgroups"], bufs[:1])
    del bufs, sink
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel (plain 16-byte streaming reads, libw4a16_ceiling.so)",
            "bytes_per_launch": nbytes, "copies": copies, "best": best,
            "same_buffer_GB/s": round(nbytes / (warm_ms * 1e-3) / 1e9, 1),
            "swept": len(table),
            "top5": sorted(table, key=lambda r: r["us"])[:5]}


def mfma_ceiling(torch, launches=20):
    """The measured dense fp16 matrix-core ceiling: a HIP kernel (libw4a16_ceiling.so)
    whose waves only issue independent 16x16x32 fp16 MFMAs from registers, about 2e12
    flops per launch, timed with HIP events around `launches` back-to-back launches
    after two untimed ones.  Chains per wave (8, 16, 32) and workgroups (one to four
    waves per SIMD) are swept; the fastest is the ceiling.  It shows the rate the
    matrix cores sustain at the clock they run at under full load, beside the
    nominal 2.5 PFLOP/s."""
    import ctypes
    from weight_only_int4_group_amd.build import CEILING_LIB_PATH
    if not os.path.exists(CEILING_LIB_PATH):
        raise RuntimeError(f"{CEILING_LIB_PATH} is missing: build the library first")
    L = ctypes.CDLL(CEILING_LIB_PATH)
    L.mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                            ctypes.c_void_p]
    L.mfma_peak.restype = ctypes.c_int
    grids = (256, 512, 1024)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    table = []
    for chains in (8, 16, 32):
        for blocks in grids:
            iters = max(1, int(2e12 / (blocks * 4 * chains * 16384)))
            flops = blocks * 4 * chains * iters * 16384

            def go():
                rc = L.mfma_peak(chains, blocks, iters, sink.data_ptr(), stream.cuda_stream)
                if rc:
                    raise RuntimeError(f"mfma_peak failed: {rc}")
            go()
            go()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(launches):
                go()
            e1.record(stream)
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / launches * 1e-3
            table.append({"chains": chains, "workgroups": blocks, "us": round(sec * 1e6, 1),
                          "TFLOP/s": round(flops / sec / 1e12, 1)})
    del sink
    best = max(table, key=lambda r: r["TFLOP/s"])
    return {"kernel": "mfma_peak_kernel (independent 16x16x32 fp16 MFMAs from registers, "
                      "libw4a16_ceiling.so)",
            "TFLOP/s": best["TFLOP/s"], "best": best,
            "frac_of_nominal": round(best["TFLOP/s"] / FP16_PEAK_TFLOPS, 4), "table": table}


def ceilings(torch, reps=10):
    """Measured ceilings on this GPU, for context: a plain device-to-device copy, and
    the vendor dense fp16 GEMM (torch.matmul on contiguous fp16 operands) at the 70B
    prefill shapes, M = 4096."""
    stream = torch.cuda.current_stream()

    def time_it(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3  # seconds per call

    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    t = time_it(lambda: b.copy_(a), reps)
    out = {"device_copy_GBps": round(2 * a.numel() / t / 1e9, 1),
           "device_copy": "1 GiB device-to-device copy_, read + write bytes / time"}
    del a, b
    gemm = {}
    M = 4096
    for name, N, K in (("q/o 8192x8192", 8192, 8192), ("gate/up 28672x8192", 28672, 8192),
                       ("down 8192x28672", 8192, 28672)):
        X = torch.randn(M, K, dtype=torch.float16, device="cuda")
        Wt = torch.randn(K, N, dtype=torch.float16, device="cuda")  # W^T, contiguous
        t = time_it(lambda: torch.matmul(X, Wt), reps)
        gemm[name] = round(2 * M * N * K / t / 1e12, 1)
        del X, Wt
    out["fp16_gemm_TFLOPs"] = gemm
    out["fp16_gemm"] = ("torch.matmul, fp16 X[4096][K] @ W^T[K][N] with dense fp16 weights "
                        "(4x the bytes of the packed INT4 weights); context, not a target")
    torch.cuda.empty_cache()
    return out


CPU_SAMPLE_ROWS = {"gemv_1024": 1024, "llama3_8b_decode": 512, "llama3_8b_verify": 512,
                   "qwen2_7b_batched_decode": 256, "llama_70b_prefill": 64}


def cpu_baseline(cfg, M, workloads, budget_s=10.0, item_s=1.0):
    """The fp64 CPU oracle as it stands (oracle.quantize / pack_codes / pack_meta and
    oracle.gemm = dequantize then one BLAS matmul), timed on this host.  Cores are the
    CPUs this process may run on (len(os.sched_getaffinity(0))); the BLAS thread count
    is set to that number.  Every timing runs on a bounded row sample, stated with it:
      * value: oracle.gemm over the first CPU_SAMPLE_ROWS rows of each matrix of the
        benchmark's own workload (the M = 1 decode layer), repeated for about
        `budget_s`, in TB/s of algorithmic bytes like the GPU figure;
      * per_config: for each of the five configurations, oracle.quantize + pack over
        that config's row sample (MB of fp16 weights per s), and for each of its M,
        oracle.gemm over the same sample (TB/s of algorithmic bytes, and TFLOP/s),
        each repeated for about `item_s`;
      * gemv_1024_one_thread_ms: oracle.gemm on config 1 with one BLAS thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))

    def sample(c, M_):
        n_rows = CPU_SAMPLE_ROWS[c.name]
        parts = []
        for mi, mat in enumerate(c.matrices):
            n = min(n_rows, mat.N)
            Wr = workloads.weight_rows(c.weight_key, mi, mat.N, mat.K, 0, n)
            sv = workloads.awq_scales(c.weight_key, mi, mat.K) if c.awq else None
            parts.append((mi, mat, n, Wr, sv))
        return parts

    def time_gemm(c, M_, parts, quants, budget):
        xs = [workloads.activations(c.weight_key, mi, M_, mat.K, outliers=c.act_outliers)
              for mi, mat, n, Wr, sv in parts]
        byts = flops = reps = 0
        t0 = time.perf_counter()
        while True:
            for X, (mi, mat, n, Wr, sv), ref in zip(xs, parts, quants):
                oracle.gemm(X, ref.q, ref.scales, ref.zeros, sv)
                byts += alg_bytes(M_, n, mat.K, sv is not None)
                flops += 2 * M_ * n * mat.K
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                return byts / dt, flops / dt, reps, dt

    with threadpool_limits(limits=cores, user_api="blas"):
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] + [1])
        parts = sample(cfg, M)
        quants = [oracle.quantize(Wr, sv) for mi, mat, n, Wr, sv in parts]
        bps, fps, reps, dt = time_gemm(cfg, M, parts, quants, budget_s)
        out = {"value": float(f"{bps / 1e12:.6g}"), "unit": "TB/s", "cores": cores,
               "blas_threads": blas_threads, "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"first {CPU_SAMPLE_ROWS[cfg.name]} rows of each of the "
                         f"{len(cfg.matrices)} matrices of {cfg.name} at M={M}: oracle.gemm "
                         f"(fp64 dequantize + matmul) repeated {reps}x"}
        per = []
        for c in workloads.CONFIGS:
            parts = sample(c, c.Ms[0])
            t0, wbytes, qreps = time.perf_counter(), 0, 0
            while True:
                quants = []
                for mi, mat, n, Wr, sv in parts:
                    ref = oracle.quantize(Wr, sv)
                    oracle.pack_codes(ref.q)
                    oracle.pack_meta(ref.scales)
                    oracle.pack_meta(ref.zeros)
                    quants.append(ref)
                    wbytes += 2 * n * mat.K
                qreps += 1
                if time.perf_counter() - t0 >= item_s:
                    break
            qdt = time.perf_counter() - t0
            entry = {"config": c.name, "sample_rows": CPU_SAMPLE_ROWS[c.name],
                     "quantize_pack": {"MB_of_fp16_weights_per_s": round(wbytes / qdt / 1e6, 3),
                                       "reps": qreps},
                     "gemm": []}
            for M_ in c.Ms:
                bps, fps, reps, dt = time_gemm(c, M_, parts, quants, item_s)
                entry["gemm"].append({"M": M_, "TB/s": float(f"{bps / 1e12:.4g}"),
                                      "TFLOP/s": float(f"{fps / 1e12:.4g}"), "reps": reps})
            per.append(entry)
        out["per_config"] = per
    # config 1 once more with one BLAS thread (the oracle's quantize and pack are
    # single-threaded NumPy anyway)
    g1 = workloads.config_by_name("gemv_1024")
    W1 = workloads.weights(g1.weight_key, 0, 1024, 1024)
    X1 = workloads.activations(g1.weight_key, 0, 1, 1024)
    r1 = oracle.quantize(W1, None)
    with threadpool_limits(limits=1, user_api="blas"):
        t0, n1 = time.perf_counter(), 0
        while time.perf_counter() - t0 < item_s:
            oracle.gemm(X1, r1.q, r1.scales, r1.zeros, None)
            n1 += 1
        out["gemv_1024_one_thread_ms"] = round((time.perf_counter() - t0) / n1 * 1e3, 3)
    out["per_config_note"] = (
        f"each config: its matrices' first sample_rows rows; quantize_pack = oracle.quantize "
        f"+ pack_codes + pack_meta (scales, zeros); gemm = oracle.gemm at each M, about "
        f"{item_s:g} s each")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=4000,
                    help="untimed steps before the timed ones (4000 decode steps: about 0.1 s, "
                         "enough for the clocks to settle)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--no-spec", action="store_true")
    ap.add_argument("--no-outliers", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-gptq", action="store_true")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", nargs="?", const="layer", choices=["layer", "verify", "batched"],
                    help="only a short fixed sequence for counter collection: 'layer' (the "
                         "default: a calibration copy, 20 decode steps, the 70B prefill "
                         "matrices), 'verify' (8B layer at M=2, 5, 9 and Qwen2-7B layer at "
                         "M=16: the streaming kernel's whole-row, 16-wave, hybrid and windowed "
                         "launches) or 'batched' (Qwen2-7B layer at M=64, 256)")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="only the M-dispatch crossover sweep (tiled vs 16-row streaming "
                         "pieces, M = 17..256 on the 8B, Qwen2-7B and 70B layers), as one "
                         "JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_int4_group_amd as w4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w4.lib()  # fail loudly if the HIP library is missing
    if args.profile_run == "verify":
        profile_run_batches(torch, w4, workloads, "llama3_8b_verify", (2, 5, 9))
        profile_run_batches(torch, w4, workloads, "qwen2_7b_batched_decode", (16,))
        return
    if args.profile_run == "batched":
        profile_run_batches(torch, w4, workloads, "qwen2_7b_batched_decode", (64, 256))
        return
    if args.profile_run:
        profile_run(torch, w4, workloads)
        return
    if args.dispatch_sweep:
        print(json.dumps({"dispatch_sweep": dispatch_sweep(torch, w4, workloads)}), flush=True)
        return
    cfg = workloads.config_by_name("llama3_8b_decode")
    M = cfg.Ms[0]
    log(f"preparing {cfg.name} M={M}")
    mats, pool, layer_w, copies = prepare_layer(cfg, M, torch, w4, workloads)
    step_bytes = sum(m["bytes"] for m in mats)
    names = [m["name"] for m in mats]
    one = [list(range(len(mats)))]
    log(f"{copies} layer copies, {layer_w * copies / 2**30:.2f} GiB of packed weights; "
        f"timing {args.steps} steps")
    wall, lms = timed(make_calls(mats, pool, copies, one, w4, torch), args.steps, args.warmup,
                      torch, min_warm_s=0)
    ms_per_step = wall / args.steps * 1e3
    avg_ms = float(np.mean(lms[0]))
    achieved = step_bytes / (avg_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(step_bytes / (ms_per_step * 1e-3) / 1e12, 4),
        "unit": "TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "llama3_8b_decode_layer: the 7 matrices of a Llama-3-8B-shaped "
                               "decoder layer, M=1, group 128, AWQ s, asym uint4 + fp16 "
                               "scale/zero, one grouped launch per step",
                   "M": M, "step_bytes": step_bytes, "weight_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "skinny_kernel (grouped, 7 problems)",
                     "avg_launch_us": round(avg_ms * 1e3, 3), "per_launch_bytes": step_bytes,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic("skinny_decode_llama3_8b_layer_m1_counters.txt",
                                                 "skinny.hip"),
                     # spread of the per-launch durations (blocks of 10 launches)
                     "launch_us_p10_median_p90": [round(float(np.percentile(lms[0], q)) * 1e3, 3)
                                                  for q in (10, 50, 90)]},
    }
    if not args.no_ceilings:
        # the plain streaming-read ceiling on the same bytes, same rotation
        log("measuring the streaming-read ceiling")
        rc_ = read_ceiling(torch, step_bytes)
        out["roofline"]["read_ceiling"] = rc_
        out["roofline"]["frac_of_read_ceiling"] = round(
            achieved / rc_["best"]["GB/s"], 4)
    if not args.no_variants:
        # the same launches over one buffer copy: the 116 MB layer then largely
        # stays in the 256 MB last-level cache, so this is not an HBM figure
        wwall, wl = timed(make_calls(mats, [[p[0]] for p in pool], 1, one, w4, torch), 200, 20,
                          torch)
        wms = float(np.mean(wl[0]))
        out["warm_same_buffer"] = {"workload": f"{cfg.name}, one weight copy reused every step",
                                   "kernel_us_per_step": round(wms * 1e3, 2),
                                   "kernel_TB/s": round(step_bytes / (wms * 1e-3) / 1e12, 4)}
        out["gemv_1024"] = gemv_line(torch, w4, workloads)
        idx = {n: i for i, n in enumerate(names)}
        dep = [[idx["q"], idx["k"], idx["v"]], [idx["o"]], [idx["gate"], idx["up"]], [idx["down"]]]
        sep = [[j] for j in range(len(mats))]
        vs = {}
        for label, groups in (("dependency_order_4_launches", dep), ("separate_7_launches", sep)):
            w, l = timed(make_calls(mats, pool, copies, groups, w4, torch), 200, 20, torch)
            vs[label] = variant(mats, groups, l, 200, w, "bytes")
        out["layer_variants"] = vs
    if not args.no_bf16:
        bmats = with_bf16(mats, cfg, M, torch, workloads)
        bwall, blms = timed(make_calls(bmats, pool, copies, one, w4, torch), args.steps // 2,
                            args.warmup, torch)
        bkern = float(np.mean(blms[0])) * 1e-3
        out["bf16"] = {"workload": f"{cfg.name} with bf16 activations and outputs, M={M}, "
                                   "the same packed weights, one grouped launch per step",
                       "us_per_step": round(bwall / (args.steps // 2) * 1e6, 2),
                       "kernel_us_per_step": round(bkern * 1e6, 2),
                       "kernel_TB/s": round(step_bytes / bkern / 1e12, 4),
                       "vs_fp16_kernel_time": round(bkern / (avg_ms * 1e-3), 4)}
        del bmats
    if not args.no_batched:
        vcfg = workloads.config_by_name("llama3_8b_verify")
        assert vcfg.weight_key == cfg.weight_key  # verify runs the decode layer's weights
        lines = [batched_line(vcfg, vm, mats, pool, copies, w4, torch, workloads)
                 for vm in vcfg.Ms]
        del pool, mats
        torch.cuda.empty_cache()
        qcfg = workloads.config_by_name("qwen2_7b_batched_decode")
        log(f"preparing {qcfg.name}")
        qmats, qpool, _, qc = prepare_layer(qcfg, qcfg.Ms[0], torch, w4, workloads)
        lines += [batched_line(qcfg, qm, qmats, qpool, qc, w4, torch, workloads)
                  for qm in qcfg.Ms]
        out["batched"] = lines
        del qpool, qmats
    else:
        del pool, mats
    torch.cuda.empty_cache()

    if not args.no_outliers:
        log(f"preparing {cfg.name} with fp16 outliers")
        omats, opool, ow, oc = prepare_layer(cfg, M, torch, w4, workloads, outliers=True)
        ob = sum(m["bytes"] for m in omats)
        owall, olms = timed(make_calls(omats, opool, oc, one, w4, torch), args.steps // 2,
                            args.warmup, torch)
        okern = float(np.mean(olms[0])) * 1e-3
        out["outliers"] = {
            "workload": f"{cfg.name} with fp16 outliers: the same 7 matrices, M={M}, each with "
                        "its top 0.1% |W/s| kept in fp16 (row-compressed) and added in the "
                        "epilogue, one grouped launch per step",
            "kept": int(sum(m["pw"].o_col.numel() for m in omats)),
            "step_bytes": ob, "outlier_bytes": int(sum(outlier_bytes(m["pw"]) for m in omats)),
            "us_per_step": round(owall / (args.steps // 2) * 1e6, 2),
            "kernel_us_per_step": round(okern * 1e6, 2),
            "kernel_TB/s": round(ob / okern / 1e12, 4),
            "vs_plain_kernel_time": round(okern / (avg_ms * 1e-3), 4)}
        del opool, omats
        torch.cuda.empty_cache()

    if not args.no_int8:
        log(f"preparing {cfg.name} with INT8 codes")
        imats, ipool, _, ic = prepare_layer(cfg, M, torch, w4, workloads, int8=True)
        ib = sum(m["bytes"] for m in imats)
        iwall, ilms = timed(make_calls(imats, ipool, ic, one, w4, torch), args.steps // 2,
                            args.warmup, torch)
        ikern = float(np.mean(ilms[0])) * 1e-3
        out["int8"] = {
            "workload": f"{cfg.name} with INT8 codes (W8A16): the same 7 matrices, M={M}, "
                        "group 128, asym uint8 + fp16 scale/zero, one grouped launch per step",
            "step_bytes": ib, "us_per_step": round(iwall / (args.steps // 2) * 1e6, 2),
            "kernel_us_per_step": round(ikern * 1e6, 2),
            "kernel_TB/s": round(ib / ikern / 1e12, 4),
            "frac_of_hbm_peak": round(ib / ikern / 1e9 / HBM_PEAK_GBS, 4),
            "vs_int4_kernel_time": round(ikern / (avg_ms * 1e-3), 4)}
        if not args.no_bf16:
            ibm = with_bf16(imats, cfg, M, torch, workloads)
            _, iblms = timed(make_calls(ibm, ipool, ic, one, w4, torch), args.steps // 2,
                             args.warmup, torch)
            ibkern = float(np.mean(iblms[0])) * 1e-3
            out["int8"]["bf16"] = {"workload": "the same INT8 layer with bf16 activations and outputs",
                                   "kernel_us_per_step": round(ibkern * 1e6, 2),
                                   "kernel_TB/s": round(ib / ibkern / 1e12, 4),
                                   "vs_fp16_kernel_time": round(ibkern / ikern, 4)}
            del ibm
        del ipool, imats
        torch.cuda.empty_cache()

    if not args.no_spec:
        log("timing speculative verification")
        out["spec_verify"] = [spec_verify_line(torch, w4, B, 4, 128256) for B in (1, 64)]
        torch.cuda.empty_cache()

    if not args.no_prefill:
        pcfg = workloads.config_by_name("llama_70b_prefill")
        PM = pcfg.Ms[0]
        log(f"preparing {pcfg.name} M={PM}")
        pmats, ppool, _, pc = prepare_layer(pcfg, PM, torch, w4, workloads, copies_min_bytes=0)
        groups = [[j] for j in range(len(pmats))]
        pcalls = make_calls(pmats, ppool, pc, groups, w4, torch)
        pwall, pms = timed(pcalls, args.prefill_steps, 2, torch, per=1)
        flops = sum(m["flops"] for m in pmats)
        tot_ms = sum(float(np.mean(x)) for x in pms)
        # The GEMM kernel alone: the same calls on X * s computed beforehand (the same fp16
        # rounding as the library's prescale) with s = NULL launch exactly the same GEMM
        # kernel, without the prescale pass; their outputs must be bit-identical.
        gmats = [dict(m, X=(m["X"] * m["s"]).contiguous() if m["s"] is not None else m["X"],
                      s=None) for m in pmats]
        gcalls = make_calls(gmats, ppool, pc, groups, w4, torch)
        same = True
        for a, b, m in zip(pcalls[0], gcalls[0], pmats):
            a()
            ya = m["Y"].clone()
            b()
            same &= bool(torch.equal(ya.view(torch.int16), m["Y"].view(torch.int16)))
        _, gms = timed(gcalls, args.prefill_steps, 2, torch, per=1)
        g_ms = sum(float(np.mean(x)) for x in gms)
        del gmats, gcalls
        out["prefill"] = {
            "workload": f"{pcfg.name}: the 7 matrices of a 70B-shaped layer, M={PM}, AWQ s, "
                        "1% activation channels x20, one launch per matrix",
            "TFLOP/s": round(flops / (pwall / args.prefill_steps) / 1e12, 2),
            "ms_per_step": round(pwall / args.prefill_steps * 1e3, 4),
            "roofline": {"bound": "mfma",
                         "kernel": "tiled_dma_kernel<8, 4, 1, false, false>, one launch per matrix (k and v: plus "
                                   "split_reduce_kernel); timed on calls whose X * s was formed "
                                   "beforehand, which launch exactly this kernel",
                         "outputs_identical_to_calls_with_s": same,
                         "avg_launch_us": round(g_ms / len(pmats) * 1e3, 2),
                         "achieved": round(flops / (g_ms * 1e-3) / 1e12, 2),
                         "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (g_ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                         "traffic": profiled_traffic("tiled_dma_prefill_70b_layer_m4096_counters.txt",
                                                     "tiled.hip"),
                         "with_prescale": {
                             "what": "the whole call with s: prescale_f16_kernel (X * s into the "
                                     "workspace) + the GEMM",
                             "avg_call_us": round(tot_ms / len(pmats) * 1e3, 2),
                             "TFLOP/s": round(flops / (tot_ms * 1e-3) / 1e12, 2),
                             "frac": round(flops / (tot_ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4)}},
            "per_matrix": variant(pmats, groups, pms, args.prefill_steps, pwall, "flops")["launches"],
        }
        if not args.no_ceilings:
            # the matrix cores' own sustained rate on this GPU, for context
            log("measuring the MFMA-only ceiling")
            mc = mfma_ceiling(torch)
            out["prefill"]["roofline"]["mfma_ceiling"] = mc
            out["prefill"]["roofline"]["frac_of_mfma_ceiling"] = round(
                out["prefill"]["roofline"]["achieved"] / mc["TFLOP/s"], 4)
        if not args.no_bf16:
            bpm = with_bf16(pmats, pcfg, PM, torch, workloads)
            _, bpms = timed(make_calls(bpm, ppool, pc, groups, w4, torch), args.prefill_steps, 2,
                            torch, per=1)
            btot = sum(float(np.mean(x)) for x in bpms)
            out["prefill"]["bf16"] = {
                "workload": "the same layer with bf16 activations and outputs",
                "kernel_ms_per_step": round(btot, 4),
                "TFLOP/s": round(flops / (btot * 1e-3) / 1e12, 2),
                "frac_of_dense_bf16_peak": round(flops / (btot * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                "vs_fp16_kernel_time": round(btot / tot_ms, 4)}
            del bpm
        del ppool, pmats
        torch.cuda.empty_cache()
        if not args.no_int8:
            log(f"preparing {pcfg.name} M={PM} with INT8 codes")
            imats, ipool, _, ipc = prepare_layer(pcfg, PM, torch, w4, workloads,
                                                 copies_min_bytes=0, int8=True)
            _, ims = timed(make_calls(imats, ipool, ipc, groups, w4, torch), args.prefill_steps,
                           2, torch, per=1)
            itot = sum(float(np.mean(x)) for x in ims)
            out["prefill"]["int8"] = {
                "workload": "the same layer with INT8 codes (W8A16)",
                "kernel_ms_per_step": round(itot, 4),
                "TFLOP/s": round(flops / (itot * 1e-3) / 1e12, 2),
                "frac_of_dense_fp16_peak": round(flops / (itot * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                "vs_int4_kernel_time": round(itot / tot_ms, 4)}
            del ipool, imats
            torch.cuda.empty_cache()
        if not args.no_outliers:
            log(f"preparing {pcfg.name} M={PM} with fp16 outliers")
            omats, opool, _, opc = prepare_layer(pcfg, PM, torch, w4, workloads,
                                                 copies_min_bytes=0, outliers=True)
            _, oms = timed(make_calls(omats, opool, opc, groups, w4, torch), args.prefill_steps, 2,
                           torch, per=1)
            otot = sum(float(np.mean(x)) for x in oms)
            out["prefill"]["outliers"] = {
                "workload": "the same layer with each matrix's top 0.1% |W/s| kept in fp16",
                "kernel_ms_per_step": round(otot, 4),
                "TFLOP/s": round(flops / (otot * 1e-3) / 1e12, 2),
                "vs_plain_kernel_time": round(otot / tot_ms, 4)}
            del opool, omats
            torch.cuda.empty_cache()

    if not args.no_gptq:
        log("timing the GPTQ packer")
        out["gptq"] = gptq_line(torch, w4)
        torch.cuda.empty_cache()

    if not args.no_ceilings:
        log("measuring the copy and dense fp16 GEMM ceilings")
        out["ceilings"] = ceilings(torch)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, M, workloads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
