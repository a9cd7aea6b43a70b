#!/usr/bin/env python3
"""Benchmark of the exact tiled attention forward (and, with --bwd, backward) on one MI355X.

One step = one full forward pass (work partition, Q/K/V tiles, scores, mask, online softmax, P*V,
epilogue; for the fp8 workload also the preparation launch for Q, K and V) over one batch of seeded
synthetic inputs already resident in HBM.  Default workload: fp16 B1 H8 N16384 d256 causal (the
largest one-GPU workload).
With --bwd a step is one backward pass (the dQ launch, which also forms D, then dK/dV) from the forward's saved o and
lse, counted as 10*B*H*N^2*d flops (/2 causal).  --decode times the decode path (K/V cache read
GB/s); --naive times the unfused path (scores, softmax, P*V through HBM) beside the fused kernel.

Prints ONE JSON line (rank 0):
  metric/value/unit         attention fwd TFLOP/s = 4*B*H*N^2*d (/2 causal) / time per step
  roofline                  dominant kernel: algorithmic flops per launch / its GPU time per launch
                            over the timed region (HIP events on the launch stream), against the
                            MI355X dense peak; "settled" adds the same launches after the timed
                            region once the clock has settled (context, not the value)
  cpu_baseline              the float64 CPU oracle timed on a bounded sample of the same workload
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")
# sources of the kernels each workload launches (a counter record is valid while these are unchanged)
KERNEL_SOURCES = {
    "bf16": ["fa_fwd.hip", "fa_common.h"], "f16": ["fa_fwd.hip", "fa_common.h"],
    "f32": ["fa_fwd_f32.hip", "fa_common.h"], "fp8": ["fa_fwd_fp8.hip", "fa_fp8_prep.hip", "fa_common.h"],
}


def kernel_source_hash(dtype: str = "bf16") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, "exact_tiled_attention_22_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(cfg_id: int, dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the sources."""
    path = os.path.join(PROFILES, f"traffic_cfg{cfg_id}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(dtype):
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20


def ingest_counters(cfg_id: int, fetch_csv: str, write_csv: str) -> int:
    """HBM bytes per attention launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by the same counter on a plain copy of COPY_BYTES (which reads and writes
    exactly COPY_BYTES)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        attn = [v for k, v in vals.items() if "fa_fwd" in k]
        copy = [v for k, v in vals.items() if "copyBuffer" in k]
        if not attn or not copy:
            raise SystemExit(f"{path}: need attention and copy dispatches, found {list(vals)}")
        attn_kib = sum(attn[0]) / len(attn[0])
        copy_kib = sum(copy[0]) / len(copy[0])
        factor = (COPY_BYTES / 1024.0) / copy_kib
        out[counter] = {"attention_kib_per_dispatch": attn_kib, "copy_kib_per_dispatch": copy_kib,
                        "copy_scale_factor": factor, "bytes_per_launch": attn_kib * 1024.0 * factor}
    from synth import WORKLOADS

    rec = {"config": cfg_id, "kernel_source_sha256_16": kernel_source_hash(WORKLOADS[cfg_id].dtype),
           "counters": out,
           "hbm_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"traffic_cfg{cfg_id}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def time_steps(step, steps: int, dev) -> float:
    """Wall-clock ms per step over exactly `steps` back-to-back steps, synchronised on both sides (the
    launches are enqueued without anything between them, as a caller would issue them)."""
    return timed_region(step, steps, dev)[0]


def timed_region(step, steps: int, dev, inner=None):
    """The timed region: exactly `steps` back-to-back steps, synchronised on both sides.  Returns
    (wall-clock ms per step, GPU ms per step).  The GPU time comes from HIP events recorded on the launch
    stream (torch's current stream, on which the binding launches) right before the first and right after
    the last step, so it covers the same launches as the wall clock and cannot exceed it.  With `inner`
    (a pair of callables (pre, kernel) making up one step), an event pair brackets each kernel() call
    inside the region instead, and the GPU time is the average of those pairs: the dominant kernel's own
    launch duration when a step holds several launches."""
    import torch

    stream = torch.cuda.current_stream(dev)
    if inner is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            step()
        b.record(stream)
        torch.cuda.synchronize(dev)
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return wall, a.elapsed_time(b) / steps
    pre, kernel = inner
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for a, b in ev:
        pre()
        a.record(stream)
        kernel()
        b.record(stream)
    torch.cuda.synchronize(dev)
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, sum(a.elapsed_time(b) for a, b in ev) / steps


def settled_stats(step, dev, min_ms: float = 300.0, min_steps: int = 20, pre=None) -> dict:
    """Per-step event durations after the timed region, once the clock has settled: steps run back to
    back for at least `min_ms` first, then event pairs around each of at least `min_steps` further steps
    (and at least `min_ms` of them).  Context beside the timed region, never the reported value."""
    import torch

    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            if pre is not None:
                pre()
            step()
        torch.cuda.synchronize(dev)
    t = []
    t0 = time.perf_counter()
    while len(t) < min_steps or (time.perf_counter() - t0) * 1e3 < min_ms:
        st = launch_stats(step, min_steps, dev, pre=pre)
        t.extend(st["all"])
    t.sort()
    return {"steps": len(t), "median_ms": round(t[len(t) // 2], 5), "min_ms": round(t[0], 5),
            "avg_ms": round(sum(t) / len(t), 5)}


def launch_stats(step, steps: int, dev, pre=None) -> dict:
    """Mean, median and minimum of the per-step event durations (ms) of a pass of `steps` steps.  With
    `pre`, each step is pre() then step(), and only step() is inside the event pair."""
    import torch

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    for a, b in ev:
        if pre is not None:
            pre()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize(dev)
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"avg": sum(t) / len(t), "median": t[len(t) // 2], "min": t[0], "all": t}


def cold_launch_ms(step, reps: int, dev, flush_bytes: int = 512 << 20, pre=None) -> float:
    """Median event-timed duration of a step issued right after a 512 MiB device write, which evicts the
    inputs from the caches (L2 and the memory-side cache)."""
    import torch

    stream = torch.cuda.current_stream(dev)
    junk = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    t = []
    for i in range(reps):
        if pre is not None:
            pre()
        junk.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize(dev)
        t.append(a.elapsed_time(b))
    del junk
    return sorted(t)[len(t) // 2]


def tensor_sha16(t) -> str:
    """First 16 hex digits of the SHA-256 of a host tensor's bytes (the generated inputs, before upload)."""
    import torch

    x = t.detach().contiguous().cpu()
    if x.dtype in (torch.bfloat16, torch.float16):
        x = x.view(torch.int16)
    return hashlib.sha256(x.numpy().tobytes()).hexdigest()[:16]


def cpu_baseline(w, seed: int, budget_s: float = 12.0, bwd: bool = False):
    """Time the float64 oracle on whole heads of the workload until ~budget_s of CPU work."""
    import numpy as np

    from oracle import attention_bwd_rows, attention_rows
    from synth import gen_qkv

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    # one head's worth of inputs (the generator draws whole tensors; take the first heads)
    q, k, v = gen_qkv(1, min(w.H, 4), w.N, w.d, "bf16" if w.dtype == "fp8" else w.dtype, seed)
    per_head = (10.0 if bwd else 4.0) * w.N * w.N * w.d / (2.0 if w.causal else 1.0)
    done_flops, heads, t0 = 0.0, 0, time.perf_counter()
    chunk = 1024
    while True:
        h = heads % q.shape[1]
        if bwd:
            attention_bwd_rows(q[0, h], k[0, h], v[0, h], q[0, (h + 1) % q.shape[1]], w.causal, w.scale)
        else:
            for r0 in range(0, w.N, chunk):
                rows = np.arange(r0, min(w.N, r0 + chunk))
                attention_rows(q[0, h], k[0, h], v[0, h], rows, w.causal, w.scale)
        heads += 1
        done_flops += per_head
        if time.perf_counter() - t0 >= budget_s or heads >= 512:
            break
    dt = time.perf_counter() - t0
    return {
        "value": done_flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} (b,h) heads of the workload ({'backward, ' if bwd else ''}float64 NumPy/OpenBLAS, "
                  f"full score rows), "
                  f"{dt:.1f} s",
    }


DECODE = {"B": 8, "H": 32, "Nq": 1, "Nk": 32768, "d": 128, "dtype": "bf16", "causal": False}


def bench_decode(args) -> int:
    """Decode leg: one query per (b, h) against a 32768-key bf16 cache.  HBM-bound: the metric is the
    K/V cache bytes read per second (2 * B * H * Nk * d * 2 bytes per step)."""
    import torch

    import exact_tiled_attention_22_amd as fa
    from synth import gen_qkv

    c = dict(DECODE, Nq=args.nq)
    if not 1 <= c["Nq"] <= 32:
        print(f"--nq must be 1..32 (the decode path takes at most 32 queries), got {c['Nq']}", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qf, k, v = (t.to(dev) for t in gen_qkv(c["B"], c["H"], c["Nk"], c["d"], c["dtype"], 7))
    q = qf[:, :, c["Nk"] - c["Nq"]:, :].contiguous()
    del qf
    scale = 1.0 / math.sqrt(c["d"])
    o = torch.empty_like(q)
    lse = torch.empty((c["B"], c["H"], c["Nq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(c["B"], c["H"], c["Nq"], c["Nk"], c["d"]), dtype=torch.uint8, device=dev)

    def step():
        return fa.fwd_decode(q, k, v, causal=c["causal"], scale=scale, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    ms_per_step, avg_ms = timed_region(step, args.steps, dev)
    nbytes = 2.0 * c["B"] * c["H"] * c["Nk"] * c["d"] * 2
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    line = {
        "metric": "decode attention K/V cache read GB/s (2*B*H*Nk*d*2 bytes per step)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": f"bf16 decode B8 H32 Nq{c['Nq']} Nk32768 d128 non-causal", **c, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": ("decode_vec_kernel" if c["Nq"] == 1 else "decode_split_kernel")
                     + " + decode_merge_kernel (the launches of one fa_fwd_decode call)",
                     "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": None, "kernel_avg_ms": round(avg_ms, 5),
                     "timing": "HIP events on the launch stream over the timed region (first to last launch, / steps)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = decode_cpu_baseline(c)
    print(json.dumps(line), flush=True)
    return 0


def bench_shard(args, w) -> int:
    """One GPU's share of a sequence-sharded causal forward: with the query rows cut into G equal ranges
    (rank r owns rows [r*N/G, (r+1)*N/G)) and K/V gathered on every GPU, rank r attends its rows to the
    keys they can see, [0, (r+1)*N/G).  A share has only B*H*N/(G*BM) query tiles, too few workgroups
    to fill the GPU, so it runs through fa_fwd_split with each query tile's keys cut into enough shares
    to fill every workgroup slot (fa_fwd_rect, unsplit, is timed beside it).  Every rank's share is
    timed on this one GPU (HIP events, median); the line reports the heaviest share (the last rank),
    which sets the step time of the sharded forward.  Flops per share follow the metric's convention:
    4*B*H*d*(Nq*q_start + Nq^2/2), which sums over the ranks to the workload's 4*B*H*N^2*d/2."""
    import torch

    import exact_tiled_attention_22_amd as fa
    from synth import gen_qkv

    G = args.shard
    if not w.causal or w.dtype not in ("bf16", "f16") or G < 2 or w.N % G:
        print(f"--shard needs a causal 16-bit workload whose N divides by G (workload {w.cfg_id}, G {G})",
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    q, k, v = (t.to(dev) for t in gen_qkv(w.B, w.H, w.N, w.d, w.dtype, w.cfg_id))
    nq = w.N // G
    # workgroups of the forward kernel: 128 query rows, two per CU (d <= 128); 256 rows, one per CU (d = 256)
    bm, per_cu = (256, 1) if w.d >= 256 else (128, 2)
    base_wg = w.B * w.H * ((nq + bm - 1) // bm)
    nsplit = max(1, min(64, -(-per_cu * cus // base_wg)))
    ws = torch.empty(fa.split_workspace_bytes(w.B, w.H, nq, w.d, nsplit), dtype=torch.uint8, device=dev)
    shares = []
    for r in range(G):
        q0, nk = r * nq, (r + 1) * nq
        qr = q[:, :, q0:q0 + nq].contiguous()
        kr, vr = k[:, :, :nk].contiguous(), v[:, :, :nk].contiguous()
        o = torch.empty_like(qr)
        lse = torch.empty((w.B, w.H, nq), dtype=torch.float32, device=dev)

        def split_step(qr=qr, kr=kr, vr=vr, o=o, lse=lse, q0=q0):
            return fa.fwd_split(qr, kr, vr, nsplit=nsplit, causal=True, q_start=q0, scale=w.scale, out=o, lse=lse,
                                workspace=ws)

        def rect_step(qr=qr, kr=kr, vr=vr, o=o, lse=lse, q0=q0):
            return fa.fwd_rect(qr, kr, vr, causal=True, q_start=q0, scale=w.scale, out=o, lse=lse)

        flops = 4.0 * w.B * w.H * w.d * (nq * q0 + nq * nq / 2.0)
        row = {"rank": r, "q_rows": [q0, q0 + nq], "keys": nk}
        for name, step in (("split", split_step), ("rect", rect_step)):
            for _ in range(args.warmup):
                step()
            st = launch_stats(step, args.steps, dev)
            row[f"{name}_median_ms"] = round(st["median"], 5)
            row[f"{name}_tflops"] = round(flops / (st["median"] * 1e-3) / 1e12, 2)
        shares.append(row)
        del qr, kr, vr, o, lse
    top = shares[-1]
    line = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, /2 causal; one GPU's share of a sequence split)",
        "value": top["split_tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": top["split_median_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": f"{w.name}: query rows {top['q_rows'][0]}..{top['q_rows'][1] - 1} of a {G}-way "
                               f"sequence split against keys 0..{top['keys'] - 1} (one GPU's share, fa_fwd_split "
                               f"with {nsplit} key shares per query tile)",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True, "shards": G, "key_shares": nsplit,
                   "parallelism": "single GPU", "shares": shares},
        "roofline": {"bound": "mfma", "kernel": "fa_fwd16_kernel (key shares) + decode_merge_kernel",
                     "achieved": top["split_tflops"], "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                     "frac": round(top["split_tflops"] / PEAK_TFLOPS[w.dtype], 4), "traffic": None,
                     "kernel_median_ms": top["split_median_ms"]},
    }
    print(json.dumps(line), flush=True)
    return 0


def decode_cpu_baseline(c, budget_s: float = 10.0):
    """The float64 oracle (attention_rect: full score rows) on whole (b, h) heads of the decode workload
    until ~budget_s, in the same unit: K/V cache bytes (2 * Nk * d * 2 per head) per second."""
    import numpy as np  # noqa: F401

    from oracle import attention_rect
    from synth import gen_qkv

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    qf, k, v = gen_qkv(1, 4, c["Nk"], c["d"], c["dtype"], 7)
    q = qf[:, :, c["Nk"] - c["Nq"]:, :]
    scale = 1.0 / math.sqrt(c["d"])
    heads, t0 = 0, time.perf_counter()
    while True:
        h = heads % 4
        attention_rect(q[0, h], k[0, h], v[0, h], c["causal"], scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s or heads >= 4096:
            break
    dt = time.perf_counter() - t0
    return {"value": heads * 2.0 * c["Nk"] * c["d"] * 2 / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} (b,h) heads of the workload (float64 NumPy/OpenBLAS, full score rows), {dt:.1f} s"}


def bench_naive(args, w) -> int:
    """Unfused comparison leg: S = scale Q K^T (float32) -> softmax -> P V, each step three launches with
    the N x N matrices in HBM, each launch timed with HIP events; the fused kernel is timed beside it on
    the same inputs.  Every stage is HBM-bound: the roofline is the slowest stage's algorithmic bytes
    per second against 8 TB/s."""
    import torch

    import exact_tiled_attention_22_amd as fa
    from synth import gen_qkv

    if w.dtype not in ("bf16", "f16"):
        print(f"the unfused path covers bf16/fp16, not workload {w.cfg_id}", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (t.to(dev) for t in gen_qkv(w.B, w.H, w.N, w.d, w.dtype, w.cfg_id))
    ld = fa.naive_row_stride(w.N)
    s = torch.empty((w.B, w.H, w.N, ld), dtype=torch.float32, device=dev)
    p = torch.empty((w.B, w.H, w.N, ld), dtype=q.dtype, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    n = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]

    def step(e=None):
        if e: e[0].record(stream)
        fa.naive_scores(q, k, scale=w.scale, s=s)
        if e: e[1].record(stream)
        fa.naive_softmax(s, dtype=q.dtype, causal=w.causal, p=p, lse=lse)
        if e: e[2].record(stream)
        fa.naive_pv(p, v, out=o)
        if e: e[3].record(stream)

    for _ in range(args.warmup):
        step()
    # timed region: exactly K back-to-back steps; then each stage from event pairs in a pass of its own
    ms_per_step = time_steps(step, n, dev)
    torch.cuda.synchronize(dev)
    for i in range(n):
        step(ev[i])
    torch.cuda.synchronize(dev)
    stage_ms = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)) / n for j in range(3)]

    # the fused kernel on the same inputs, same protocol
    o2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)

    def fused():
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o2, lse=lse2)

    for _ in range(args.warmup):
        fused()
    fused_ms = time_steps(fused, n, dev)

    e = 2
    BH, N, d = w.B * w.H, w.N, w.d
    visible = N * (N + 1) / 2 if w.causal else float(N) * N
    stage_bytes = [BH * (2 * N * d * e + 4.0 * N * N),            # read Q, K; write S
                   BH * (4.0 * visible + e * N * ld),              # read the visible S; write P (with padding)
                   BH * (e * N * ld + 2 * e * N * d)]              # read P, V; write O
    names = ["naive_scores_kernel", "naive_softmax_kernel", "naive_pv_kernel"]
    stages = {nm: {"avg_ms": round(t, 5), "GB/s": round(b / (t * 1e-3) / 1e9, 1), "bytes": b}
              for nm, t, b in zip(names, stage_ms, stage_bytes)}
    dom = max(range(3), key=lambda j: stage_ms[j])
    achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    line = {
        "metric": "unfused attention fwd TFLOP/s (4*B*H*N^2*d, /2 causal; S and P through HBM)",
        "value": round(w.flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": n, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": w.name.replace(" fwd", " unfused fwd"), "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": round(achieved, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(achieved / 8000.0, 4), "traffic": None,
                     "kernel_avg_ms": round(stage_ms[dom], 5)},
        "stages": stages,
        "fused": {"ms_per_step": round(fused_ms, 5), "value": round(w.flops / (fused_ms * 1e-3) / 1e12, 2),
                  "speedup_over_unfused": round(ms_per_step / fused_ms, 2)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, w.cfg_id)
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # the GPU needs ~40 ms of sustained load to reach its working clock: warm up well past that
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=4,
                    help="workload id 1..5 (default 4: fp16 B1 H8 N16384 d256 causal, the largest one-GPU workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode path (1 query against a 32768-key cache, B8 H32 d128 bf16)")
    ap.add_argument("--nq", type=int, default=1,
                    help="queries per (b, h) for --decode (1: vector-ALU kernel; 2..32: matrix kernel)")
    ap.add_argument("--naive", action="store_true",
                    help="time the unfused path (S and P through HBM) and the fused kernel beside it")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (dQ, dK, dV from the saved lse) instead of the forward")
    ap.add_argument("--shard", type=int, default=0, metavar="G",
                    help="time one GPU's share of a G-way sequence-sharded causal forward (--config 3: bf16 B2 H16 N8192 d128, or --config 4: fp16 B1 H8 N16384 d256)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) "
                         "into profiles/traffic_cfg<N>.json and exit")
    args = ap.parse_args()
    if args.ingest_counters:
        return ingest_counters(args.config, *args.ingest_counters)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the (b,h) slices would "
              "shard across GPUs with no communication, but this library measures a single GPU.",
              file=sys.stderr)
        return 2

    import torch

    import exact_tiled_attention_22_amd as fa
    from synth import WORKLOADS, gen_fp8_workload, gen_qkv

    if args.decode:
        return bench_decode(args)
    w = WORKLOADS[args.config]
    if args.naive:
        return bench_naive(args, w)
    if args.shard:
        return bench_shard(args, w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = w.cfg_id
    if args.bwd:
        if w.dtype not in ("bf16", "f16"):
            print(f"the backward pass covers bf16/fp16, not workload {w.cfg_id}", file=sys.stderr)
            return 2
        host = gen_qkv(w.B, w.H, w.N, w.d, w.dtype, seed)
        hashes = {n: tensor_sha16(t) for n, t in zip("qkv", host)}
        q, k, v = (t.to(dev) for t in host)
        dh = gen_qkv(w.B, w.H, w.N, w.d, w.dtype, seed + 1000)[0]
        hashes["dout"] = tensor_sha16(dh)
        do = dh.to(dev)
        o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            return fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, delta=delta)
    elif w.dtype == "fp8":
        qs, ks, vs, signs = gen_fp8_workload(w, seed)
        hashes = {n: tensor_sha16(t) for n, t in zip("qkv", (qs, ks, vs))}
        qs, ks, vs = qs.to(dev), ks.to(dev), vs.to(dev)

        prepped = {}

        def prep():
            # one launch quantises Q, K (rotated with the shared signs) and V
            prepped["q"], prepped["k"], prepped["v"] = fa.fp8_prep_qkv(qs, ks, vs, signs, w.fp8_block)

        def fwd8():
            (q8, sq), (k8, sk), (v8, sv) = prepped["q"], prepped["k"], prepped["v"]
            return fa.fwd(q8, k8, v8, causal=w.causal, scale=w.scale, fp8_scales=(sq, sk, sv), block=w.fp8_block)

        def step():
            prep()
            return fwd8()
    else:
        host = gen_qkv(w.B, w.H, w.N, w.d, w.dtype, seed)
        hashes = {n: tensor_sha16(t) for n, t in zip("qkv", host)}
        q, k, v = (t.to(dev) for t in host)
        del host
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            return fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    # timed region: exactly K back-to-back steps, wall clock and HIP events on the launch stream.  The
    # e4m3 step holds the preparation launch and the forward kernel: event pairs bracket each
    # forward launch inside the region, so the roofline covers that kernel alone.
    fp8_fwd = w.dtype == "fp8" and not args.bwd
    ms_per_step, avg_launch_ms = timed_region(step, args.steps, dev, inner=(prep, fwd8) if fp8_fwd else None)
    # context, after the timed region: the same launches once the clock has settled, and cold caches
    if fp8_fwd:
        settled = settled_stats(fwd8, dev, pre=prep)
        cold_ms = cold_launch_ms(fwd8, 20, dev, pre=prep)
    else:
        settled = settled_stats(step, dev)
        cold_ms = cold_launch_ms(step, 20, dev)

    flops = w.flops * (2.5 if args.bwd else 1.0)  # backward: dS, dQ, dK, dV and the recomputed S = 10 N^2 d
    kernel = ("fa_bwd (dQ and dK/dV launches of one call)" if args.bwd else
              "fa_fwd8_kernel (the preparation launch excluded)" if w.dtype == "fp8" else
              "fa_fwd32_kernel" if w.dtype == "f32" else "fa_fwd16_kernel")
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = None if args.bwd else load_traffic(w.cfg_id, w.dtype)
    line = {
        "metric": ("attention bwd TFLOP/s (10*B*H*N^2*d, /2 causal) and % of MI355X MFMA peak" if args.bwd else
                   "attention fwd TFLOP/s (4*B*H*N^2*d, /2 causal) and % of MI355X MFMA peak"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "f32": "f32", "fp8": "fp8_e4m3"}[w.dtype],
        "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": w.name.replace(" fwd", " bwd") if args.bwd else w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "parallelism": "single GPU", "inputs_sha256_16": hashes},
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            # GPU time per launch over the timed region (HIP events on the launch stream)
            "kernel_avg_ms": round(avg_launch_ms, 5),
            "timing": "HIP events on the launch stream over the timed region" + (
                " (one pair around each forward launch)" if fp8_fwd else " (first to last launch, / steps)"),
            # context only: after the timed region, with the clock settled; and with cold caches
            "settled": dict(settled, tflops=round(flops / (settled["median_ms"] * 1e-3) / 1e12, 2),
                            frac=round(flops / (settled["median_ms"] * 1e-3) / 1e12 / peak, 4)),
            "cold_kernel_ms": round(cold_ms, 5),
        },
    }
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, seed, bwd=args.bwd)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
