#!/usr/bin/env python3
"""Benchmark of the pi-Attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_8k]

A step is one piattn_fwd call over the whole workload (every query row of
every (sequence, head)): window and skip enumeration, QK^T, gate prior,
single online softmax, PV and the bf16 store all run inside it.  Inputs are
seeded synthetic tensors already resident in HBM; several input sets are
rotated so that successive steps do not hit the 256 MB Infinity Cache.

Prints ONE JSON line on stdout.  Progress goes to stderr.
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

METRIC = "π-attn fwd queries/s + achieved HBM GB/s & MFMA %, n=8192 d=64 bf16, 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16
MALL_BYTES = 256 << 20
KERNEL_SOURCES = ["pattern.hpp", "common.hpp", "gather.hpp", "mfma_util.hpp", "fwd_gather.hip",
                  "fwd_resid.hip", "fwd_split.hip", "decode.hip", "api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest() -> str:
    """Digest of the kernel sources with comments and blank space removed, so
    that counters stay matched to the code they were taken on across edits
    that change no code."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_long_context_piattn_amd", "csrc")
    for name in KERNEL_SOURCES:
        p = os.path.join(csrc, name)
        if os.path.exists(p):
            text = open(p).read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(name.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def pair_counts(w, lengths=None):
    """(local, skip) scored pairs of the workload from the pattern's closed
    range arithmetic (vectorised over rows)."""
    import numpy as np

    # the distinct skip distances beyond the window (one level, or the union
    # of a schedule's levels); distance dd is a skip of the rows i >= dd
    # (and, bidirectional, of the rows i + dd <= n - 1)
    dist = sorted({m * p for p, M in [(w.pi, w.M)] + list(w.levels) for m in range(1, M + 1) if m * p > w.k})

    def one(n):
        i = np.arange(n, dtype=np.int64)
        lo = np.maximum(0, i - w.k)
        hi = np.minimum(n - 1, i + w.k) if w.bidir else i
        sk = sum(max(0, n - dd) for dd in dist) * (2 if w.bidir else 1)
        return int((hi - lo + 1).sum()), int(sk)

    if w.nseq:
        tot = [one(n) for n in lengths]
        loc, sk = sum(t[0] for t in tot), sum(t[1] for t in tot)
    else:
        loc, sk = one(w.n)
        loc, sk = loc * w.B, sk * w.B
    return loc * w.H, sk * w.H


def algorithmic(w, lengths=None):
    """Per-launch algorithmic bytes (q, k, v, out once each plus the fp32
    gate) and flops (4*d per scored pair), and the number of query rows."""
    esz = 4 if w.dtype == "f32" else 2
    T = sum(lengths) if w.nseq else w.B * w.n
    rows = T * w.H
    loc, sk = pair_counts(w, lengths)
    bytes_ = rows * (4 * w.d * esz + 4)
    flops = 4 * w.d * (loc + sk)
    return bytes_, flops, rows, loc, sk


def traffic_record(workload: str):
    """HBM bytes per step (all kernels of one hot-path pass) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_digest") != kernel_digest():
        return None
    return rec.get("hbm_bytes_per_step")


def cpu_baseline(w, x, budget_s: float):
    """Time the fp64 CPU oracle on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle

    threads = oracle.max_threads()
    B, H, n, d = x["q"].shape

    def host(t):
        t = t.detach().permute(0, 2, 1, 3).reshape(B * n, H, d).contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16)

    q, k, v = host(x["q"]), host(x["k"]), host(x["v"])
    g = x["g"].detach().permute(0, 2, 1).reshape(B * n, H).double().cpu().numpy()
    cu = np.arange(B + 1, dtype=np.int64) * n
    rng = np.random.default_rng(0)
    total_rows = B * n * H
    count = 4096
    elapsed = 0.0
    while True:
        rows = np.sort(rng.integers(0, total_rows, count))
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, g, cu, w.k, w.pi, w.M, w.bidir, w.scale, rows=rows, levels=w.levels)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s * 0.5 or count >= total_rows:
            break
        count = min(total_rows, int(count * max(2.0, budget_s / max(elapsed, 1e-3))))
    passes = 1
    if elapsed < budget_s * 0.5:
        # the whole workload is a small sample: repeat it up to half the budget
        passes = max(1, min(200, int(budget_s * 0.5 / max(elapsed, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(passes):
            oracle.fwd(q, k, v, g, cu, w.k, w.pi, w.M, w.bidir, w.scale, rows=rows, levels=w.levels)
        elapsed = time.perf_counter() - t0
    what = ("%d uniformly sampled query rows" % count if count < total_rows
            else "all query rows, %d pass%s," % (passes, "es" if passes > 1 else ""))
    return {"value": passes * count / elapsed, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": "%s of the %s workload (%d rows), fp64, OpenMP over rows, %.1f s"
                      % (what, w.name, total_rows, elapsed)}


def decode_algorithmic(w):
    """Per-call algorithmic bytes of decode: the K and V rows each (sequence,
    head) row touches, plus q, out and the fp32 gate; flops 4*d per pair."""
    import numpy as np
    i = w.n - 1
    loc = min(i, w.k) + 1
    mlo = w.k // w.pi + 1
    sk = max(0, min(w.M, i // w.pi) - mlo + 1)
    rows = w.B * w.H
    bytes_ = rows * (2 * (loc + sk) * w.d * 2 + 2 * w.d * 2 + 4)
    flops = rows * 4 * w.d * (loc + sk)
    return bytes_, flops, rows, loc, sk


def bench_decode(args, w, dev):
    import torch

    import sparse_long_context_piattn_amd as pa
    from sparse_long_context_piattn_amd import workloads as wl

    alg_bytes, alg_flops, rows, loc, sk = decode_algorithmic(w)
    log("workload %s: %d (sequence, head) rows x (%d local + %d skip) keys, %.1f MB/call"
        % (w.name, rows, loc, sk, alg_bytes / 1e6))
    x = wl.make_decode_inputs(w, device=dev)
    slots = None
    if args.rolling:
        # a rolling cache of W = max(k, M pi) + 1 rows holding the last W positions
        slots = pa.rolling_slots(w.k, w.pi, w.M)
        j = torch.arange(w.n - slots, w.n, device=dev)
        for name in ("k_cache", "v_cache"):
            ring = torch.empty((w.B, w.H, slots, w.d), dtype=x[name].dtype, device=dev)
            for s0 in range(0, w.B, 8):
                ring[s0:s0 + 8][:, :, j % slots] = x[name][s0:s0 + 8][:, :, j]
            x[name] = ring
            torch.cuda.empty_cache()
        log("rolling cache of %d rows per (sequence, head)" % slots)
    out = torch.empty_like(x["q"])
    pat = pa.make_pattern(w.k, w.pi, w.M)
    splits = args.splits
    need = pa.decode_workspace_bytes(w.B, w.H, w.d, splits, pat)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(_j):
        pa.decode(x["q"], x["k_cache"], x["v_cache"], x["lens"], x["g"], window_k=w.k,
                  period_pi=w.pi, num_skips=w.M, num_splits=splits, workspace=ws, out=out,
                  rolling=bool(args.rolling))

    ms_per_step = timed(step, args, dev)
    if args.calibrate_copy:
        calibrate_copy(dev)
    sec = ms_per_step / 1e3
    gbps = alg_bytes / sec / 1e9
    log("%.4f ms/call  %.3e row-queries/s  %.0f GB/s (%.1f%% of HBM peak)"
        % (ms_per_step, rows / sec, gbps, 100 * gbps / HBM_PEAK_GBPS))
    res = {"metric": "pi-attn decode (sequence, head) queries/s, 32K cache d=128 bf16, 1 GPU",
           "value": round(rows / sec, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) cache, query and gate logits)",
           "config": {"workload": w.name, "sequences": w.B, "H": w.H, "cache_len": w.n,
                      "d": w.d, "k": w.k, "pi": w.pi, "M": w.M, "num_splits": splits,
                      "cache": "rolling, %d rows" % slots if slots else "linear"},
           "hbm_gbps_algorithmic": round(gbps, 1), "kernel_digest": kernel_digest(),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "traffic": traffic_record(w.name)},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)


def bench_backward(args, w, dev, sets, outs, lengths, rows):
    """Time piattn_bwd (gradients of q, k, v and the gate logits) on the
    workload; the forward outputs and log-sum-exp it takes are computed
    first, untimed.  Algorithmic bytes per row: q, k, v, out, dout read and
    dq, dk, dv written once (8 d e), the fp32 gate logit and lse read and the
    gate gradient written (12)."""
    import torch

    import sparse_long_context_piattn_amd as pa

    nsets = len(sets)
    lses = []
    for j, x in enumerate(sets):
        lses.append(torch.empty_like(x["g"]))
        pa.fwd(x["q"], x["k"], x["v"], x["g"], window_k=w.k, period_pi=w.pi, num_skips=w.M,
               levels=w.levels, bidirectional=w.bidir, cu_seqlens=x.get("cu_seqlens"),
               max_seqlen=max(lengths) if lengths else None, out=outs[j], lse=lses[j])
    douts = []
    for j, x in enumerate(sets):
        gen = torch.Generator(device=dev).manual_seed(1000 + j)
        douts.append(torch.randn(x["q"].shape, generator=gen, device=dev).to(x["q"].dtype))
    e = 2 if w.dtype == "bf16" else 4
    alg_bytes = rows * (8 * w.d * e + 12)
    nb = pa.binding.lib().piattn_bwd_workspace_bytes(len(lengths) if lengths else w.B, w.H,
                                                       max(lengths) if lengths else w.n)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step(j):
        x = sets[j % nsets]
        pa.bwd(x["q"], x["k"], x["v"], x["g"], outs[j % nsets], douts[j % nsets], window_k=w.k,
               period_pi=w.pi, num_skips=w.M, levels=w.levels, bidirectional=w.bidir,
               cu_seqlens=x.get("cu_seqlens"),
               max_seqlen=max(lengths) if lengths else None, lse=lses[j % nsets], workspace=ws)

    ms_per_step = timed(step, args, dev)
    sec = ms_per_step / 1e3
    gbps = alg_bytes / sec / 1e9
    log("backward: %.4f ms/step  %.3e rows/s  %.0f GB/s (%.1f%% of HBM peak)"
        % (ms_per_step, rows / sec, gbps, 100 * gbps / HBM_PEAK_GBPS))
    res = {"metric": "pi-attn backward (dq, dk, dv, d gate) query rows/s, 1 GPU", "value": round(rows / sec, 1),
           "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
           "data": "synthetic (seeded N(0,1) q/k/v/dout, N(0,1) gate logits)",
           "config": {"workload": w.name, "pass": "backward", "B": w.B if not w.nseq else len(lengths),
                      "H": w.H, "n": w.n if not w.nseq else max(lengths), "d": w.d, "k": w.k, "pi": w.pi,
                      "M": w.M, "bidirectional": w.bidir, **({"levels": [list(l) for l in w.levels]} if w.levels else {})},
           "kernel_digest": kernel_digest(),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)


def bench_layer(args, w, dev):
    """gate logits -> attention -> output projection on the workload's shape
    (dense bf16 workloads; model width Dm = H d, random weights).  One step
    runs the three calls; each stage is also timed alone with HIP events on
    the launch stream.  The roofline is the output projection's (a GEMM on
    bf16 MFMA: 2 M Dm Dm flops)."""
    import torch

    import sparse_long_context_piattn_amd as pa
    from sparse_long_context_piattn_amd import workloads as wl

    if w.nseq or w.kind != "fwd" or w.dtype != "bf16":
        raise SystemExit("--layer takes a dense bf16 prefill workload")
    B, H, n, d = w.B, w.H, w.n, w.d
    Dm = H * d
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    rnd = lambda shape, std: (torch.randn(shape, generator=gen, device=dev) * std).to(torch.bfloat16)
    xs = wl.make_fwd_inputs(w, device=dev)
    x = rnd((B, n, Dm), 1.0)
    wg = rnd((H, Dm), Dm ** -0.5)
    wo = rnd((Dm, Dm), Dm ** -0.5)
    g = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    o = torch.empty_like(xs["q"])
    y = torch.empty((B, n, Dm), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, pa.fwd_workspace_bytes(1, B, H, n, d, pa.make_pattern(w.k, w.pi, w.M, w.bidir, 0.0,
                                                                                 w.levels))),
                     dtype=torch.uint8, device=dev)
    stages = {
        "gate": lambda: pa.gate_logits(x, wg, out=g),
        "attention": lambda: pa.fwd(xs["q"], xs["k"], xs["v"], g, window_k=w.k, period_pi=w.pi, num_skips=w.M,
                                    levels=w.levels, bidirectional=w.bidir, out=o, workspace=ws),
        "out_proj": lambda: pa.out_proj(o, wo, out=y),
    }

    def step(_):
        for f in stages.values():
            f()

    ms_per_step = timed(step, args, dev)
    stream = torch.cuda.current_stream(dev)
    per = {}
    for name, f in stages.items():
        for _ in range(20):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 100
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        per[name] = e0.elapsed_time(e1) / reps
    # the same GEMM in torch's library path, for context (o token-major and
    # contiguous there: the head concatenation is a copy in that path)
    ocat = o.permute(0, 2, 1, 3).reshape(B * n, Dm).contiguous()
    lib_gemm = lambda: torch.nn.functional.linear(ocat, wo)
    for _ in range(20):
        lib_gemm()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(100):
        lib_gemm()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    lib_ms = e0.elapsed_time(e1) / 100
    M = B * n
    flops = 2.0 * M * Dm * Dm
    tflops = flops / (per["out_proj"] / 1e3) / 1e12
    gate_bytes = M * Dm * 2 + M * H * 4
    log("layer: %.4f ms/step  gate %.4f ms (%.0f GB/s)  attention %.4f ms  out_proj %.4f ms (%.0f TFLOP/s, "
        "%.1f%% of bf16 MFMA peak); torch linear on a contiguous copy %.4f ms"
        % (ms_per_step, per["gate"], gate_bytes / (per["gate"] / 1e3) / 1e9, per["attention"], per["out_proj"],
           tflops, 100 * tflops / BF16_MFMA_PEAK_TFLOPS, lib_ms))
    res = {"metric": "pi-attn layer (gate + attention + output projection) tokens/s, 1 GPU",
           "value": round(M / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) x, q/k/v; random-init gate and projection weights)",
           "config": {"workload": w.name, "pass": "layer", "B": B, "H": H, "n": n, "d": d, "Dm": Dm, "k": w.k,
                      "pi": w.pi, "M": w.M, "bidirectional": w.bidir},
           "stages_ms": {k_: round(v_, 5) for k_, v_ in per.items()},
           "torch_linear_ms": round(lib_ms, 5),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)


COPY_ELEMS = 256 << 20          # bf16 elements of the calibration copy (512 MiB each way)


def calibrate_copy(dev):
    """A plain streaming copy of known size: reads and writes 512 MiB."""
    import torch
    src = torch.empty(COPY_ELEMS, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def step_stats(step, dev, nsteps=60):
    """Secondary timings after the timed region: per-step durations (HIP
    events around each step on the launch stream; p10 / p50 / p90 in ms) and
    a warm time with one input set repeated (which the Infinity Cache may then
    serve)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    evs[0].record(stream)
    for j in range(nsteps):
        step(j)
        evs[j + 1].record(stream)
    torch.cuda.synchronize(dev)
    per = sorted(evs[j].elapsed_time(evs[j + 1]) for j in range(nsteps))
    q = lambda f: per[min(nsteps - 1, int(f * nsteps))]
    for _ in range(10):
        step(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(nsteps):
        step(0)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    return {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5),
            "warm_ms_per_step": round(e0.elapsed_time(e1) / nsteps, 5)}


def copy_peak_gbps(dev):
    """Achievable HBM rate: a plain 512 MiB bf16 copy (read + write), timed
    with HIP events."""
    import torch
    src = torch.empty(COPY_ELEMS, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    gbps = 2 * COPY_ELEMS * 2 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return gbps


def _counter_rows(d):
    """(kernel name, counter, value, dispatch id) from a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % d)
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]),
                         r["Dispatch_Id"]))
    return rows


def _per_dispatch(rows, counter, match):
    """Per matching kernel, the median over its dispatches of the summed
    counter value; returned summed over the kernels (one step launches each
    matching kernel once), with the number of dispatches and kernel names."""
    import statistics
    per = {}
    for name, cn, val, disp in rows:
        if cn == counter and match(name):
            d = per.setdefault(name, {})
            d[disp] = d.get(disp, 0.0) + val
    if not per:
        raise SystemExit("no %s dispatch matched" % counter)
    total = sum(statistics.median(d.values()) for d in per.values())
    return total, sum(len(d) for d in per.values()), sorted(per)


def pmc_summary(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the forward kernels, each
    scaled by the reading of the same counter on the plain copy, summed over
    the kernels of one step into the HBM bytes per step that bench.py
    reports as roofline.traffic."""
    fetch_rows, write_rows = _counter_rows(args.pmc_summary[0]), _counter_rows(args.pmc_summary[1])
    is_fwd = lambda name: "fwd_" in name and "kernel" in name
    is_copy = lambda name: "elementwise" in name and "MulFunctor" in name   # calibrate_copy
    f_fwd, nf, knames = _per_dispatch(fetch_rows, "FETCH_SIZE", is_fwd)
    w_fwd, nw, _ = _per_dispatch(write_rows, "WRITE_SIZE", is_fwd)
    f_cp, _, _ = _per_dispatch(fetch_rows, "FETCH_SIZE", is_copy)
    w_cp, _, _ = _per_dispatch(write_rows, "WRITE_SIZE", is_copy)
    copy_kib = COPY_ELEMS * 2 / 1024.0
    fs, ws = copy_kib / f_cp, copy_kib / w_cp
    rec = {"workload": args.workload, "kernels": knames, "kernel_digest": kernel_digest(),
           "fetch_kib_per_step": f_fwd, "write_kib_per_step": w_fwd,
           "dispatches": [nf, nw],
           "copy_kib_each_way": copy_kib, "copy_fetch_kib": f_cp, "copy_write_kib": w_cp,
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "hbm_bytes_per_step": int(round((f_fwd * fs + w_fwd * ws) * 1024))}
    out = os.path.join(ROOT, "profiles", "traffic_%s.json" % args.workload)
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def timed(step, args, dev):
    import torch
    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for j in range(args.steps):
        step(j)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / args.steps


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # 200 untimed steps (~25 ms of prefill_8k) let the GPU reach its steady clocks;
    # after only 10 the timed steps of prefill_8k ran ~5% slower
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = auto)")
    ap.add_argument("--splits", type=int, default=0, help="decode key-range splits (0 = auto)")
    ap.add_argument("--layer", action="store_true",
                    help="time gate logits + attention + output projection (dense bf16 prefill workloads)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (piattn_bwd) instead of the forward (prefill workloads)")
    ap.add_argument("--rolling", action="store_true",
                    help="decode over a rolling cache of max(k, M pi) + 1 rows")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 512 MiB bf16 copy three times "
                         "(reference dispatches for the HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv runs of "
                         "'bench.py --calibrate-copy' into profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(args)

    if args.gpus != 1:
        log("bench.py runs on exactly one GPU: this build has no multi-GPU path "
            "(a (sequence, head) shard per GPU would need no exchange; see the design notes).")
        sys.exit(2)

    import torch

    import sparse_long_context_piattn_amd as pa
    from sparse_long_context_piattn_amd import workloads as wl

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[args.workload]
    if w.kind == "decode":
        return bench_decode(args, w, dev)
    if args.layer:
        return bench_layer(args, w, dev)
    lengths = wl.varlen_lengths(w) if w.nseq else None
    alg_bytes, alg_flops, rows, loc, sk = algorithmic(w, lengths)
    set_bytes = alg_bytes
    nsets = args.sets or max(1, math.ceil(3 * MALL_BYTES / set_bytes))
    nsets = min(nsets, 6)
    log("workload %s: %d rows, %d local + %d skip pairs, %.1f MB/launch, %d input sets"
        % (w.name, rows, loc, sk, alg_bytes / 1e6, nsets))
    sets = [wl.make_fwd_inputs(w, device=dev, seed=w.seed + s, lengths=lengths)
            for s in range(nsets)]
    outs = [torch.empty_like(x["q"]) for x in sets]
    # one workspace for every step (the steps are ordered on one stream)
    nb = pa.fwd_workspace_bytes(1 if w.dtype == "bf16" else 0, len(lengths) if lengths else w.B, w.H,
                                max(lengths) if lengths else w.n, w.d,
                                pa.make_pattern(w.k, w.pi, w.M, w.bidir, w.scale, w.levels))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

    def step(j):
        x = sets[j % nsets]
        pa.fwd(x["q"], x["k"], x["v"], x["g"], window_k=w.k, period_pi=w.pi, num_skips=w.M,
               levels=w.levels, bidirectional=w.bidir, cu_seqlens=x.get("cu_seqlens"),
               max_seqlen=max(lengths) if lengths else None, out=outs[j % nsets], workspace=ws)

    if args.backward:
        return bench_backward(args, w, dev, sets, outs, lengths, rows)

    ms_per_step = timed(step, args, dev)
    if args.calibrate_copy:
        calibrate_copy(dev)
    sec = ms_per_step / 1e3
    qps = rows / sec
    achieved_gbps = alg_bytes / sec / 1e9
    tflops = alg_flops / sec / 1e12
    log("%.4f ms/step  %.3e queries/s  %.0f GB/s (%.1f%% of HBM peak)  %.2f TFLOP/s (%.2f%% MFMA)"
        % (ms_per_step, qps, achieved_gbps, 100 * achieved_gbps / HBM_PEAK_GBPS, tflops,
           100 * tflops / BF16_MFMA_PEAK_TFLOPS))

    stats = step_stats(step, dev)
    copy_gbps = copy_peak_gbps(dev)
    log("steps p10/p50/p90 %.4f/%.4f/%.4f ms, warm (one input set) %.4f ms; copy %.0f GB/s -> %.1f%% of it"
        % (stats["p10"], stats["p50"], stats["p90"], stats["warm_ms_per_step"], copy_gbps,
           100 * achieved_gbps / copy_gbps))

    traffic = traffic_record(w.name)
    roof = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a sample ...")
        cpu = cpu_baseline(w, sets[0], args.cpu_budget)
        log("oracle: %.3e queries/s on %d threads" % (cpu["value"], cpu["cores"]))

    cfg = {"workload": w.name, "B": w.B if not w.nseq else len(lengths), "H": w.H,
           "n": w.n if not w.nseq else max(lengths), "d": w.d, "k": w.k, "pi": w.pi, "M": w.M,
           "bidirectional": w.bidir, "global_batch": w.B, "seq_len": w.n,
           "parallelism": "single GPU", "input_sets": nsets}
    if w.levels:
        cfg["levels"] = [list(l) for l in w.levels]
    res = {"metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
           if w.dtype == "bf16" else "f32", "data": "synthetic (seeded N(0,1) q/k/v, N(0,1) "
           "gate logits)", "config": cfg,
           "hbm_gbps_algorithmic": round(achieved_gbps, 1),
           "tflops_algorithmic": round(tflops, 3),
           "mfma_pct_algorithmic": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 3),
           "tokens_per_s": round(qps / w.H, 1),
           "step_ms": {k_: v_ for k_, v_ in stats.items() if k_ != "warm_ms_per_step"},
           "warm_ms_per_step": stats["warm_ms_per_step"],
           "copy_gbps_measured": round(copy_gbps, 1),
           "frac_of_measured_copy": round(achieved_gbps / copy_gbps, 4),
           "kernel_digest": kernel_digest(),
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
