#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X: microseconds per call and achieved HBM GB/s.

A "step" is one mla_decode call (stage 1 + stage 2 when S > 1) over one batch
of synthetic inputs already resident in HBM.  The headline workload is
bs=256, kv_len=8192, bf16 Q over an fp8 e4m3fn paged cache (page 8, shuffled
pages), where the 70%-of-HBM-peak target is stated.  `value` is achieved
GB/s of compulsory traffic (cache incl. scales + Q + page table + indptr +
output) per second; split-K partials are not credited.  The remaining
workloads (the five benchmark shapes) are timed too and listed under
"workloads", each with rotated buffer replicas when its working set would fit
the 256 MB Infinity Cache.

Prints ONE JSON line.  --gpus must be 1 (this build runs on a single GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

import mla_latent_kv_13_amd as mla  # noqa: E402
from mla_latent_kv_13_amd import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
HEADLINE = "bs256_kv8192_a16w8"
FMT = {"bf16": mla.BF16, "fp8": mla.FP8, "mxfp4": mla.MXFP4}


def compulsory_bytes(w, page_size) -> int:
    T = w.batch * w.kv_len
    kv = {"bf16": 1152, "fp8": 576, "mxfp4": 288 + 18}[w.kv_fmt] * T
    q = {"bf16": 2 * 576, "fp8": 576, "mxfp4": 288 + 18}[w.q_fmt] * w.batch * 16
    pt = 4 * math.ceil(T / page_size)
    return kv + q + pt + 4 * (w.batch + 1) + 2 * w.batch * 16 * 512


def build_inputs(w, device):
    case = synth.workload_case(w, device=device)
    B = w.batch
    ops = {"kv_indptr": case["kv_indptr"], "page_table": case["page_table"]}
    if w.kv_fmt == "fp8":
        ops["kv"], ops["kv_scale"] = mla.quantize_fp8(case["kv"])
    elif w.kv_fmt == "mxfp4":
        ops["kv"], ops["kv_scale"] = mla.quantize_mxfp4(case["kv"])
    else:
        ops["kv"], ops["kv_scale"] = case["kv"], None
    if w.q_fmt == "fp8":
        ops["q"], ops["q_scale"] = mla.quantize_fp8(case["q"], w.q_scale)
    elif w.q_fmt == "mxfp4":
        p, s = mla.quantize_mxfp4(case["q"].reshape(B * 16, 576))
        ops["q"], ops["q_scale"] = p.reshape(B, 16, 288), s
    else:
        ops["q"], ops["q_scale"] = case["q"], None
    del case
    return ops


def replicate(ops, n):
    reps = [ops]
    for _ in range(n - 1):
        reps.append({k: (None if v is None else v.clone()) for k, v in ops.items()})
    return reps


def time_workload(w, steps, warmup, device):
    S = w.num_splits or mla.choose_num_splits(w.batch, w.kv_len, FMT[w.kv_fmt])
    ops = build_inputs(w, device)
    ws_bytes = mla.workspace_bytes(w.batch, S)
    work = sum(v.numel() * v.element_size() for v in ops.values() if v is not None) + ws_bytes + w.batch * 16 * 1024
    nrep = 1 if work >= (512 << 20) else min(256, max(2, math.ceil((1 << 30) / work)))
    reps = replicate(ops, nrep)
    for r in reps:
        r["out"] = torch.empty((w.batch, 16, 512), dtype=torch.bfloat16, device=device)
        r["ws"] = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device) if ws_bytes else None

    def call(i):
        r = reps[i % nrep]
        mla.decode(r["q"], r["kv"], r["kv_indptr"], r["page_table"], w.page_size, S, q_scale=r["q_scale"],
                   kv_scale=r["kv_scale"], out=r["out"], workspace=r["ws"])

    # warm up for at least `warmup` calls and ~0.3 s, so clocks and caches settle
    i = 0
    t_end = time.perf_counter() + 0.3
    while i < warmup or time.perf_counter() < t_end:
        call(i)
        i += 1
        if i % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # `steps` timed calls, in five back-to-back groups timed with HIP events on
    # the launch stream; the headline is the median group (per call)
    ngroups = 5
    per = max(1, steps // ngroups)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ngroups)]
    t0 = time.perf_counter()
    k = i
    for r in range(ngroups):
        evs[r][0].record(stream)
        for _ in range(per):
            call(k)
            k += 1
        evs[r][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / (ngroups * per)
    group_ms = sorted(e0.elapsed_time(e1) / per for e0, e1 in evs)
    ev_ms = group_ms[len(group_ms) // 2]
    nbytes = compulsory_bytes(w, w.page_size)
    res = {
        "workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q": w.q_fmt, "kv": w.kv_fmt,
        "page_size": w.page_size, "num_splits": S, "replicas": nrep,
        "us_per_call": round(ev_ms * 1e3, 3), "us_min": round(group_ms[0] * 1e3, 3),
        "us_max": round(group_ms[-1] * 1e3, 3), "wall_us_per_call": round(wall * 1e6, 3),
        "compulsory_bytes": nbytes, "gbs": round(nbytes / (ev_ms * 1e-3) / 1e9, 1),
        "frac_of_peak": round(nbytes / (ev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "partial_bytes": 2 * ws_bytes,
        "tflops": round(2 * 16 * w.batch * w.kv_len * (576 + 512) / (ev_ms * 1e-3) / 1e12, 2),
    }
    del reps, ops
    torch.cuda.empty_cache()
    return res, wall


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the headline workload (whole requests, all heads)."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    case = synth.workload_case(w, device="cuda")
    kv_bits = case["kv"].view(torch.int16).cpu().numpy().view(np.uint16)
    q_bits = case["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    del case
    sc = oracle.fp8_scale_from_amax(oracle.amax_bf16(kv_bits)) if w.kv_fmt == "fp8" else None
    P = w.page_size
    npages = math.ceil(w.batch * w.kv_len / P)
    perm = (torch.randperm(npages, generator=torch.Generator().manual_seed(synth.BASE_SEED + w.index + 1000)).numpy()
            if w.shuffle else np.arange(npages))

    def run(n):
        # the first n requests, compacted to their own rows behind an identity page table
        gpos = np.arange(n * w.kv_len)
        rows = perm[gpos // P].astype(np.int64) * P + gpos % P
        sub = np.ascontiguousarray(kv_bits[rows])
        if w.kv_fmt == "fp8":
            kv, _ = oracle.quant_fp8(sub, sc)
            extra = {"kv_dtype": "fp8", "kv_scale": sc}
        else:
            kv, extra = sub, {"kv_dtype": "bf16"}
        ind = (np.arange(n + 1) * w.kv_len).astype(np.int32)
        t0 = time.perf_counter()
        oracle.decode(q_bits[:n], kv, ind, np.arange(n * w.kv_len, dtype=np.int32), 1, nthreads=cores, **extra)
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(w.batch, int(budget_s / max(t1, 1e-3))))
    t = run(n) if n > 1 else t1
    per_req = t / n
    full = per_req * w.batch
    nbytes = compulsory_bytes(w, P)
    return {"value": round(nbytes / full / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.batch} requests x 16 heads x {w.kv_len} tokens ({w.name}), fp64 C oracle, "
                      f"{t:.1f} s; full call extrapolated to {full:.1f} s",
            "us_per_call": round(full * 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(synth.WORKLOADS))
    ap.add_argument("--only-headline", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of decoding, run a plain device-to-device copy of this many bytes "
                         "(the known-size reference used to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(requests shard across GPUs with no communication; see the design notes).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mla.load()
    device = "cuda"
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"metric": "device copy", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "us_per_copy": round(dt * 1e6, 2), "gbs": round(2 * src.numel() * 4 / dt / 1e9, 1)}))
        return
    w = synth.WORKLOADS[args.workload]
    print(f"[bench] headline {w.name}", file=sys.stderr, flush=True)
    head, wall = time_workload(w, args.steps, args.warmup, device)
    others = []
    if not args.only_headline:
        for name, ow in synth.WORKLOADS.items():
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            others.append(time_workload(ow, max(10, args.steps // 2), args.warmup, device)[0])
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
    gbs = head["gbs"]
    line = {
        "metric": "us/call and achieved HBM GB/s (% of peak) for MLA decode, bs x kv_len",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "us_per_call": head["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.q_fmt == "bf16" else w.q_fmt,
        "data": "synthetic (seeded N(0,1) bf16 Q and cache rows, quantised on the GPU)",
        "config": {"workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q": w.q_fmt, "kv": w.kv_fmt,
                   "page_size": w.page_size, "num_splits": head["num_splits"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["frac_of_peak"], "traffic": None},
        "cpu_baseline": cpu,
        "workloads": [head] + others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
