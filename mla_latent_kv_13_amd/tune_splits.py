"""Offline split-count tuner: times mla_decode on the 8-shape grid and writes
the table that mla_choose_num_splits consults.

For every batch in {4, 32, 64, 256}, kv_len in {1024, 8192} and cache format
(bf16, fp8, mxfp4; bf16 Q, page size 8, shuffled pages) it times every split
count S in 1..64 that leaves at least one 32-token sub-tile per split, as HIP
graph replays over rotated buffer replicas (at least 1 GB of working set, so
the figures are HBM figures rather than Infinity Cache ones), and keeps the
fastest S.  It also times the split count the library's cost model picks
on its own (the fallback for shapes off the grid), so the table records how
far that model is from the measured optimum.  Output: a C include file of
{batch, kv_len, kv_dtype, splits, us, model_splits, model_us} rows (the
library is rebuilt with it) and one JSON line per measurement on stdout.

    python -m mla_latent_kv_13_amd.tune_splits --out mla_latent_kv_13_amd/csrc/split_table.inc > sweep.jsonl

The table can be rewritten from such a log without a GPU:

    python -m mla_latent_kv_13_amd.tune_splits --from-log sweep.jsonl --out mla_latent_kv_13_amd/csrc/split_table.inc

Needs a GPU; the shapes follow the pages' benchmark grid (bs x kv_len) with
N(0,1) synthetic inputs, like the benchmark workloads.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

from . import (BF16, FP8, MXFP4, choose_num_splits, decode, load, new_workspace, quantize_fp8, quantize_mxfp4,
               workspace_bytes)
from . import synth

BATCHES = (4, 32, 64, 256)
KV_LENS = (1024, 8192)
FORMATS = (("bf16", BF16), ("fp8", FP8), ("mxfp4", MXFP4))
SPLITS = (1, 2, 4, 8, 16, 32, 64)
CODES = {fmt: code for fmt, code in FORMATS}
# The tuned table applies on 256 CUs only; asking for one CU more returns the
# cost model's own pick (the two agree on rounds of workgroups for every grid
# shape).
MODEL_CUS = 257


def model_splits(batch, kv_len, code):
    return int(choose_num_splits(batch, kv_len, code, MODEL_CUS))


def _inputs(batch, kv_len, fmt, seed):
    case = synth.make_case(batch, kv_len, 8, shuffle=True, seed=seed, device="cuda")
    ops = {"q": case["q"], "ind": case["kv_indptr"], "pt": case["page_table"], "ks": None}
    if fmt == "fp8":
        ops["kv"], ops["ks"] = quantize_fp8(case["kv"])
    elif fmt == "mxfp4":
        ops["kv"], ops["ks"] = quantize_mxfp4(case["kv"])
    else:
        ops["kv"] = case["kv"]
    del case
    return ops


def _time(reps, S, nrep, calls_per_group=None, groups=5):
    """Median us per call of graph-replayed calls cycling over the replicas."""
    per = calls_per_group or max(nrep, 8)

    def call(i):
        r = reps[i % nrep]
        decode(r["q"], r["kv"], r["ind"], r["pt"], 8, S, kv_scale=r["ks"], out=r["out"], workspace=r["ws"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per):
            call(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(groups)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) / per for e0, e1 in evs)
    del g
    return ms[len(ms) // 2] * 1e3


def tune(out_path: str | None):
    load()
    rows = []
    for bi, batch in enumerate(BATCHES):
        for ki, kv_len in enumerate(KV_LENS):
            for fmt, code in FORMATS:
                base = _inputs(batch, kv_len, fmt, synth.BASE_SEED + 100 + 10 * bi + ki)
                smax = max(s for s in SPLITS if s == 1 or kv_len // s >= 32)
                ws_bytes = workspace_bytes(batch, smax)
                work = sum(v.numel() * v.element_size() for v in base.values() if v is not None) + ws_bytes
                nrep = 1 if work >= (512 << 20) else min(256, max(2, math.ceil((1 << 30) / work)))
                reps = []
                for r in range(nrep):
                    d = base if r == 0 else {k: (None if v is None else v.clone()) for k, v in base.items()}
                    d = dict(d)
                    d["out"] = torch.empty((batch, 16, 512), dtype=torch.bfloat16, device="cuda")
                    d["ws"] = new_workspace(ws_bytes, "cuda")
                    reps.append(d)
                model = model_splits(batch, kv_len, code)
                timed = {}
                for S in sorted(set(s for s in SPLITS if s <= smax) | {model}):
                    us = _time(reps, S, nrep)
                    timed[S] = us
                    print(json.dumps({"batch": batch, "kv_len": kv_len, "kv": fmt, "splits": S, "us": round(us, 3),
                                      "replicas": nrep}), flush=True)
                rows.append(_row(batch, kv_len, fmt, timed, model))
                del reps, base
                torch.cuda.empty_cache()
    if out_path:
        dev = getattr(torch.cuda.get_device_properties(0), "gcnArchName", torch.cuda.get_device_name(0))
        _write(out_path, rows, f"{dev}, {time.strftime('%Y-%m-%d')}")
    return rows


def _row(batch, kv_len, fmt, timed, model):
    best = min(timed, key=lambda s: (timed[s], s))
    row = (batch, kv_len, CODES[fmt], best, timed[best], model, timed[model], fmt)
    print(json.dumps({"batch": batch, "kv_len": kv_len, "kv": fmt, "best_splits": best, "best_us": round(timed[best], 3),
                      "model_splits": model, "model_us": round(timed[model], 3)}), flush=True)
    return row


def _write(out_path, rows, where):
    with open(out_path, "w") as f:
        f.write("// Generated by mla_latent_kv_13_amd/tune_splits.py (HIP graph replays, rotated buffers,\n")
        f.write(f"// bf16 Q, page size 8, shuffled pages) on {where}.\n")
        f.write("// {batch, kv_len, kv_dtype, fastest num_splits, microseconds at that count,\n")
        f.write("//  the cost model's own num_splits, microseconds at that count}\n")
        for batch, kv_len, code, s, us, model, model_us, fmt in rows:
            f.write(f"{{{batch}, {kv_len}, {code}, {s}, {us:.2f}, {model}, {model_us:.2f}}},  // {fmt}\n")


def from_log(log_path, out_path, where=None):
    """Rebuild the table from the JSON lines of an earlier GPU run (no GPU);
    `where` names that run (device and date) in the table's header."""
    timed = {}
    for line in open(log_path):
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        if "splits" in r:
            timed.setdefault((r["batch"], r["kv_len"], r["kv"]), {})[r["splits"]] = r["us"]
    rows = []
    for batch in BATCHES:
        for kv_len in KV_LENS:
            for fmt, code in FORMATS:
                t = timed[(batch, kv_len, fmt)]
                model = model_splits(batch, kv_len, code)
                if model not in t:
                    raise SystemExit(f"the log has no timing of the model's pick S={model} for {(batch, kv_len, fmt)}")
                rows.append(_row(batch, kv_len, fmt, t, model))
    _write(out_path, rows, where or f"the GPU run logged in {os.path.basename(log_path)}")
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the C table here")
    ap.add_argument("--from-log", default=None, help="rebuild the table from this run's JSON lines (no GPU)")
    ap.add_argument("--where", default=None, help="with --from-log: the device and date of that run, for the header")
    args = ap.parse_args()
    if args.from_log:
        load()
        from_log(args.from_log, args.out, args.where)
        return
    if not torch.cuda.is_available():
        print("tune_splits needs a GPU", file=sys.stderr)
        sys.exit(2)
    tune(args.out)


if __name__ == "__main__":
    main()
