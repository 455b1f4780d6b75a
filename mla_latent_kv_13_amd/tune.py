"""Offline tuner of the split count and page size: times mla_decode on the
8-shape grid for every (Q, cache) format pair and writes the table that
mla_choose_num_splits and mla_recommend_page_size consult.

Grid: batch {4, 32, 64, 256} x kv_len {1024, 8192} x (Q, cache) in
{bf16/bf16, bf16/fp8, fp8/fp8, bf16/mxfp4, mxfp4/mxfp4} (fp8 Q with the static
6/448 scale), shuffled pages.  Per grid point:

  1. every split count S in {1, 2, 4, ..., 64} that leaves each split at
     least one 32-token sub-tile and at most four rounds of workgroups per
     CU, at page size 8;
  2. every page size P in {1, 2, 4, ..., 64} at the fastest S of step 1;
  3. S / 2 and 2 S around that S at the fastest P of step 2 (when P != 8);
  4. the pick of the library's own cost models (the fallback off the grid),
     so the table records how far the models are from the measured optimum.

Each timing is the median of seven groups of HIP graph replays of
back-to-back calls over rotated buffer replicas (at least 1 GB of working
set, so the figures are HBM figures, not Infinity Cache ones), after at
least half a second of warm-up replays on each new shape; steps 1 and 2 are
timed twice, forward then in reverse order, keeping the faster of the two
(neighbouring points otherwise differ by a few per cent of noise).  The cache
contents stay the same for every P: only the page table (a seeded random
permutation of the T / P pages) changes.  Output: one JSON line per timing on
stdout and, with --out, the C include file of rows
{batch, kv_len, q_dtype, kv_dtype, splits, page_size, us, model_splits,
model_page_size, model_us} (the library is rebuilt with it).

    python -m mla_latent_kv_13_amd.tune --out mla_latent_kv_13_amd/csrc/tune_table.inc > sweep.jsonl

The table can be rewritten from such a log without a GPU:

    python -m mla_latent_kv_13_amd.tune --from-log sweep.jsonl --out mla_latent_kv_13_amd/csrc/tune_table.inc

The shapes follow the pages' benchmark grid (bs x kv_len) with N(0,1)
synthetic inputs, like the benchmark workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

from . import (BF16, FP8, MXFP4, choose_num_splits, decode, load, new_workspace, quantize_fp8, quantize_mxfp4,
               recommend_page_size, workspace_bytes)
from . import synth

BATCHES = (4, 32, 64, 256)
KV_LENS = (1024, 8192)
PAIRS = (("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8"), ("bf16", "mxfp4"), ("mxfp4", "mxfp4"))
SPLITS = (1, 2, 4, 8, 16, 32, 64)
PAGES = (1, 2, 4, 8, 16, 32, 64)
REF_PAGE = 8
CODES = {"bf16": BF16, "fp8": FP8, "mxfp4": MXFP4}
Q_STATIC = 6.0 / 448.0
# The tuned table applies on 256 CUs only; asking for one CU more returns the
# cost models' own picks.
MODEL_CUS = 257
KERNEL_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "mla_decode.hip")


def kernel_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def model_pick(batch, kv_len, q, kv):
    return (int(choose_num_splits(batch, kv_len, CODES[kv], MODEL_CUS, q_dtype=CODES[q])),
            int(recommend_page_size(batch, kv_len, CODES[q], CODES[kv], MODEL_CUS)))


def split_candidates(batch, kv_len):
    return [s for s in SPLITS if s == 1 or (kv_len // s >= 32 and batch * s <= 4 * 256)]


def _inputs(batch, kv_len, q, kv, seed):
    case = synth.make_case(batch, kv_len, 1, shuffle=False, seed=seed, device="cuda")
    ops = {"ind": case["kv_indptr"], "ks": None, "qs": None}
    if kv == "fp8":
        ops["kv"], ops["ks"] = quantize_fp8(case["kv"])
    elif kv == "mxfp4":
        ops["kv"], ops["ks"] = quantize_mxfp4(case["kv"])
    else:
        ops["kv"] = case["kv"]
    if q == "fp8":
        ops["q"], ops["qs"] = quantize_fp8(case["q"], Q_STATIC)
    elif q == "mxfp4":
        p, s = quantize_mxfp4(case["q"].reshape(batch * 16, 576))
        ops["q"], ops["qs"] = p.reshape(batch, 16, 288), s
    else:
        ops["q"] = case["q"]
    del case
    return ops


def _page_table(T, P, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(T // P, generator=g).to(torch.int32).to("cuda")


def _time(reps, S, P, nrep, groups=7, warmup_s=0.0):
    """Median us per call of graph-replayed calls cycling over the replicas."""
    per = max(nrep, 8)

    def call(i):
        r = reps[i % nrep]
        decode(r["q"], r["kv"], r["ind"], r["pt"][P], P, S, q_scale=r["qs"], kv_scale=r["ks"], out=r["out"],
               workspace=r["ws"])

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
    t_end = time.perf_counter() + warmup_s
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(groups)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) / per for e0, e1 in evs)
    del g
    return ms[len(ms) // 2] * 1e3


def tune_point(batch, kv_len, q, kv, seed):
    T = batch * kv_len
    base = _inputs(batch, kv_len, q, kv, seed)
    cands = split_candidates(batch, kv_len)
    ms, mp = model_pick(batch, kv_len, q, kv)
    ws_bytes = workspace_bytes(batch, max(cands + [ms]))
    pts = {P: _page_table(T, P, seed + P) for P in PAGES}
    work = sum(v.numel() * v.element_size() for v in base.values() if v is not None) + ws_bytes
    work += 4 * T  # the page-table set of one replica, as read
    nrep = 1 if work >= (512 << 20) else min(256, max(2, math.ceil((1 << 30) / work)))
    reps = []
    for r in range(nrep):
        d = dict(base) if r == 0 else {k: (None if v is None else v.clone()) for k, v in base.items()}
        d["pt"] = pts if r == 0 else {P: t.clone() for P, t in pts.items()}
        d["out"] = torch.empty((batch, 16, 512), dtype=torch.bfloat16, device="cuda")
        d["ws"] = new_workspace(ws_bytes, "cuda")
        reps.append(d)
    timed = {}

    def run(S, P, again=False):
        if (S, P) not in timed or again:
            us = _time(reps, S, P, nrep)
            timed[(S, P)] = min(us, timed.get((S, P), us))
            print(json.dumps({"batch": batch, "kv_len": kv_len, "q": q, "kv": kv, "splits": S, "page": P,
                              "us": round(us, 3), "replicas": nrep}), flush=True)
        return timed[(S, P)]

    _time(reps, cands[-1], REF_PAGE, nrep, warmup_s=0.5)  # clocks, caches and TLBs settle on the new buffers
    for S in cands:
        run(S, REF_PAGE)
    for S in reversed(cands):
        run(S, REF_PAGE, again=True)
    s_best = min(cands, key=lambda s: (timed[(s, REF_PAGE)], s))
    for P in PAGES:
        run(s_best, P, again=P == REF_PAGE)
    for P in reversed(PAGES):
        run(s_best, P, again=True)
    p_best = min(PAGES, key=lambda p: (timed[(s_best, p)], p))
    if p_best != REF_PAGE:
        for S in (s_best // 2, 2 * s_best):
            if S in cands:
                run(S, p_best)
    run(ms, mp)
    del reps, base, pts
    torch.cuda.empty_cache()
    return timed


def _row(batch, kv_len, q, kv, timed):
    """Fastest (S, P) of one grid point (ties: smaller S, then smaller P) and
    the models' pick with its time."""
    best = min(timed, key=lambda k: (timed[k], k))
    ms, mp = model_pick(batch, kv_len, q, kv)
    if (ms, mp) not in timed:
        raise SystemExit(f"no timing of the models' pick S={ms} P={mp} for {(batch, kv_len, q, kv)}")
    row = (batch, kv_len, CODES[q], CODES[kv], best[0], best[1], timed[best], ms, mp, timed[(ms, mp)], f"{q}/{kv}")
    print(json.dumps({"batch": batch, "kv_len": kv_len, "q": q, "kv": kv, "best_splits": best[0], "best_page": best[1],
                      "best_us": round(timed[best], 3), "model_splits": ms, "model_page": mp,
                      "model_us": round(timed[(ms, mp)], 3)}), flush=True)
    return row


def _write(out_path, rows, where):
    with open(out_path, "w") as f:
        f.write("// Generated by mla_latent_kv_13_amd/tune.py (HIP graph replays, rotated buffers, shuffled\n")
        f.write(f"// pages) on {where}.\n")
        f.write("// {batch, kv_len, q_dtype, kv_dtype, fastest num_splits, fastest page_size, microseconds there,\n")
        f.write("//  the cost models' num_splits and page_size, microseconds there}\n")
        for batch, kv_len, qc, kc, s, p, us, ms, mp, mus, name in rows:
            f.write(f"{{{batch}, {kv_len}, {qc}, {kc}, {s}, {p}, {us:.2f}, {ms}, {mp}, {mus:.2f}}},  // {name}\n")


def tune(out_path: str | None):
    load()
    print(json.dumps({"kernel_source_sha256": kernel_sha()}), flush=True)
    rows = []
    for bi, batch in enumerate(BATCHES):
        for ki, kv_len in enumerate(KV_LENS):
            for pi, (q, kv) in enumerate(PAIRS):
                timed = tune_point(batch, kv_len, q, kv, synth.BASE_SEED + 100 + 20 * bi + 10 * ki + pi)
                rows.append(_row(batch, kv_len, q, kv, timed))
    if out_path:
        dev = getattr(torch.cuda.get_device_properties(0), "gcnArchName", torch.cuda.get_device_name(0))
        _write(out_path, rows, f"{dev}, {time.strftime('%Y-%m-%d')}, kernel source sha256 {kernel_sha()[:16]}")
    return rows


def from_log(log_path, out_path, where=None):
    """Rebuild the table from the JSON lines of an earlier GPU run (no GPU);
    `where` names that run (device, date, kernel) in the table's header."""
    timed = {}
    sha = None
    for line in open(log_path):
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        if "kernel_source_sha256" in r:
            sha = r["kernel_source_sha256"]
        if "splits" in r and "page" in r:
            t = timed.setdefault((r["batch"], r["kv_len"], r["q"], r["kv"]), {})
            k = (r["splits"], r["page"])
            t[k] = min(r["us"], t.get(k, r["us"]))  # repeated timings: the faster, as the sweep keeps
    rows = []
    for batch in BATCHES:
        for kv_len in KV_LENS:
            for q, kv in PAIRS:
                rows.append(_row(batch, kv_len, q, kv, timed[(batch, kv_len, q, kv)]))
    if where is None:
        where = f"the GPU run logged in {os.path.basename(log_path)}"
        if sha:
            where += f", kernel source sha256 {sha[:16]}"
    _write(out_path, rows, where)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the C table here")
    ap.add_argument("--from-log", default=None, help="rebuild the table from this run's JSON lines (no GPU)")
    ap.add_argument("--where", default=None, help="with --from-log: the device, date and kernel of that run")
    args = ap.parse_args()
    if args.from_log:
        load()
        from_log(args.from_log, args.out, args.where)
        return
    if not torch.cuda.is_available():
        print("tune needs a GPU", file=sys.stderr)
        sys.exit(2)
    tune(args.out)


if __name__ == "__main__":
    main()
