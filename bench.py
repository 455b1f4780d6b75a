#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X: microseconds per call and achieved HBM GB/s.

A "step" is one mla_decode call (stage 1 + stage 2 when S > 1) over one batch
of synthetic inputs already resident in HBM.  Calls are captured into a HIP
graph and replayed, as a serving loop issues decode, so short calls measure
the GPU rather than the Python launch path.  The headline workload is
bs=256, kv_len=8192, bf16 Q over an fp8 e4m3fn paged cache (page 8, shuffled
pages); at one split per request a call is a single stage-1 launch, so the
per-call event time is that kernel's launch duration.  `value` is achieved
GB/s of compulsory traffic (cache incl. scales + Q + page table + indptr +
output) per second; split-K partials are not credited.  The remaining
workloads (the five benchmark shapes) are timed too and listed under
"workloads", each with rotated buffer replicas when its working set would fit
the 256 MB Infinity Cache.

Prints ONE JSON line.  --gpus must be 1: the decode path runs on a single GPU.
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

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

import mla_latent_kv_13_amd as mla  # noqa: E402
from mla_latent_kv_13_amd import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
HEADLINE = "bs256_kv8192_a16w8"
FMT = {"bf16": mla.BF16, "fp8": mla.FP8, "mxfp4": mla.MXFP4}
FLOPS_PER_TOKEN = 2 * 16 * (576 + 512)  # QK^T and P*V multiply-adds, all 16 heads
# MI355X dense MFMA peaks (AMD's published figures without sparsity), TFLOP/s
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
KERNEL_SOURCE = os.path.join(REPO, "mla_latent_kv_13_amd", "csrc", "mla_decode.hip")
TRAFFIC_FILE = os.path.join(REPO, "profiles", "stage1_hbm_traffic_per_workload.txt")


def mfma_tiles(q_fmt: str, kv_fmt: str):
    """MFMA operand type of the QK^T and P*V tiles, and the multiply-adds each
    executes per token and head (the reduction padded to the instruction's
    K; two passes where bf16 Q runs as an exact fp8 hi + lo pair)."""
    if q_fmt == "bf16" and kv_fmt in ("bf16", "fp8"):
        qk, qk_k = "bf16", 576  # an fp8 cache is widened exactly to bf16 for 16x16x32 bf16
    elif kv_fmt == "fp8":
        qk, qk_k = "fp8", 640  # 16x16x128 f8f6f4, five K blocks
    elif q_fmt == "mxfp4":
        qk, qk_k = "fp4", 640
    else:
        qk, qk_k = "fp8", 2 * 640  # e2m1 K x fp8 hi and lo: fp4 x fp8 runs at the fp8 rate
    return {"qk": (qk, qk_k), "pv": ("bf16", 512)}


def mfma_report(q_fmt, kv_fmt, tokens, us):
    """Achieved MFMA rate of each tile against the dense peak of its own
    operand type: algorithmic multiply-adds (576 / 512 per token and head) and
    executed ones (padded, two passes for the hi + lo pair)."""
    out = {}
    for tile, (dt, k_exec) in mfma_tiles(q_fmt, kv_fmt).items():
        k_alg = 576 if tile == "qk" else 512
        alg = 2.0 * 16 * tokens * k_alg / (us * 1e-6) / 1e12
        exe = 2.0 * 16 * tokens * k_exec / (us * 1e-6) / 1e12
        out[tile] = {"dtype": dt, "algorithmic_tflops": round(alg, 2), "executed_tflops": round(exe, 2),
                     "peak_tflops": PEAK_MFMA_TFLOPS[dt], "frac": round(exe / PEAK_MFMA_TFLOPS[dt], 4)}
    return out


def kernel_source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per stage-1 launch of `workload` from the committed FETCH_SIZE /
    WRITE_SIZE summary (each counter scaled by what it reads for the library's
    own streaming-read kernel over a known byte count).

    Reported only while the kernel source is byte-identical to the one the
    counters were taken on (the summary records its sha256); otherwise None.
    """
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha, rows = None, {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            k, sep, v = line.strip().partition(":")
            if not sep:
                continue
            if k.strip() == "kernel_source_sha256" and v.split():
                sha = v.split()[0]
            elif k.startswith("workload "):
                fields = dict(zip(v.split()[::2], v.split()[1::2]))
                rows[k.split()[1]] = fields
    if sha != kernel_source_sha256() or workload not in rows:
        return None
    try:
        r = rows[workload]
        return {"fetch_bytes": int(r["fetch_bytes"]), "write_bytes": int(r["write_bytes"]),
                "traffic_bytes": int(r["traffic_bytes"])}
    except (KeyError, ValueError):
        return None


def compulsory_bytes(w, page_size) -> int:
    """Bytes one call must move at least: cache rows (with mxfp4 scale rows),
    Q (with its scales), the fp32 per-tensor scales of fp8 operands, the page
    table, kv_indptr and the bf16 output."""
    T = w.batch * w.kv_len
    kv = {"bf16": 1152, "fp8": 576, "mxfp4": 288 + 18}[w.kv_fmt] * T
    q = {"bf16": 2 * 576, "fp8": 576, "mxfp4": 288 + 18}[w.q_fmt] * w.batch * 16
    scales = 4 * ((w.kv_fmt == "fp8") + (w.q_fmt == "fp8"))
    pt = 4 * math.ceil(T / page_size)
    return kv + q + scales + pt + 4 * (w.batch + 1) + 2 * w.batch * 16 * 512


def build_inputs(w, device):
    case = synth.workload_case(w, device=device)
    mla.check_tables(case["kv_indptr"], case["page_table"], w.page_size, case["kv"].shape[0])
    B = w.batch
    ops = {"kv_indptr": case["kv_indptr"], "page_table": case["page_table"]}
    if w.kv_fmt == "fp8":
        ops["kv"], ops["kv_scale"] = mla.quantize_fp8(case["kv"])
    elif w.kv_fmt == "mxfp4":
        ops["kv"], ops["kv_scale"] = mla.quantize_mxfp4(case["kv"])
    else:
        ops["kv"], ops["kv_scale"] = case["kv"], None
    if w.q_fmt != "bf16":
        ops["q_bf16"] = case["q"]  # kept for the timing that includes the Q quantiser
    if w.q_fmt == "fp8":
        ops["q_scale_static"] = torch.tensor([w.q_scale], dtype=torch.float32, device=device)
        ops["q"], ops["q_scale"] = mla.quantize_fp8(case["q"], ops["q_scale_static"])
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


def time_calls(call, steps, warmup, warmup_s, per_graph=None):
    """Time `steps` calls (rounded to whole graphs) replayed from a HIP graph.

    The calls are captured once into a graph of `per_graph` consecutive calls
    (call(i) for i in [0, per_graph)), so the GPU sees back-to-back kernels with
    no host launch overhead -- the way a serving loop issues decode.  After a
    warm-up of at least `warmup` calls and `warmup_s` seconds, groups of whole
    graph replays are timed with HIP events on the launch stream: without
    `per_graph`, exactly `steps` calls in up to ten equal groups; with it
    (rotated replicas), ten groups of whole graphs covering at least `steps`.
    Returns (median, min, max, p90) ms per call over the groups, the host wall
    time per call and the number of timed calls."""
    if per_graph is None:
        # exactly `steps` timed calls: up to ten equal groups of one graph each
        steps = max(1, steps)
        ngroups = next(g for g in (10, 5, 4, 3, 2, 1) if steps % g == 0)
        per_graph = steps // ngroups
    else:
        ngroups = 10
    reps_per_group = max(1, math.ceil(steps / (ngroups * per_graph)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager calls first: nothing is lazily initialised inside the capture
        for i in range(per_graph):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            call(i)
    torch.cuda.synchronize()
    n = 0
    t_end = time.perf_counter() + warmup_s
    while n < warmup or time.perf_counter() < t_end:
        graph.replay()
        n += per_graph
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ngroups)]
    t0 = time.perf_counter()
    for r in range(ngroups):
        evs[r][0].record(stream)
        for _ in range(reps_per_group):
            graph.replay()
        evs[r][1].record(stream)
    torch.cuda.synchronize()
    calls = ngroups * reps_per_group * per_graph
    wall = (time.perf_counter() - t0) / calls
    group_ms = sorted(e0.elapsed_time(e1) / (reps_per_group * per_graph) for e0, e1 in evs)
    del graph
    p90 = group_ms[min(len(group_ms) - 1, math.ceil(0.9 * len(group_ms)) - 1)]
    return group_ms[len(group_ms) // 2], group_ms[0], group_ms[-1], p90, wall, calls


def time_workload(w, steps, warmup, device, warmup_s=0.3, extras=True):
    """Time one workload with its stated split count on rotated buffer replicas
    (the headline figure).  With `extras`, also time it on one set of buffers
    (warm, Infinity-Cache resident when small) and with the library heuristic's
    split count when that differs."""
    S_heur = mla.choose_num_splits(w.batch, w.kv_len, FMT[w.kv_fmt], q_dtype=FMT[w.q_fmt])
    S = w.num_splits or S_heur
    ops = build_inputs(w, device)
    ws_bytes = max(mla.workspace_bytes(w.batch, S), mla.workspace_bytes(w.batch, S_heur))
    work = sum(v.numel() * v.element_size() for v in ops.values() if v is not None) + ws_bytes + w.batch * 16 * 1024
    nrep = 1 if work >= (512 << 20) else min(256, max(2, math.ceil((1 << 30) / work)))
    reps = replicate(ops, nrep)
    for r in reps:
        r["out"] = torch.empty((w.batch, 16, 512), dtype=torch.bfloat16, device=device)
        r["ws"] = mla.new_workspace(ws_bytes, device)

    def caller(nsplit, nr):
        def call(i):
            r = reps[i % nr]
            mla.decode(r["q"], r["kv"], r["kv_indptr"], r["page_table"], w.page_size, nsplit, q_scale=r["q_scale"],
                       kv_scale=r["kv_scale"], out=r["out"], workspace=r["ws"])
        return call

    per_graph = nrep if nrep > 1 else None
    ev_ms, mn, mx, p90, wall, calls = time_calls(caller(S, nrep), steps, warmup, warmup_s, per_graph)
    nbytes = compulsory_bytes(w, w.page_size)
    res = {
        "workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q": w.q_fmt, "kv": w.kv_fmt,
        "page_size": w.page_size, "num_splits": S, "replicas": nrep, "timed_calls": calls,
        "us_per_call": round(ev_ms * 1e3, 3), "us_min": round(mn * 1e3, 3),
        "us_p90": round(p90 * 1e3, 3), "us_max": round(mx * 1e3, 3), "wall_us_per_call": round(wall * 1e6, 3),
        "compulsory_bytes": nbytes, "gbs": round(nbytes / (ev_ms * 1e-3) / 1e9, 1),
        "frac_of_peak": round(nbytes / (ev_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "partial_bytes": 2 * mla.workspace_bytes(w.batch, S),
        "tflops": round(FLOPS_PER_TOKEN * w.batch * w.kv_len / (ev_ms * 1e-3) / 1e12, 2),
        "mfma": mfma_report(w.q_fmt, w.kv_fmt, w.batch * w.kv_len, ev_ms * 1e3),
        "traffic": measured_traffic(w.name),
    }
    if extras and w.q_fmt != "bf16":
        # end to end from bf16 Q: the Q quantiser (one launch) plus the decode
        def call_q(i):
            r = reps[i % nrep]
            if w.q_fmt == "fp8":
                mla.quantize_fp8(r["q_bf16"], r["q_scale_static"], out=r["q"])
            else:
                mla.quantize_mxfp4(r["q_bf16"].view(w.batch * 16, 576),
                                   out=(r["q"].view(w.batch * 16, 288), r["q_scale"]))
            mla.decode(r["q"], r["kv"], r["kv_indptr"], r["page_table"], w.page_size, S, q_scale=r["q_scale"],
                       kv_scale=r["kv_scale"], out=r["out"], workspace=r["ws"])
        res["us_with_q_quant"] = round(time_calls(call_q, steps, warmup, 0.05, per_graph)[0] * 1e3, 3)
        if w.q_fmt == "fp8":
            # the same from bf16 Q with the quantiser inside the decode
            # (MLA_Q_BF16_FP8_STATIC): one launch fewer
            def call_qi(i):
                r = reps[i % nrep]
                mla.decode(r["q_bf16"], r["kv"], r["kv_indptr"], r["page_table"], w.page_size, S,
                           kv_scale=r["kv_scale"], out=r["out"], workspace=r["ws"], q_fp8_scale=r["q_scale_static"])
            res["us_q_quant_in_call"] = round(time_calls(call_qi, steps, warmup, 0.05, per_graph)[0] * 1e3, 3)
        else:
            # the same from bf16 Q with the mxfp4 quantiser inside the decode
            # (MLA_Q_BF16_MXFP4)
            def call_qi(i):
                r = reps[i % nrep]
                mla.decode(r["q_bf16"], r["kv"], r["kv_indptr"], r["page_table"], w.page_size, S,
                           kv_scale=r["kv_scale"], out=r["out"], workspace=r["ws"], q_to_mxfp4=True)
            res["us_q_quant_in_call"] = round(time_calls(call_qi, steps, warmup, 0.05, per_graph)[0] * 1e3, 3)
    if extras and nrep > 1:
        warm = time_calls(caller(S, 1), steps, warmup, 0.05, min(nrep, 64))[0]
        res["us_warm_same_buffers"] = round(warm * 1e3, 3)
    if extras and S_heur != S:
        heur = time_calls(caller(S_heur, nrep), steps, warmup, 0.05, per_graph)[0]
        res["heuristic_num_splits"] = S_heur
        res["us_heuristic_splits"] = round(heur * 1e3, 3)
    del reps, ops
    torch.cuda.empty_cache()
    return res, wall


def time_ragged(steps, warmup, device, warmup_s=0.3):
    """A ragged batch: 64 requests with seeded lognormal lengths (sigma 1, mean
    8192 tokens; the total of bs=64 kv_len=8192), bf16 Q over the fp8 cache,
    page 8 shuffled.  Uniform splits (the heuristic's S for the mean length)
    against the host-planned work list."""
    B, mean_len = 64, 8192
    lengths = synth.ragged_lengths(B, mean_len, 1.0, synth.BASE_SEED + 50)
    case = synth.make_case(B, lengths, 8, shuffle=True, seed=synth.BASE_SEED + 51, device=device)
    mla.check_tables(case["kv_indptr"], case["page_table"], 8, case["kv"].shape[0])
    kv, ks = mla.quantize_fp8(case["kv"])
    q, ind, pt = case["q"], case["kv_indptr"], case["page_table"]
    del case
    S = mla.choose_num_splits(B, mean_len, mla.FP8)
    items, req, ns = mla.plan_worklist(ind.cpu())
    items_d, req_d = items.to(device), req.to(device)
    ws = mla.new_workspace(max(mla.workspace_bytes(B, S), mla.worklist_workspace_bytes(ns)), device)
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=device)
    uni = time_calls(lambda i: mla.decode(q, kv, ind, pt, 8, S, kv_scale=ks, out=out, workspace=ws), steps, warmup,
                     warmup_s)[0]
    wl = time_calls(lambda i: mla.decode_worklist(q, kv, ind, pt, 8, items_d, req_d, ns, kv_scale=ks, out=out,
                                                  workspace=ws), steps, warmup, warmup_s)[0]
    T = sum(lengths)
    nbytes = 576 * T + B * 16 * 1152 + 4 * math.ceil(T / 8) + 4 * (B + 1) + B * 16 * 1024
    res = {"workload": "bs64_ragged_lognormal_a16w8", "batch": B, "kv_len_mean": mean_len,
           "kv_len_min": min(lengths), "kv_len_max": max(lengths), "q": "bf16", "kv": "fp8", "page_size": 8,
           "work_items": len(items), "partial_slots": ns,
           "us_per_call": round(wl * 1e3, 3), "gbs": round(nbytes / (wl * 1e-3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (wl * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "uniform_num_splits": S, "us_uniform_splits": round(uni * 1e3, 3), "compulsory_bytes": nbytes}
    del kv, q, ws
    torch.cuda.empty_cache()
    return res


def time_multi_token(steps, warmup, device, warmup_s=0.3):
    """Multi-token decode: bs=64, kv_len=8192, 4 query tokens x 16 heads = 64
    query rows per request over the fp8 cache (page 8, shuffled), bf16 Q.
    Compulsory bytes count the cache once; split count from the heuristic
    with the 4 query groups per request counted as workgroups."""
    B, L, rows = 64, 8192, 64
    case = synth.make_case(B, L, 8, shuffle=True, seed=synth.BASE_SEED + 60, device=device)
    mla.check_tables(case["kv_indptr"], case["page_table"], 8, case["kv"].shape[0])
    kv, ks = mla.quantize_fp8(case["kv"])
    q = synth.normal_bf16((B, rows, 576), seed=synth.BASE_SEED + 61, device=device)
    ind, pt = case["kv_indptr"], case["page_table"]
    del case
    S = mla.choose_num_splits(B * rows // 16, L, mla.FP8)
    ws = mla.new_workspace(mla.workspace_bytes(B, S, rows), device)
    out = torch.empty((B, rows, 512), dtype=torch.bfloat16, device=device)
    ms = time_calls(lambda i: mla.decode(q, kv, ind, pt, 8, S, kv_scale=ks, out=out, workspace=ws), steps, warmup,
                    warmup_s)[0]
    T = B * L
    nbytes = 576 * T + B * rows * 1152 + 4 * (T // 8) + 4 * (B + 1) + B * rows * 1024
    res = {"workload": "bs64_kv8192_q4x16_a16w8", "batch": B, "kv_len": L, "q_rows": rows, "q": "bf16", "kv": "fp8",
           "page_size": 8, "num_splits": S, "us_per_call": round(ms * 1e3, 3),
           "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "tflops": round(2 * rows * T * (576 + 512) / (ms * 1e-3) / 1e12, 2), "compulsory_bytes": nbytes}
    del kv, q, ws
    torch.cuda.empty_cache()
    return res


def time_mixed(steps, warmup, device, warmup_s=0.3):
    """Split cache: bs=256, kv_len=8192, K from the mxfp4 cache and V from the
    fp8 cache of the same rows (page 8, shuffled), mxfp4 Q as the pages'
    mixed routes quantise it.  S = 2 (the mxfp4 benchmark shape's count) and
    the heuristic's S.  Compulsory bytes: both caches' bytes actually read
    (306 B of mxfp4 K and 512 B of fp8 V per token) + Q + page table + out."""
    B, L, P = 256, 8192, 8
    case = synth.make_case(B, L, P, shuffle=True, seed=synth.BASE_SEED + 70, device=device)
    mla.check_tables(case["kv_indptr"], case["page_table"], P, case["kv"].shape[0])
    k, ks = mla.quantize_mxfp4(case["kv"])
    v, vs = mla.quantize_fp8(case["kv"])
    qp, qe = mla.quantize_mxfp4(case["q"].reshape(B * 16, 576))
    q = qp.reshape(B, 16, 288)
    ind, pt = case["kv_indptr"], case["page_table"]
    del case
    torch.cuda.empty_cache()
    S_h = mla.choose_num_splits(B, L, mla.MIXED)
    ws = mla.new_workspace(max(mla.workspace_bytes(B, 2), mla.workspace_bytes(B, S_h)), device)
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=device)
    ms2 = time_calls(lambda i: mla.decode_mixed(q, k, ks, v, vs, ind, pt, P, 2, q_scale=qe, out=out, workspace=ws),
                     steps, warmup, warmup_s)[0]
    msh = ms2 if S_h == 2 else time_calls(
        lambda i: mla.decode_mixed(q, k, ks, v, vs, ind, pt, P, S_h, q_scale=qe, out=out, workspace=ws),
        steps, warmup, warmup_s)[0]
    T = B * L
    nbytes = (306 + 512) * T + B * 16 * 306 + 4 * (T // P) + 4 * (B + 1) + B * 16 * 1024
    res = {"workload": "bs256_kv8192_mxfp4k_fp8v_q4", "batch": B, "kv_len": L, "q": "mxfp4",
           "kv": "mxfp4 K + fp8 V", "page_size": P, "num_splits": 2, "us_per_call": round(ms2 * 1e3, 3),
           "gbs": round(nbytes / (ms2 * 1e-3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "heuristic_num_splits": S_h, "us_heuristic_splits": round(msh * 1e3, 3), "compulsory_bytes": nbytes}
    del k, v, q, ws
    torch.cuda.empty_cache()
    return res


def read_ceiling(nbytes, device, steps=50):
    """Median GB/s of the library's streaming-read probe over a buffer of
    `nbytes` bytes: the practical HBM read ceiling for a read-once kernel."""
    nbytes = (nbytes + 15) // 16 * 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    ms = time_calls(lambda i: mla.stream_read(buf, sink), steps, 10, 0.2)[0]
    del buf
    torch.cuda.empty_cache()
    return round(nbytes / (ms * 1e-3) / 1e9, 1), round(ms * 1e3, 3)


def cpu_oracle_call(w, device="cuda"):
    """One full call of the fp64 oracle for workload `w` on the host cores.

    The inputs are the workload's own (same seeds, generated on the device as
    for the GPU run, then copied to the host) and are quantised outside the
    timed region: mxfp4 by the oracle's quantiser, fp8 by torch's CPU cast of
    clamp(x / scale) with the oracle's scale (the oracle's own exhaustive
    fp8 search gives the same codes, as its tests pin against that cast, but
    would take minutes on a 1.2 G-element cache).  The timed region is one
    oracle decode of every (request, head) pair over the shuffled paged cache,
    with one OpenMP thread per core this process may run on."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    case = synth.workload_case(w, device=device)
    kv_bits = case["kv"].view(torch.int16).cpu().numpy().view(np.uint16)
    q_bits = case["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    ind = case["kv_indptr"].cpu().numpy()
    pt = case["page_table"].cpu().numpy()
    del case
    def fp8_codes(bits, scale):
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
        c = torch.clamp(x / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
        return c.view(torch.uint8).numpy()

    t0 = time.perf_counter()
    args = {}
    if w.kv_fmt == "fp8":
        sc = oracle.fp8_scale_from_amax(oracle.amax_bf16(kv_bits))
        kv = fp8_codes(kv_bits, sc)
        args.update(kv_dtype="fp8", kv_scale=sc)
    elif w.kv_fmt == "mxfp4":
        kv, e8 = oracle.quant_mxfp4(kv_bits)
        args.update(kv_dtype="mxfp4", kv_e8m0=e8)
    else:
        kv = kv_bits
    del kv_bits
    if w.q_fmt == "fp8":
        qs = float(np.float32(w.q_scale))
        q = fp8_codes(q_bits, qs)
        args.update(q_dtype="fp8", q_scale=qs)
    elif w.q_fmt == "mxfp4":
        qp, qe = oracle.quant_mxfp4(q_bits.reshape(w.batch * 16, 576))
        q = qp.reshape(w.batch, 16, 288)
        args.update(q_dtype="mxfp4", q_e8m0=qe)
    else:
        q = q_bits
    t_quant = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.decode(q, kv, ind, pt, w.page_size, nthreads=cores, **args)
    t = time.perf_counter() - t0
    return {"s_per_call": round(t, 3), "cores": cores, "quantise_s_untimed": round(t_quant, 2),
            "sample": f"one full call: {w.batch} requests x 16 heads x {w.kv_len} tokens"}


def cpu_baseline(w, oracle_call):
    """The headline's CPU baseline object from its full oracle call."""
    nbytes = compulsory_bytes(w, w.page_size)
    t = oracle_call["s_per_call"]
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": oracle_call["cores"], "kind": "oracle",
            "sample": f"{oracle_call['sample']} ({w.name}), fp64 C oracle with OpenMP, measured (no extrapolation); "
                      f"its own quantisation of the inputs ({oracle_call['quantise_s_untimed']} s) is untimed",
            "us_per_call": round(t * 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(synth.WORKLOADS))
    ap.add_argument("--only-headline", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-only", choices=["ragged", "multi_token", "mixed"], default=None,
                    help="time only this extra workload (for profiling) and print its JSON")
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="minimum warm-up time per workload (0 for short profiled runs)")
    ap.add_argument("--calib-bytes", type=int, default=0,
                    help="instead of decoding, read this many bytes with the library's streaming-read kernel "
                         "and write as many with a fill kernel (the known-size references that scale the "
                         "FETCH_SIZE and WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              "(requests would shard across GPUs by batch, with no communication).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    mla.load()
    device = "cuda"
    if args.calib_bytes:
        n = args.calib_bytes // 16 * 16
        src = torch.ones(n // 4, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        sink = torch.zeros(1, dtype=torch.int32, device=device)
        for _ in range(args.warmup + args.steps):
            mla.stream_read(src, sink)  # reads n bytes, writes none
            dst.fill_(2.0)              # writes n bytes, reads none
        torch.cuda.synchronize()
        print(json.dumps({"metric": "counter calibration", "stream_read_bytes": n, "fill_bytes": n,
                          "launches_each": args.warmup + args.steps}))
        return
    if args.extra_only:
        fn = {"ragged": time_ragged, "multi_token": time_multi_token, "mixed": time_mixed}[args.extra_only]
        print(json.dumps(fn(args.steps, args.warmup, device, args.warmup_seconds)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    print(f"[bench] headline {w.name}", file=sys.stderr, flush=True)
    head, wall = time_workload(w, args.steps, args.warmup, device, args.warmup_seconds, extras=False)
    print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
    ceil_gbs, ceil_us = read_ceiling(head["compulsory_bytes"], device)
    others = []
    if not args.only_headline:
        for name, ow in synth.WORKLOADS.items():
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            others.append(time_workload(ow, max(10, args.steps // 2), args.warmup, device, args.warmup_seconds)[0])
        print("[bench] ragged batch (work list)", file=sys.stderr, flush=True)
        others.append(time_ragged(max(10, args.steps // 2), args.warmup, device, args.warmup_seconds))
        print("[bench] multi-token decode (64 query rows)", file=sys.stderr, flush=True)
        others.append(time_multi_token(max(10, args.steps // 2), args.warmup, device, args.warmup_seconds))
        print("[bench] split cache (mxfp4 K, fp8 V)", file=sys.stderr, flush=True)
        others.append(time_mixed(max(10, args.steps // 2), args.warmup, device, args.warmup_seconds))
    cpu = None
    if not args.no_cpu_baseline:
        # after every GPU timing, so host work cannot disturb them: one full
        # oracle call per synthetic workload
        for entry in [head] + others:
            ow = synth.WORKLOADS.get(entry["workload"])
            if ow is None:
                continue
            print(f"[bench] cpu oracle, full call: {ow.name}", file=sys.stderr, flush=True)
            entry["cpu_oracle"] = cpu_oracle_call(ow)
            entry["gpu_speedup_vs_cpu_oracle"] = round(entry["cpu_oracle"]["s_per_call"] * 1e6 / entry["us_per_call"])
        cpu = cpu_baseline(w, head["cpu_oracle"])
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
        "launch": "HIP graph replay of back-to-back mla_decode calls",
        "config": {"workload": w.name, "batch": w.batch, "kv_len": w.kv_len, "q": w.q_fmt, "kv": w.kv_fmt,
                   "page_size": w.page_size, "num_splits": head["num_splits"], "parallelism": "single GPU"},
        "roofline": {"kernel": "stage1_kernel" + ("" if head["num_splits"] == 1 else " + stage2_kernel"),
                     "bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["frac_of_peak"],
                     "traffic": (head["traffic"] or {}).get("traffic_bytes"),
                     "traffic_unit": "bytes per launch",
                     "read_ceiling": {"achieved": ceil_gbs, "us": ceil_us, "bytes": head["compulsory_bytes"],
                                      "kernel": "stream_read_kernel (16-B non-temporal loads, read once)"},
                     "frac_of_read_ceiling": round(head["gbs"] / ceil_gbs, 4)},
        "mfma": head["mfma"],
        "cpu_baseline": cpu,
        "workloads": [head] + others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
