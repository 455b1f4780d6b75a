"""The allocation-free entry point (mla_decode_noalloc, static per-GPU scratch)
against the existing entry point (mla_decode with a caller workspace) on the
same inputs and split count -- same kernels, so the outputs must be identical
-- and against the oracle, on two calls in a row, the second smaller."""
import numpy as np
import pytest
import torch

import mla_latent_kv_13_amd as mla
from mla_latent_kv_13_amd import synth

from test_gpu_parity import DEV, check_close, gpu_decode, oracle_decode, prepare

pytestmark = pytest.mark.gpu


def noalloc(case, g, S):
    B = case["kv_indptr"].numel() - 1
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=DEV)
    mla.decode_noalloc(g["q"], g["kv"], g["kv_indptr"], g["page_table"], case["page_size"], S, out,
                       q_scale=g["q_scale"], kv_scale=g["kv_scale"], page_indptr=g["page_indptr"])
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_decode_twice_second_smaller(orc):
    # first call: 6 requests (one empty), 7 splits, fp8 cache with bf16 Q
    big = synth.make_case(6, [3000, 1, 0, 777, 2049, 65], 8, shuffle=True, seed=900)
    print("[noalloc] call 1: batch 6, S=7, bf16/fp8", flush=True)
    g1, o1 = prepare(big, "bf16", "fp8", orc)
    a1 = noalloc(big, g1, 7)
    r1 = gpu_decode(big, g1, 7)
    assert torch.equal(a1, r1)
    ref1, _ = oracle_decode(big, o1, orc)
    check_close(a1, ref1, what="noalloc call 1")
    assert not a1[2].any()
    # second call, smaller: 2 requests, 3 splits, mxfp4 Q over the mxfp4
    # cache, per-request page tables -- the scratch still holds call 1's
    # partials, which must not leak into this result
    small = synth.make_case(2, [513, 96], 3, shuffle=True, seed=901, per_request_pages=True)
    print("[noalloc] call 2: batch 2, S=3, mxfp4/mxfp4", flush=True)
    g2, o2 = prepare(small, "mxfp4", "mxfp4", orc)
    a2 = noalloc(small, g2, 3)
    r2 = gpu_decode(small, g2, 3)
    assert torch.equal(a2, r2)
    ref2, _ = oracle_decode(small, o2, orc)
    check_close(a2, ref2, what="noalloc call 2")


def test_noalloc_one_split_and_limits(orc):
    case = synth.make_case(3, [100, 1, 300], 4, shuffle=True, seed=902)
    g, o = prepare(case, "fp8", "fp8", orc)
    a = noalloc(case, g, 1)  # S = 1 writes out directly and needs no scratch
    assert torch.equal(a, gpu_decode(case, g, 1))
    ref, _ = oracle_decode(case, o, orc)
    check_close(a, ref, what="noalloc S=1")
    # more partial bytes than the scratch holds: rejected on the host, nothing launched
    assert mla.workspace_bytes(256, 4) > mla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((256, 16, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((8, 576), dtype=torch.bfloat16, device=DEV)
    ind = torch.zeros(257, dtype=torch.int32, device=DEV)
    pt = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty((256, 16, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.StatusError) as e:
        mla.decode_noalloc(q, kv, ind, pt, 8, 4, out)
    assert e.value.status == -5


def test_noalloc_graph_replay(orc):
    """Captured into a HIP graph (a caller that cannot allocate inside the
    capture): every replay gives the eager result."""
    case = synth.make_case(3, [700, 45, 1200], 8, shuffle=True, seed=903)
    g, o = prepare(case, "bf16", "fp8", orc)
    eager = noalloc(case, g, 4).clone()
    out = torch.empty_like(eager)

    def call():
        mla.decode_noalloc(g["q"], g["kv"], g["kv_indptr"], g["page_table"], case["page_size"], 4, out,
                           kv_scale=g["kv_scale"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        noalloc(case, g, 2)  # eager work on the same scratch between replays
