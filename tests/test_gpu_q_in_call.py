"""GPU: bf16 Q quantised inside the decode (q_dtype MLA_Q_BF16_FP8_STATIC over
the fp8 cache, MLA_Q_BF16_MXFP4 over the mxfp4 cache).

The stage-1 workgroups quantise bf16 Q themselves, code for code as
mla_quantize_fp8 (static scale) or mla_quantize_mxfp4 does.  So the decode's
output must equal, bit for bit, the output of that quantiser followed by the
fp8-Q or mxfp4-Q decode: any code or block scale that differed would change
its logits.  The Q tensors hold every non-NaN bf16 bit pattern (zeros of both
signs, subnormals, values far beyond the fp8 clamp, infinities); the fp8
scales include ones outside the reciprocal-division range, which take the
plain division.  The oracle checks run the in-call paths against the fp64
oracle on the oracle's own codes of Q, like the other parity tests.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_13_amd as mla
from mla_latent_kv_13_amd import synth

from test_gpu_parity import DEV, RANDOM_SCALE, SHAPES, bits, check_close, gpu_decode, oracle_decode, prepare

pytestmark = pytest.mark.gpu


def all_finite_bf16(shape, seed):
    """A bf16 tensor holding every non-NaN bf16 bit pattern at least once,
    in a seeded order (tiled when the tensor is larger)."""
    pats = np.arange(65536, dtype=np.uint32)
    finite = ((pats >> 7) & 0xFF) != 0xFF
    inf = (pats & 0x7FFF) == 0x7F80
    pats = pats[finite | inf].astype(np.uint16)
    n = int(np.prod(shape))
    assert n >= pats.size
    rng = np.random.default_rng(seed)
    full = np.concatenate([pats, rng.choice(pats, n - pats.size)])
    rng.shuffle(full)
    return torch.from_numpy(full.view(np.int16).copy()).view(torch.bfloat16).reshape(shape)


def fp8_cache(case):
    kv, ks = mla.quantize_fp8(case["kv"].to(DEV))
    return kv, ks, case["kv_indptr"].to(DEV), case["page_table"].to(DEV)


def mxfp4_cache(case):
    kv, ks = mla.quantize_mxfp4(case["kv"].to(DEV))
    return kv, ks, case["kv_indptr"].to(DEV), case["page_table"].to(DEV)


def both_paths_mx(q, kv, ks, ind, pt, P, S):
    """(in-call mxfp4 quantisation, separate quantiser + mxfp4-Q decode) outputs."""
    B, R = q.shape[0], q.shape[1]
    q4, s4 = mla.quantize_mxfp4(q.reshape(B * R, 576))
    fused = mla.decode(q, kv, ind, pt, P, S, kv_scale=ks, q_to_mxfp4=True)
    two = mla.decode(q4.reshape(B, R, 288), kv, ind, pt, P, S, q_scale=s4, kv_scale=ks)
    torch.cuda.synchronize()
    return fused, two


def both_paths(q, kv, ks, ind, pt, P, S, scale):
    """(in-call quantisation, separate quantiser + fp8-Q decode) outputs."""
    q8, sc = mla.quantize_fp8(q, scale)
    fused = mla.decode(q, kv, ind, pt, P, S, kv_scale=ks, q_fp8_scale=sc)
    two = mla.decode(q8, kv, ind, pt, P, S, q_scale=sc, kv_scale=ks)
    torch.cuda.synchronize()
    return fused, two


def assert_same_bits(a, b, what):
    ba, bb = bits(a), bits(b)
    diff = int((ba != bb).sum())
    assert diff == 0, f"{what}: {diff} output elements differ"


@pytest.mark.parametrize("scale", [6.0 / 448.0, 0.37, 2.0 ** -70, 2.0 ** 70])
@pytest.mark.parametrize("S", [1, 3])
def test_in_call_q8_every_bf16_pattern(scale, S):
    lengths = [100, 37, 300, 1, 64, 129, 0, 250]
    print(f"[q8-in-call] every bf16 pattern, scale={scale} S={S}", flush=True)
    case = synth.make_case(len(lengths), lengths, 8, shuffle=True, seed=900 + S)
    q = all_finite_bf16((len(lengths), 16, 576), seed=901).to(DEV)
    kv, ks, ind, pt = fp8_cache(case)
    fused, two = both_paths(q, kv, ks, ind, pt, 8, S, scale)
    assert_same_bits(fused, two, f"scale {scale} S {S}")
    assert not fused[6].any()  # the empty request


@pytest.mark.parametrize("batch,length,rows,S", [
    (300, 40, 16, 1),    # 300 workgroups: the two-wave layout
    (300, 40, 16, 2),
    (8, 700, 64, 2),     # four query groups per request
    (3, 2048, 16, 32),
])
def test_in_call_q8_layouts(batch, length, rows, S):
    print(f"[q8-in-call] batch={batch} L={length} rows={rows} S={S}", flush=True)
    case = synth.make_case(batch, length, 8, shuffle=True, seed=910 + S)
    q = synth.normal_bf16((batch, rows, 576), seed=911, device=DEV, std=2.0)
    kv, ks, ind, pt = fp8_cache(case)
    fused, two = both_paths(q, kv, ks, ind, pt, 8, S, 6.0 / 448.0)
    assert_same_bits(fused, two, f"batch {batch} rows {rows} S {S}")


@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_in_call_q8_matches_oracle(orc, shape):
    lengths, P, S, per_req = SHAPES[shape]
    print(f"[q8-in-call] oracle lengths={lengths} P={P} S={S} per_request={per_req}", flush=True)
    case = synth.make_case(len(lengths), lengths, P, shuffle=True, seed=400 + shape, per_request_pages=per_req,
                           extra_pages=2)
    g, o = prepare(case, "fp8", "fp8", orc)  # asserts the quantisers' codes agree
    out = mla.decode(case["q"].to(DEV), g["kv"], g["kv_indptr"], g["page_table"], case["page_size"], S,
                     kv_scale=g["kv_scale"], page_indptr=g["page_indptr"], q_fp8_scale=g["q_scale"])
    torch.cuda.synchronize()
    ref, _ = oracle_decode(case, o, orc)
    check_close(out, ref, what=f"in-call fp8 Q, shape {shape}")
    assert_same_bits(out, gpu_decode(case, g, S), f"shape {shape}")


@pytest.mark.parametrize("name", ["bs4_kv8192_a8w8", "bs256_kv8192_a8w8"])
def test_in_call_q8_full_size(name):
    w = synth.WORKLOADS[name]
    S = w.num_splits or mla.choose_num_splits(w.batch, w.kv_len, mla.FP8, q_dtype=mla.FP8)
    print(f"[q8-in-call] full size {name} S={S}", flush=True)
    case = synth.workload_case(w)
    kv, ks, ind, pt = fp8_cache(case)
    fused, two = both_paths(case["q"].to(DEV), kv, ks, ind, pt, w.page_size, S, w.q_scale)
    assert_same_bits(fused, two, name)


# ----------------------------------------------------------- mxfp4 Q
@pytest.mark.parametrize("S", [1, 2])
def test_in_call_mxfp4_every_bf16_pattern(S):
    lengths = [100, 37, 300, 1, 64, 129, 0, 250]
    print(f"[q4-in-call] every bf16 pattern, S={S}", flush=True)
    case = synth.make_case(len(lengths), lengths, 8, shuffle=True, seed=920 + S)
    q = all_finite_bf16((len(lengths), 16, 576), seed=921).to(DEV)
    kv, ks, ind, pt = mxfp4_cache(case)
    fused, two = both_paths_mx(q, kv, ks, ind, pt, 8, S)
    assert_same_bits(fused, two, f"mxfp4 S {S}")
    assert not fused[6].any()


@pytest.mark.parametrize("batch,length,rows,S", [
    (300, 40, 16, 1),    # 300 workgroups: the two-wave layout
    (300, 40, 16, 2),
    (8, 700, 64, 2),     # four query groups per request
    (3, 2048, 16, 32),
])
def test_in_call_mxfp4_layouts(batch, length, rows, S):
    print(f"[q4-in-call] batch={batch} L={length} rows={rows} S={S}", flush=True)
    case = synth.make_case(batch, length, 8, shuffle=True, seed=930 + S)
    q = synth.normal_bf16((batch, rows, 576), seed=931, device=DEV, std=2.0)
    kv, ks, ind, pt = mxfp4_cache(case)
    fused, two = both_paths_mx(q, kv, ks, ind, pt, 8, S)
    assert_same_bits(fused, two, f"mxfp4 batch {batch} rows {rows} S {S}")


@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_in_call_mxfp4_matches_oracle(orc, shape):
    lengths, P, S, per_req = SHAPES[shape]
    print(f"[q4-in-call] oracle lengths={lengths} P={P} S={S} per_request={per_req}", flush=True)
    case = synth.make_case(len(lengths), lengths, P, shuffle=True, seed=400 + shape, per_request_pages=per_req,
                           extra_pages=2)
    g, o = prepare(case, "mxfp4", "mxfp4", orc)  # asserts the quantisers' codes agree
    out = mla.decode(case["q"].to(DEV), g["kv"], g["kv_indptr"], g["page_table"], case["page_size"], S,
                     kv_scale=g["kv_scale"], page_indptr=g["page_indptr"], q_to_mxfp4=True)
    torch.cuda.synchronize()
    ref, _ = oracle_decode(case, o, orc)
    check_close(out, ref, what=f"in-call mxfp4 Q, shape {shape}")
    assert_same_bits(out, gpu_decode(case, g, S), f"mxfp4 shape {shape}")


@pytest.mark.parametrize("S", [2, 1])
def test_in_call_mxfp4_full_size(S):
    w = synth.WORKLOADS["bs256_kv8192_mxfp4_q4"]
    print(f"[q4-in-call] full size {w.name} S={S}", flush=True)
    case = synth.workload_case(w)
    kv, ks, ind, pt = mxfp4_cache(case)
    fused, two = both_paths_mx(case["q"].to(DEV), kv, ks, ind, pt, w.page_size, S)
    assert_same_bits(fused, two, f"{w.name} S {S}")


# ------------------------------------------------------ random layouts
@pytest.mark.parametrize("i", range(16 * RANDOM_SCALE))
def test_in_call_random_configurations(i):
    """Seeded random layouts (ragged lengths with empty and one-token
    requests, any page size, both paging conventions, 16-128 query rows,
    S up to 64) for both in-call modes, bit for bit against the separate
    quantiser followed by the decode."""
    rng = np.random.default_rng(11000 + i)
    batch = int(rng.integers(1, 7))
    lengths = [0 if u < 0.12 else 1 if u < 0.24 else int(rng.integers(2, 2500)) for u in rng.random(batch)]
    P = int(rng.choice([1, 2, 3, 5, 8, 16, 32]))
    per_req = bool(rng.random() < 0.5)
    S = int(rng.choice([1, 2, 3, 4, 5, 8, 13, 16, 32, 64]))
    rows = int(rng.choice([16, 16, 32, 64, 128]))
    mode = "fp8" if i % 2 == 0 else "mxfp4"
    print(f"[in-call random {i}] {mode} rows={rows} lengths={lengths} P={P} S={S} per_request={per_req}",
          flush=True)
    case = synth.make_case(batch, lengths, P, shuffle=True, seed=11100 + i, per_request_pages=per_req,
                           extra_pages=1)
    q = synth.normal_bf16((batch, rows, 576), seed=11200 + i, device=DEV, std=float(rng.choice([0.1, 1.0, 30.0])))
    pind = None if case["page_indptr"] is None else case["page_indptr"].to(DEV)
    if mode == "fp8":
        kv, ks, ind, pt = fp8_cache(case)
        q8, sc = mla.quantize_fp8(q, 6.0 / 448.0)
        fused = mla.decode(q, kv, ind, pt, P, S, kv_scale=ks, q_fp8_scale=sc, page_indptr=pind)
        two = mla.decode(q8, kv, ind, pt, P, S, q_scale=sc, kv_scale=ks, page_indptr=pind)
    else:
        kv, ks, ind, pt = mxfp4_cache(case)
        q4, s4 = mla.quantize_mxfp4(q.reshape(batch * rows, 576))
        fused = mla.decode(q, kv, ind, pt, P, S, kv_scale=ks, q_to_mxfp4=True, page_indptr=pind)
        two = mla.decode(q4.reshape(batch, rows, 288), kv, ind, pt, P, S, q_scale=s4, kv_scale=ks, page_indptr=pind)
    torch.cuda.synchronize()
    assert_same_bits(fused, two, f"in-call random {i}")
