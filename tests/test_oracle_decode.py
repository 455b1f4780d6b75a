"""Pins for the oracle's MLA decode against things other than itself.

* Library special case: torch's scaled_dot_product_attention in float64 on the
  CPU (default scale 1/sqrt(576) for a 576-wide head, Ev = 512), with every
  input dequantised by torch / the closed-form codecs rather than by the oracle.
* Closed forms: one token gives exactly V; two tokens give the sigmoid mix.
* Invariants: constant logits give the mean of V; a rope component common to
  all keys changes nothing; (q_scale/2, kv_scale*2) doubles the output
  exactly; permuting physical pages (with the table) changes nothing; a key
  planted as c*q dominates (one-hot probe of the gather).
* Split-wise partial/merge form agrees with the unsplit softmax to 1e-12.
* Split cache (keys from an mxfp4 cache, values from an fp8 cache of the same
  rows): torch SDPA with separately dequantised K and V, one token gives that
  token's fp8 value row exactly, and identical keys give the mean of the fp8
  value rows.
* Planted mistakes (patched copies of oracle.c, tests/oracle_mutants.py) each
  fail at least one pin.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_13_amd import synth

from oracle_mutants import MUTANTS, mutant_source

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def bits(x):
    return x.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def rows_f64(case, fmt, orc):
    """Cache rows in the oracle's input format plus an independent fp64 dequantisation."""
    kv = case["kv"]
    if fmt == "bf16":
        return bits(kv), {}, kv.to(torch.float64).numpy()
    if fmt == "fp8":
        codes, sc = orc.quant_fp8(bits(kv))
        deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * sc
        return codes, {"kv_scale": sc}, deq
    packed, e8 = orc.quant_mxfp4(bits(kv))
    nib = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], 576)
    deq = E2M1[nib] * np.repeat(np.ldexp(1.0, e8.astype(np.int64) - 127), 32, axis=1)
    return packed, {"kv_e8m0": e8}, deq


def logical_rows(case, b, L):
    P = case["page_size"]
    pt = case["page_table"].numpy()
    pind = case["page_indptr"]
    base = 0 if pind is not None else int(case["kv_indptr"][b])
    first = int(pind[b]) if pind is not None else 0
    return np.array([pt[first + (base + t) // P] * P + (base + t) % P for t in range(L)], dtype=np.int64)


def sdpa_ref(case, deq_kv, q64):
    """torch SDPA (float64, CPU) per request; returns [B,16,512]."""
    B = case["kv_indptr"].numel() - 1
    out = np.zeros((B, 16, 512))
    for b in range(B):
        L = case["lengths"][b]
        if L == 0:
            continue
        k = torch.from_numpy(deq_kv[logical_rows(case, b, L)])
        qq = torch.from_numpy(q64[b]).reshape(1, 16, 1, 576)
        kk = k.reshape(1, 1, L, 576).expand(1, 16, L, 576)
        vv = k[:, :512].reshape(1, 1, L, 512).expand(1, 16, L, 512)
        out[b] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).reshape(16, 512).numpy()
    return out


def run(orc, case, kvdata, extra, **kw):
    return orc.decode(bits(case["q"]), kvdata, case["kv_indptr"].numpy(), case["page_table"].numpy(),
                      case["page_size"], kv_dtype=kw.pop("kv_dtype", "bf16"),
                      page_indptr=None if case["page_indptr"] is None else case["page_indptr"].numpy(),
                      **extra, **kw)


# ------------------------------------------------------------------ pins
def pin_sdpa(orc, fmt, per_request=False, seed=11):
    case = synth.make_case(3, [17, 5, 9], 4, shuffle=True, seed=seed, per_request_pages=per_request, extra_pages=2)
    kvd, extra, deq = rows_f64(case, fmt, orc)
    out, _ = run(orc, case, kvd, extra, kv_dtype=fmt)
    ref = sdpa_ref(case, deq, case["q"].to(torch.float64).numpy())
    return np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def pin_one_token(orc):
    case = synth.make_case(2, [1, 1], 1, shuffle=True, seed=12)
    out, _ = run(orc, case, bits(case["kv"]), {})
    kv = case["kv"].to(torch.float64).numpy()
    ok = True
    for b in range(2):
        row = logical_rows(case, b, 1)[0]
        ok &= np.array_equal(out[b], np.broadcast_to(kv[row, :512], (16, 512)))
    return ok


def pin_two_tokens(orc):
    case = synth.make_case(1, [2], 2, shuffle=False, seed=13)
    out, _ = run(orc, case, bits(case["kv"]), {})
    q = case["q"].to(torch.float64).numpy()[0]
    k = case["kv"].to(torch.float64).numpy()[:2]
    s = q @ k.T / 24.0
    sig = 1.0 / (1.0 + np.exp(-(s[:, 1] - s[:, 0])))
    ref = sig[:, None] * k[1, :512] + (1 - sig[:, None]) * k[0, :512]
    return np.allclose(out[0], ref, rtol=1e-12, atol=1e-14)


def pin_constant_logits(orc):
    # Q = 0 makes every logit 0: uniform weights, output = mean of V
    case = synth.make_case(2, [7, 12], 3, shuffle=True, seed=14)
    case["q"] = torch.zeros_like(case["q"])
    out, _ = run(orc, case, bits(case["kv"]), {})
    kv = case["kv"].to(torch.float64).numpy()
    ok = True
    for b in range(2):
        ref = kv[logical_rows(case, b, case["lengths"][b]), :512].mean(axis=0)
        ok &= np.allclose(out[b], np.broadcast_to(ref, (16, 512)), rtol=1e-13, atol=1e-15)
    return ok


def pin_split_agreement(orc):
    case = synth.make_case(3, [33, 7, 64], 8, shuffle=True, seed=15)
    ref, _ = run(orc, case, bits(case["kv"]), {})
    ok = True
    for S in (1, 2, 3, 7, 64):
        out, _ = run(orc, case, bits(case["kv"]), {}, num_splits=S)
        ok &= np.allclose(out, ref, rtol=1e-12, atol=1e-14)
    return ok


def pin_page_permutation(orc):
    # identity layout vs the same logical rows scattered into shuffled pages
    P = 4
    case = synth.make_case(2, [13, 22], P, shuffle=False, seed=16, extra_pages=3)
    out_id, _ = run(orc, case, bits(case["kv"]), {})
    npg = case["kv"].shape[0] // P
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(99))
    phys = torch.empty_like(case["kv"])
    for j in range(npg):
        phys[perm[j] * P:(perm[j] + 1) * P] = case["kv"][j * P:(j + 1) * P]
    case2 = dict(case, kv=phys, page_table=perm[: case["page_table"].numel()].to(torch.int32))
    out_sh, _ = run(orc, case2, bits(phys), {})
    return np.array_equal(out_id, out_sh)


def pin_one_hot_probe(orc):
    # key t* = 8*q_h for head 0 (16-way shared key, so plant per request and check head 0)
    P = 2
    case = synth.make_case(2, [11, 9], P, shuffle=True, seed=17)
    kv = case["kv"].clone()
    ok = True
    for b, tstar in ((0, 7), (1, 2)):
        row = logical_rows(case, b, case["lengths"][b])[tstar]
        kv[row] = (case["q"][b, 0].to(torch.float32) * 8).to(torch.bfloat16)
    case = dict(case, kv=kv)
    out, _ = run(orc, case, bits(kv), {})
    kv64 = kv.to(torch.float64).numpy()
    for b, tstar in ((0, 7), (1, 2)):
        row = logical_rows(case, b, case["lengths"][b])[tstar]
        ok &= np.allclose(out[b, 0], kv64[row, :512], rtol=0, atol=1e-6 * np.abs(kv64[row]).max())
    return ok


def pin_rope_shift(orc):
    case = synth.make_case(2, [10, 6], 2, shuffle=True, seed=18)
    ref, _ = run(orc, case, bits(case["kv"]), {})
    kv = case["kv"].clone()
    kv[:, 512:] = kv[0:1, 512:]  # all keys share one rope vector -> logits shift by a per-head constant
    base, _ = run(orc, dict(case, kv=kv), bits(kv), {})
    kv2 = kv.clone()
    kv2[:, 512:] = torch.ones(64, dtype=torch.bfloat16) * 2.0  # a different common rope vector
    shifted, _ = run(orc, dict(case, kv=kv2), bits(kv2), {})
    return np.allclose(base, shifted, rtol=1e-12, atol=1e-14) and not np.allclose(ref, base, atol=1e-6)


def pin_scale_fold(orc):
    case = synth.make_case(2, [9, 14], 2, shuffle=True, seed=19)
    codes, sc = orc.quant_fp8(bits(case["kv"]))
    qcodes, qs = orc.quant_fp8(bits(case["q"]), 6.0 / 448.0)
    common = dict(q_dtype="fp8", kv_dtype="fp8")
    a, _ = orc.decode(qcodes, codes, case["kv_indptr"].numpy(), case["page_table"].numpy(), 2,
                      q_scale=qs, kv_scale=sc, **common)
    b, _ = orc.decode(qcodes, codes, case["kv_indptr"].numpy(), case["page_table"].numpy(), 2,
                      q_scale=qs / 2, kv_scale=sc * 2, **common)
    return np.array_equal(b, 2 * a)


def pin_mxfp4_sdpa(orc):
    return pin_sdpa(orc, "mxfp4", seed=20)


def pin_sdpa_multi_row(orc, fmt="fp8", rows=64):
    """rows query rows per request (q_seq_len 4 x 16 heads), each attending to
    the request's whole cache: torch SDPA with the rows as heads."""
    case = synth.make_case(3, [17, 5, 9], 4, shuffle=True, seed=25, extra_pages=2)
    q = synth.normal_bf16((3, rows, 576), seed=26)
    kvd, extra, deq = rows_f64(case, fmt, orc)
    out, _ = orc.decode(bits(q), kvd, case["kv_indptr"].numpy(), case["page_table"].numpy(), case["page_size"],
                        kv_dtype=fmt, **extra)
    ref = np.zeros((3, rows, 512))
    for b in range(3):
        L = case["lengths"][b]
        k = torch.from_numpy(deq[logical_rows(case, b, L)])
        qq = q[b].to(torch.float64).reshape(1, rows, 1, 576)
        kk = k.reshape(1, 1, L, 576).expand(1, rows, L, 576)
        vv = k[:, :512].reshape(1, 1, L, 512).expand(1, rows, L, 512)
        ref[b] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).reshape(rows, 512).numpy()
    return out.shape == (3, rows, 512) and np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def mixed_case(orc, lengths, P, seed, shuffle=True):
    """One logical cache in two physical forms on the same rows: mxfp4 keys
    and fp8 values, with independent fp64 dequantisations of both."""
    case = synth.make_case(len(lengths), lengths, P, shuffle=shuffle, seed=seed, extra_pages=2)
    packed, kdeq_extra, kdeq = rows_f64(case, "mxfp4", orc)
    codes, vextra, vdeq = rows_f64(case, "fp8", orc)
    return case, packed, kdeq_extra["kv_e8m0"], kdeq, codes, vextra["kv_scale"], vdeq


def run_mixed(orc, case, packed, e8, codes, vs, **kw):
    return run(orc, case, packed, {"kv_e8m0": e8}, kv_dtype="mxfp4", v=codes, v_dtype="fp8", v_scale=vs, **kw)


def pin_sdpa_mixed(orc):
    case, packed, e8, kdeq, codes, vs, vdeq = mixed_case(orc, [17, 5, 9], 4, seed=29)
    out, _ = run_mixed(orc, case, packed, e8, codes, vs)
    q64 = case["q"].to(torch.float64).numpy()
    ref = np.zeros((3, 16, 512))
    for b in range(3):
        L = case["lengths"][b]
        rws = logical_rows(case, b, L)
        kk = torch.from_numpy(kdeq[rws]).reshape(1, 1, L, 576).expand(1, 16, L, 576)
        vv = torch.from_numpy(vdeq[rws, :512]).reshape(1, 1, L, 512).expand(1, 16, L, 512)
        qq = torch.from_numpy(q64[b]).reshape(1, 16, 1, 576)
        ref[b] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).reshape(16, 512).numpy()
    return np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def pin_one_token_mixed(orc):
    case, packed, e8, _, codes, vs, vdeq = mixed_case(orc, [1, 1], 1, seed=30)
    out, _ = run_mixed(orc, case, packed, e8, codes, vs)
    ok = True
    for b in range(2):
        row = logical_rows(case, b, 1)[0]
        ok &= np.array_equal(out[b], np.broadcast_to(vdeq[row, :512], (16, 512)))
    return ok


def pin_constant_keys_mixed(orc):
    # every key row the same: uniform weights whatever Q is, output = mean of
    # the fp8 value rows
    case, packed, e8, _, codes, vs, vdeq = mixed_case(orc, [7, 12], 3, seed=31)
    packed = np.broadcast_to(packed[0], packed.shape).copy()
    e8 = np.broadcast_to(e8[0], e8.shape).copy()
    out, _ = run_mixed(orc, case, packed, e8, codes, vs)
    ok = True
    for b in range(2):
        ref = vdeq[logical_rows(case, b, case["lengths"][b]), :512].mean(axis=0)
        ok &= np.allclose(out[b], np.broadcast_to(ref, (16, 512)), rtol=1e-13, atol=1e-15)
    return ok


PINS = {
    "sdpa_bf16": lambda o: pin_sdpa(o, "bf16"),
    "sdpa_bf16_per_request_pages": lambda o: pin_sdpa(o, "bf16", per_request=True),
    "sdpa_fp8": lambda o: pin_sdpa(o, "fp8"),
    "sdpa_mxfp4": pin_mxfp4_sdpa,
    "sdpa_multi_row": pin_sdpa_multi_row,
    "one_token": pin_one_token,
    "two_tokens": pin_two_tokens,
    "constant_logits": pin_constant_logits,
    "split_agreement": pin_split_agreement,
    "page_permutation": pin_page_permutation,
    "one_hot_probe": pin_one_hot_probe,
    "rope_shift": pin_rope_shift,
    "scale_fold": pin_scale_fold,
    "sdpa_mixed": pin_sdpa_mixed,
    "one_token_mixed": pin_one_token_mixed,
    "constant_keys_mixed": pin_constant_keys_mixed,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(orc, name):
    assert PINS[name](orc)


def test_empty_request_gives_zero(orc):
    case = synth.make_case(3, [0, 5, 0], 2, shuffle=True, seed=21)
    out, outb = run(orc, case, bits(case["kv"]), {})
    assert not out[0].any() and not out[2].any() and not outb[0].any()
    assert np.abs(out[1]).sum() > 0


def test_bf16_output_is_rne_of_f64(orc):
    case = synth.make_case(2, [5, 8], 1, shuffle=False, seed=22)
    out, outb = run(orc, case, bits(case["kv"]), {})
    # re-round independently through torch: fp64 -> fp32 is exact only when it
    # does not change the bf16 decision, so compare decoded values within half a bf16 ulp
    dec = torch.from_numpy(outb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.ldexp(1.0, np.frexp(np.abs(out))[1] - 8)
    assert np.all(np.abs(dec - out) <= ulp / 2 + 1e-300)


def test_selected_pairs_match_full(orc):
    case = synth.make_case(3, [9, 4, 12], 3, shuffle=True, seed=23)
    full, _ = run(orc, case, bits(case["kv"]), {})
    pairs = [(0, 3), (2, 15), (1, 0)]
    part, _ = run(orc, case, bits(case["kv"]), {}, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(part[b, h], full[b, h])
    assert np.isnan(part[0, 0]).all()


@pytest.fixture(scope="module")
def mutant_libs(orc, tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    text = orc.source()
    return {name: orc.build_variant(mutant_source(text, name), str(d / f"liborc_{name}.so")) for name in MUTANTS}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(orc, mutant_libs, mutant):
    with orc.variant(mutant_libs[mutant]):
        failed = [n for n, f in PINS.items() if not f(orc)]
    assert failed, f"mutant {mutant} ({MUTANTS[mutant][0]}) passed every pin"


def test_shipped_oracle_has_no_planted_mistake(orc):
    """The mutants exist only as patches: the oracle source holds none of
    their replacement text."""
    text = orc.source()
    for name, (_, patches) in MUTANTS.items():
        for old, new in patches:
            assert text.count(old) == 1 and new not in text, name


def test_multi_row_equals_row_slices(orc):
    """A request's 64 query rows decode exactly as four 16-row problems."""
    case = synth.make_case(2, [40, 13], 8, shuffle=True, seed=27)
    q = synth.normal_bf16((2, 64, 576), seed=28)
    args = (bits(case["kv"]), case["kv_indptr"].numpy(), case["page_table"].numpy(), case["page_size"])
    full, fullb = orc.decode(bits(q), *args)
    for g in range(4):
        part, partb = orc.decode(bits(q[:, 16 * g:16 * g + 16].contiguous()), *args)
        assert np.array_equal(full[:, 16 * g:16 * g + 16], part)
        assert np.array_equal(fullb[:, 16 * g:16 * g + 16], partb)


def test_index_errors_are_reported(orc):
    case = synth.make_case(1, [5], 2, shuffle=False, seed=24)
    with pytest.raises(ValueError):
        orc.decode(bits(case["q"]), bits(case["kv"]), case["kv_indptr"].numpy(), np.array([0, 1, 99], np.int32), 2)
