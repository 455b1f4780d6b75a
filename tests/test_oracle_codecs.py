"""Pins for the oracle's number-format codecs, each against something other
than the oracle itself: torch's own fp8/bf16 conversions (library routines),
the e2m1 table printed on page 668813 (tests/golden/e2m1_table.txt) and the
e8m0 closed form 2^(e-127)."""
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3fn_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e2m1_matches_page_table(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_table.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = float(orc.e2m1_to_f64(np.array([int(code)]))[0])
        assert got == float(val), (code, got, val)
    # the table on the page stores code 8 as 0.0; OCP MX makes it a negative zero
    assert math.copysign(1.0, float(orc.e2m1_to_f64(np.array([8]))[0])) == -1.0


def test_e8m0_closed_form(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e8m0_to_f64(codes)
    for e in range(255):
        assert got[e] == math.ldexp(1.0, e - 127)
    assert math.isnan(got[255])


def test_bf16_all_patterns_match_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f64_to_bf16_matches_torch_on_fp32_inputs(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-39,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    ours = orc.f64_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_ties_and_nearest(orc):
    # exact midpoints between adjacent bf16 values go to the even mantissa;
    # anything off the midpoint goes to the nearer neighbour (single rounding
    # from fp64, which an fp32 intermediate would get wrong).
    for lo_bits in (0x3F80, 0x3F81, 0x4120, 0x4121, 0x0001, 0x7F7E):
        lo = orc.bf16_to_f64(np.array([lo_bits], dtype=np.uint16))[0]
        hi = orc.bf16_to_f64(np.array([lo_bits + 1], dtype=np.uint16))[0]
        mid = (lo + hi) / 2
        even = lo_bits if lo_bits % 2 == 0 else lo_bits + 1
        assert orc.f64_to_bf16(np.array([mid]))[0] == even
        assert orc.f64_to_bf16(np.array([-mid]))[0] == (even | 0x8000)
        eps = (hi - lo) * 2.0 ** -30
        assert orc.f64_to_bf16(np.array([mid + eps]))[0] == lo_bits + 1
        assert orc.f64_to_bf16(np.array([mid - eps]))[0] == lo_bits
