"""Pins for the oracle's number formats (bf16, e4m3fn, e2m1).

Each conversion is checked against something other than the oracle itself:
torch's CPU conversions (library routines), the format definitions' closed
forms (largest finite value, subnormal step, midpoints), and the page-printed
FP4 packing example (h3-blackwell-runtime compare page,
benchmarks/gb10-cute-nvfp4-conversion-contract.json).
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_e4m3_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


# ---- bf16 -----------------------------------------------------------------

def test_bf16_widen_all_patterns(orc):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f32(b).view(np.uint32)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy().view(np.uint32)
    finite = (b & 0x7F80) != 0x7F80
    assert np.array_equal(ours[finite], ref[finite])
    # Widening is exact: the pattern lands in the upper half.
    assert np.array_equal(ours, b.astype(np.uint32) << 16)


def _structured_f32_patterns():
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000,
                     0x8001, 0xBFFF, 0xC000, 0xFFFE, 0xFFFF], np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


def test_bf16_rtne_structured_exhaustive(orc):
    """Every bf16 exponent/mantissa with low halves at, below and above the
    tie point, against torch's RTNE conversion."""
    u = _structured_f32_patterns()
    f = u.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN, quiet, with its sign.
    o = ours[nan]
    assert np.all((o & 0x7F80) == 0x7F80) and np.all((o & 0x0040) != 0)
    assert np.array_equal(o >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_rtne_random_patterns(orc):
    u = np.random.default_rng(1).integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_ties_and_overflow(orc):
    f = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.3895313892515355e38,
                  3.4028234663852886e38, np.inf, -np.inf], np.float32)
    got = orc.f32_to_bf16(f)
    # 1+2^-8 is halfway between 1 and 1+2^-7: even side is 1.0 (0x3F80).
    # 1+3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even, 0x3F82).
    # bf16 max finite is 0x7F7F = 3.3895e38; FLT_MAX rounds up to infinity.
    assert list(got) == [0x3F80, 0x3F82, 0xBF80, 0x7F7F, 0x7F80, 0x7F80, 0xFF80]


# ---- e4m3fn ---------------------------------------------------------------

def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch_e4m3_values()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(ours[nan]))
    assert np.array_equal(ours[~nan], ref[~nan])
    # Closed forms of the format: 448 max, 2^-9 smallest subnormal,
    # 2^-6 smallest normal, bias 7.
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0**-9
    assert ours[0x08] == 2.0**-6 and ours[0x38] == 1.0 and ours[0x62] == 40.0


def _finite_magnitudes():
    return np.array([torch_e4m3_values()[c] for c in range(127)])


def test_e4m3_roundtrip_every_code(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch_e4m3_values()[codes].astype(np.float32)
    vals[codes == 0x80] = -0.0
    assert np.array_equal(orc.e4m3_encode_sat(vals), codes)


def test_e4m3_midpoints_ties_to_even(orc):
    mags = _finite_magnitudes()
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)  # exact in fp32
    lower = np.arange(126)
    even = np.where(lower % 2 == 0, lower, lower + 1).astype(np.uint8)
    assert np.array_equal(orc.e4m3_encode_sat(mids), even)
    assert np.array_equal(orc.e4m3_encode_sat(-mids), even | 0x80)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert np.array_equal(orc.e4m3_encode_sat(up), (lower + 1).astype(np.uint8))
    assert np.array_equal(orc.e4m3_encode_sat(dn), lower.astype(np.uint8))
    # The same points through torch's conversion (RTNE, no saturation needed).
    for v in (mids, up, dn, -mids):
        assert np.array_equal(orc.e4m3_encode_sat(v), torch_e4m3_bits(v))


def test_e4m3_random_vs_torch(orc):
    r = np.random.default_rng(2)
    v = np.concatenate([
        r.uniform(-447.9, 447.9, 500_000),
        r.standard_normal(500_000) * 40,
        r.standard_normal(200_000) * 2**-7,
    ]).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode_sat(v), torch_e4m3_bits(v))


def test_e4m3_saturation_and_specials(orc):
    v = np.array([448.0, 448.00003, 463.9, 464.0, 480.0, 1e30, np.inf,
                  -448.0, -1e30, -np.inf, np.nan, -np.nan,
                  2.0**-10, -(2.0**-11), 3 * 2.0**-10, 0.0, -0.0, 40.0], np.float32)
    got = orc.e4m3_encode_sat(v)
    assert list(got[:7]) == [0x7E] * 7
    assert list(got[7:10]) == [0xFE] * 3
    assert got[10] & 0x7F == 0x7F and got[11] & 0x7F == 0x7F
    # 2^-10 is halfway between 0 and 2^-9 -> 0 (even); -2^-11 -> -0;
    # 3*2^-10 is halfway between 2^-9 (code 1) and 2^-8 (code 2) -> code 2.
    assert list(got[12:]) == [0x00, 0x80, 0x02, 0x00, 0x80, 0x62]


# ---- e2m1 -----------------------------------------------------------------

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table(orc):
    got = orc.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == E2M1
    assert list(-got[8:]) == E2M1
    assert np.signbit(got[8])


def test_e2m1_encode_codes_and_midpoints(orc):
    vals = np.array(E2M1, np.float32)
    assert list(orc.e2m1_encode(vals)) == list(range(8))
    assert list(orc.e2m1_encode(-vals)) == [8 + c for c in range(8)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    # Ties go to the code with an even mantissa bit.
    assert list(orc.e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert list(orc.e2m1_encode(up)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(orc.e2m1_encode(dn)) == [0, 1, 2, 3, 4, 5, 6]
    big = np.array([6.0001, 7.0, 100.0, np.inf, -1e9], np.float32)
    assert list(orc.e2m1_encode(big)) == [7, 7, 7, 7, 15]
    assert list(orc.e2m1_encode(np.array([-0.1, -0.0, 0.2], np.float32))) == [8, 8, 0]


def test_e2m1_nibble_order_page_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "fp4_nibble_order.json")))
    page = np.array(g["expected_low_first_bytes"], np.uint8)
    n = g["value_count"]
    # Unpack with the oracle's order: element 2i in the low nibble of byte i.
    codes = np.empty(2 * page.size, np.uint8)
    codes[0::2] = page & 0xF
    codes[1::2] = page >> 4
    vals = orc.e2m1_decode(codes)
    sweep, pad = vals[:n], vals[n:]
    assert np.all(np.diff(sweep) >= 0), "not an ascending sweep"
    assert sweep[0] == -6.0 and sweep[-1] == 6.0
    assert np.all(pad == 0) and not np.any(np.signbit(pad))
    # The opposite nibble order does not give a sweep: the fixture
    # discriminates between the two readings.
    swapped = np.empty_like(codes)
    swapped[0::2] = page >> 4
    swapped[1::2] = page & 0xF
    assert np.any(np.diff(orc.e2m1_decode(swapped)[:n]) < 0)
    # Encoding the decoded values (signed zeros kept) and packing gives the
    # page's bytes back.
    again = orc.e2m1_encode(vals.astype(np.float32))
    assert np.array_equal(orc.fp4_pack(again), page)
