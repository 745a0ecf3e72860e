"""The gfx950 conversions the kernels rely on, checked point by point against
the oracle: packed fp32 -> e4m3 (through the standalone quantizer) and
fp32 -> bf16 (through the six-way producer with a zero table)."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from parity import act, dev_f32, host_u16, host_u8

pytestmark = pytest.mark.gpu


def e4m3_points():
    mags = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                          np.nextafter(pts, np.float32(0))])
    special = np.array([448.0, 448.00003, 463.99, 464.0, 480.0, 1e30, np.inf, np.nan,
                        2.0**-10, 2.0**-11, 3 * 2.0**-10, 1e-30, 1e-40, 0.0], np.float32)
    r = np.random.default_rng(0)
    rand = np.concatenate([r.uniform(-500, 500, 400_000), r.standard_normal(400_000) * 40,
                           r.standard_normal(200_000) * 2.0**-7]).astype(np.float32)
    return np.concatenate([pts, -pts, special, -special, rand])


def assert_e4m3_equal(v, got, ref):
    """Bitwise, except that a NaN input only has to give a NaN code: the
    hardware conversion writes 0xFF for every NaN, the oracle keeps the sign
    (NaN inputs are outside the pages' contract)."""
    nan = np.isnan(v)
    assert np.all((got[nan] & 0x7F) == 0x7F)
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_fp8_convert_matches_oracle_bitwise(orc):
    v = e4m3_points()
    got = host_u8(alnp.quant_fp8_static_f32(dev_f32(v), act(1.0)))
    assert_e4m3_equal(v, got, orc.e4m3_encode_sat(v))


def test_fp8_convert_with_act_scale(orc):
    v = e4m3_points() / np.float32(40.0)
    got = host_u8(alnp.quant_fp8_static_f32(dev_f32(v), act(0.025)))
    assert_e4m3_equal(v, got, orc.e4m3_encode_sat(v * np.float32(1.0 / np.float32(0.025))))


@pytest.mark.parametrize("a", [0.3, 0.7, 1.0 / 3.0, 3.0, 1e-3, 123.4, 6.1e-5])
def test_fp8_convert_with_inexact_reciprocal(orc, a):
    """act_scale values whose reciprocal is not exact in fp32: the kernels take
    1/act_scale as one correctly rounded fp32 division, as the oracle does, so
    v * (1/act) and its code agree bit for bit.  Points just around every e4m3
    midpoint (scaled back by the reciprocal) are the ones a reciprocal one ulp
    off would move across a rounding boundary."""
    print(f"fp8 convert act_scale={a}", flush=True)
    af = np.float32(a)
    inv = np.float32(1.0) / af
    mids = e4m3_points()
    rng = np.random.default_rng(int(af.view(np.uint32)))
    rand = (rng.standard_normal(1 << 18) * 120.0).astype(np.float32)
    v = np.concatenate([mids / inv, rand / inv]).astype(np.float32)
    got = host_u8(alnp.quant_fp8_static_f32(dev_f32(v), act(float(af))))
    assert_e4m3_equal(v, got, orc.e4m3_encode_sat((v * inv).astype(np.float32)))


def test_bf16_convert_matches_oracle(orc):
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    f = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    D = 1024
    f = f[: (f.size // (6 * D)) * 6 * D]
    params = f.reshape(1, -1, 6, D)
    mod = np.zeros((6, D), np.float32)
    outs = alnp.adaln_modulation6_bf16(dev_f32(params), dev_f32(mod))
    got = np.stack([host_u16(o) for o in outs])
    ref = orc.modulation6(params, mod)
    nan = (ref & 0x7F80) == 0x7F80
    nan &= (ref & 0x007F) != 0
    assert np.array_equal(got[~nan], ref[~nan])
    g = got[nan]
    assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)), "NaN must stay NaN"
