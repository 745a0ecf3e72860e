"""Pins of the oracle's MX block formats (OCP Microscaling Formats v1.0: blocks
of 32 values sharing an E8M0 power-of-two scale 2^(floor(log2 amax) - emax),
elements rounded to nearest even and saturated): numpy's frexp for the
exponent, closed forms at the scale's edges, torch's float8_e4m3fn conversion
for MXFP8 elements, invariance under power-of-two scaling, and composition
with the pinned FP4/FP8 paths for what gets quantized."""
import numpy as np
import pytest
import torch

from dit_adaptive_layernorm_amd import inputs

EMAX_FP4, EMAX_FP8 = 2, 8


def f32(b):
    return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32)


def test_e8m0_scale_closed_forms(orc):
    # 6 * 2^k is E2M1's largest magnitude times 2^k: the scale is exactly 2^k.
    for k in range(-120, 121, 7):
        assert orc.e8m0_scale(np.float32(6.0 * 2.0 ** k), EMAX_FP4) == k + 127
        assert orc.e8m0_scale(np.float32(448.0 * 2.0 ** k), EMAX_FP8) == k + 127
    # Powers of two and the values just below them.
    for j in (-100, -3, 0, 1, 9, 100):
        p = np.float32(2.0 ** j)
        below = np.nextafter(p, np.float32(0))
        assert orc.e8m0_scale(p, EMAX_FP8) == j - 8 + 127
        assert orc.e8m0_scale(below, EMAX_FP8) == j - 9 + 127
    # Clamps and specials.
    assert orc.e8m0_scale(np.float32(2.0 ** -140), EMAX_FP4) == 0        # E = -142 -> -127
    assert orc.e8m0_scale(np.float32(3.0e38), EMAX_FP4) == 125 + 127
    assert orc.e8m0_scale(np.float32(np.inf), EMAX_FP8) == 254
    assert orc.e8m0_scale(0.0, EMAX_FP4) == 0
    assert orc.e8m0_scale(np.float32(np.nan), EMAX_FP4) == 0


def test_e8m0_scale_matches_frexp(orc):
    r = np.random.default_rng(3)
    amax = np.abs(r.standard_normal(4000) * 10.0 ** r.uniform(-30, 30, 4000)).astype(np.float32)
    for emax in (EMAX_FP4, EMAX_FP8):
        _, e = np.frexp(amax.astype(np.float64))
        want = np.clip(e - 1 - emax, -127, 127) + 127
        got = np.array([orc.e8m0_scale(a, emax) for a in amax])
        assert np.array_equal(got, want)


def test_e8m0_decode(orc):
    for c in (0, 1, 100, 127, 128, 254):
        assert orc.e8m0_decode(c) == np.ldexp(1.0, c - 127)
    assert np.isnan(orc.e8m0_decode(255))


def test_mxfp8_elements_match_torch_e4m3(orc):
    # Elements v / X in e4m3 against torch's float8_e4m3fn conversion (round to
    # nearest even); above 448 and below 512 the MX reading saturates.
    r = np.random.default_rng(4)
    v = (r.standard_normal(32 * 400) * np.repeat(10.0 ** r.uniform(-6, 6, 400), 32)).astype(np.float32)
    codes, scales = orc.mx_block_quant(v, fp4=False)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32)
    q = (v / X).astype(np.float32)
    assert np.all(np.abs(q) < 512)
    ref = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # Every block's largest element lands in [256, 512) before saturation.
    amax = np.abs(q).reshape(-1, 32).max(1)
    assert np.all((amax >= 256) & (amax < 512))


def test_mxfp4_elements_are_the_e2m1_encoder_of_v_over_x(orc):
    r = np.random.default_rng(5)
    v = (r.standard_normal(32 * 300) * np.repeat(10.0 ** r.uniform(-5, 5, 300), 32)).astype(np.float32)
    codes, scales = orc.mx_block_quant(v, fp4=True)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32)
    q = (v / X).astype(np.float32)
    assert np.array_equal(codes, orc.e2m1_encode(q))
    amax = np.abs(q).reshape(-1, 32).max(1)
    assert np.all((amax >= 4) & (amax < 8))
    # The largest element of each block encodes to 4 or 6 (codes 6, 7).
    mag = (codes & 7).reshape(-1, 32).max(1)
    assert np.all((mag == 6) | (mag == 7))


def test_power_of_two_scaling_moves_only_the_scale(orc):
    r = np.random.default_rng(6)
    v = r.standard_normal(32 * 64).astype(np.float32)
    for fp4 in (True, False):
        c0, s0 = orc.mx_block_quant(v, fp4)
        for k in (-20, -1, 3, 40):
            c1, s1 = orc.mx_block_quant((v * np.float32(2.0 ** k)).astype(np.float32), fp4)
            assert np.array_equal(c1, c0) and np.array_equal(s1.astype(int), s0.astype(int) + k)


def test_zero_and_signed_zero_blocks(orc):
    v = np.zeros(64, np.float32)
    v[32:] = -0.0
    for fp4 in (True, False):
        codes, scales = orc.mx_block_quant(v, fp4)
        assert np.all(scales == 0)
        assert np.all(codes[:32] == 0) and np.all(codes[32:] == (0x8 if fp4 else 0x80))


def test_dequantization_error_bound(orc):
    # Unsaturated elements are within half an element step of v: E2M1 steps are
    # 0.5 below 2, 1 below 4, 2 above; E4M3 has 3 mantissa bits.
    r = np.random.default_rng(7)
    v = (r.standard_normal(32 * 200) * 3).astype(np.float32)
    codes, scales = orc.mx_block_quant(v, fp4=True)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32)
    q = v / X
    deq = orc.e2m1_decode(codes)
    step = np.where(np.abs(q) < 2, 0.5, np.where(np.abs(q) < 4, 1.0, 2.0))
    ok = (np.abs(deq - q) <= step / 2 + 1e-12) | (np.abs(q) > 6)
    assert np.all(ok)


def test_mxfp4_quantizes_the_fp4_paths_staged_values(orc):
    # What MXFP4 quantizes is the same bf16-staged value as the NVFP4 paths.
    d = inputs.make("bcast", rows=9, dim=1024, seed=41)
    p, s, m, rs, b = orc.adaln_mxfp4(d["x"], want_b=True)
    assert np.array_equal(b, orc.ln_fp4(d["x"], want_b=True)[4])
    codes, scales = orc.mx_block_quant(b, fp4=True)
    assert np.array_equal(scales.reshape(9, 32), s)
    assert np.array_equal(orc.fp4_pack(codes).reshape(9, 512), p)
    _, _, _, _, bm = orc.adaln_mxfp4(d["x"], d["scale"], d["shift"], want_b=True)
    assert np.array_equal(bm, orc.adaln_fp4(d["x"], d["scale"], d["shift"], want_b=True)[4])


def test_mxfp8_quantizes_the_fp8_paths_y(orc):
    for kind in ("ln", "bcast", "ptok"):
        d = inputs.make(kind, rows=7, dim=512, seed=42)
        if kind == "ln":
            out, s, _, _, y = orc.adaln_mxfp8(d["x"], want_y=True)
            ref_y = orc.ln_fp8(d["x"], 1.0, want_y=True)[3]
        elif kind == "bcast":
            out, s, _, _, y = orc.adaln_mxfp8(d["x"], d["scale"], d["shift"], want_y=True)
            ref_y = orc.adaln_fp8_bcast(d["x"], d["scale"], d["shift"], 1.0, want_y=True)[3]
        else:
            out, s, _, _, y = orc.adaln_mxfp8(d["x"], d["scale"], d["shift"], want_y=True)
            ref_y = orc.adaln_fp8_ptok(d["x"], d["scale"], d["shift"], 1.0, want_y=True)[3]
        assert np.array_equal(y, ref_y), kind
        codes, scales = orc.mx_block_quant(y, fp4=False)
        assert np.array_equal(codes.reshape(out.shape), out) and np.array_equal(scales.reshape(s.shape), s)


def test_mxfp8_table_quantizes_the_table_paths_y(orc):
    d = inputs.make("table", rows=6, dim=256, seed=45)
    out, s, _, _, y = orc.adaln_mxfp8_table(d["x"], d["temb"], d["table"], d["shift_idx"],
                                            d["scale_idx"], want_y=True, threads=2)
    ref_y = orc.adaln_fp8_table(d["x"], d["temb"], d["table"], d["shift_idx"], d["scale_idx"],
                                1.0, want_y=True)[3]
    assert np.array_equal(y, ref_y)
    codes, scales = orc.mx_block_quant(y, fp4=False)
    assert np.array_equal(codes.reshape(out.shape), out) and np.array_equal(scales.reshape(s.shape), s)



def _e4m3_operands(dim, seed):
    """Finite e4m3 codes (NaN codes excluded) for (dim,) modfp8 operands."""
    r = np.random.default_rng(seed)
    codes = r.integers(0, 256, dim).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    return codes


def _bf16_of_e4m3(orc, codes, deq):
    # Every e4m3 value times a power of two is exact in bf16.
    return orc.f32_to_bf16((orc.e4m3_decode(codes) * np.float64(deq)).astype(np.float32))


@pytest.mark.parametrize("deq", [(1.0, 1.0), (0.5, 0.25), (4.0, 0.125)])
def test_mxfp8_modfp8_is_broadcast_with_the_decoded_operands(orc, deq):
    d = inputs.make("bcast", rows=11, dim=512, seed=50)
    sf, hf = _e4m3_operands(512, 51), _e4m3_operands(512, 52)
    got = orc.adaln_mxfp8_modfp8(d["x"], sf, hf, deq[0], deq[1])
    ref = orc.adaln_mxfp8(d["x"], _bf16_of_e4m3(orc, sf, deq[0]), _bf16_of_e4m3(orc, hf, deq[1]),
                          want_y=True)
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8))


@pytest.mark.parametrize("deq", [(1.0, 1.0), (0.5, 2.0)])
def test_mxfp4_modfp8_is_broadcast_with_the_decoded_operands(orc, deq):
    d = inputs.make("bcast", rows=9, dim=256, seed=53)
    sf, hf = _e4m3_operands(256, 54), _e4m3_operands(256, 55)
    got = orc.adaln_mxfp4_modfp8(d["x"], sf, hf, deq[0], deq[1])
    ref = orc.adaln_mxfp4(d["x"], _bf16_of_e4m3(orc, sf, deq[0]), _bf16_of_e4m3(orc, hf, deq[1]),
                          want_b=True)
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8))


def test_mxfp8_awq_identity_and_power_of_two_smoothing(orc):
    d = inputs.make("bcast", rows=8, dim=512, seed=56)
    one = np.full(512, 0x3F80, np.uint16)                       # bf16 1.0
    got = orc.awq_adaln_mxfp8(d["x"], d["scale"], d["shift"], one)
    ref = orc.adaln_mxfp8(d["x"], d["scale"], d["shift"], want_y=True)
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8))
    # inv_s = 2^k in every channel: the same element codes, scales moved by k
    # (away from the E8M0 clamp).
    for k in (-3, 2):
        pk = np.full(512, (127 + k) << 7, np.uint16)            # bf16 2^k
        o, s, _, _, _ = orc.awq_adaln_mxfp8(d["x"], d["scale"], d["shift"], pk)
        assert np.array_equal(o, ref[0]) and np.array_equal(s.astype(int), ref[1].astype(int) + k)
