"""Pins of the RMSNorm-modulation oracle (modulated RMSNorm with segment-selected
scale/shift rows, bf16 operations): torch's own rms_norm in float64 and torch's
CPU bf16 tensor arithmetic as independent implementations, and closed forms for
the segment routing and the bf16 rounding boundaries."""
import numpy as np
import torch

from dit_adaptive_layernorm_amd import inputs

EPS = 1e-5


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(b):
    return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32)


def ordinal(b):
    """Signed ordinal of bf16 patterns: adjacent finite values differ by 1."""
    b = np.asarray(b).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def offset_rows(rows, dim, seed):
    """N(0, 1) rows shifted by a per-row offset, so a centring slip shows."""
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=seed)
    off = inputs.normal_f32((rows, 1), 2.0, seed, 99)
    d["x"] = inputs.to_bf16_bits(f32(d["x"]) + off)
    return d


def test_normalization_matches_torch_rms_norm(orc):
    # Zero scale and shift leave the bf16 RMSNorm output itself: compare with
    # torch's rms_norm evaluated in float64 and rounded once to bf16.
    rows, dim = 48, 1040
    d = offset_rows(rows, dim, 3)
    zero = np.zeros((1, dim), np.uint16)
    seg = np.zeros(rows, np.int32)
    out, rstd, n = orc.rms_modulate_seg(d["x"], d["weight"], zero, zero, seg, EPS, want_n=True)
    assert np.array_equal(out, n)
    x = torch.from_numpy(f32(d["x"]).astype(np.float64))
    w = torch.from_numpy(f32(d["weight"]).astype(np.float64))
    ref = bits(torch.nn.functional.rms_norm(x, (dim,), w, EPS).to(torch.bfloat16))
    diff = np.abs(ordinal(out) - ordinal(ref))
    assert diff.max() <= 1 and np.mean(diff == 0) >= 0.999
    ms = (f32(d["x"]).astype(np.float64) ** 2).mean(axis=1)
    assert np.allclose(rstd, 1.0 / np.sqrt(ms + EPS), rtol=1e-7)


def test_no_weight_is_unit_weight(orc):
    rows, dim = 8, 64
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=4)
    one = inputs.to_bf16_bits(np.ones(dim, np.float32))
    a = orc.rms_modulate_seg(d["x"], None, d["scale"], d["shift"], d["seg"], EPS)[0]
    b = orc.rms_modulate_seg(d["x"], one, d["scale"], d["shift"], d["seg"], EPS)[0]
    assert np.array_equal(a, b)


def test_modulation_matches_torch_bf16_ops(orc):
    # The modulation stage against torch's CPU bf16 tensor operations (each
    # computed in fp32 and rounded to bf16), on the oracle's own RMSNorm output,
    # with per-row segment gathers by index_select.
    rows, dim, segments = 64, 512, 4
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=5, segments=segments)
    sc = inputs.normal_bf16((segments, dim), 0.7, 5, 50)   # wide, so 1 + sc rounds
    sh = inputs.normal_bf16((segments, dim), 0.7, 5, 51)
    out, _, n = orc.rms_modulate_seg(d["x"], d["weight"], sc, sh, d["seg"], EPS, want_n=True)
    idx = torch.from_numpy(d["seg"].astype(np.int64))
    s_t = torch.index_select(bf16_tensor(sc), 0, idx)
    h_t = torch.index_select(bf16_tensor(sh), 0, idx)
    ref = bits((bf16_tensor(n) * (s_t + 1)) + h_t)
    assert np.array_equal(out, ref)
    assert np.array_equal(orc.bf16_modulate(n, bits(s_t), bits(h_t)), ref)


def test_closed_forms(orc):
    dim = 4
    zero = np.zeros((1, dim), np.uint16)
    seg0 = np.zeros(1, np.int32)
    # A constant row a: mean of squares a^2, so n = a / sqrt(a^2 + eps) rounds
    # to 1 (a centred LayerNorm would give 0, a 1/(dim-1) mean 0.87).
    x = inputs.to_bf16_bits(np.full((1, dim), 3.0, np.float32))
    out, rstd, _ = orc.rms_modulate_seg(x, None, zero, zero, seg0, EPS)
    assert np.all(out == 0x3F80)
    assert rstd[0] == np.float32(1.0 / np.sqrt(9.0 + EPS))
    # eps = 0 and a row of +-2: rstd = 1/2 exactly, n = +-1.
    x = inputs.to_bf16_bits(np.array([[2, -2, 2, -2]], np.float32))
    out, rstd, _ = orc.rms_modulate_seg(x, None, zero, zero, seg0, 0.0)
    assert rstd[0] == 0.5 and np.array_equal(f32(out)[0], [1, -1, 1, -1])


def test_scale_shift_identities(orc):
    rows, dim = 16, 256
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=6)
    segs = d["scale"].shape[0]
    full = lambda v: inputs.to_bf16_bits(np.full((segs, dim), v, np.float32))
    _, _, n = orc.rms_modulate_seg(d["x"], d["weight"], full(0), full(0), d["seg"], EPS,
                                   want_n=True)
    # scale = -1: 1 + scale = 0, so the output is the shift row itself.
    out = orc.rms_modulate_seg(d["x"], d["weight"], full(-1), d["shift"], d["seg"], EPS)[0]
    assert np.array_equal(out, d["shift"][d["seg"]])
    # scale = 1, shift = 0: exactly 2 n.
    out = orc.rms_modulate_seg(d["x"], d["weight"], full(1), full(0), d["seg"], EPS)[0]
    assert np.array_equal(f32(out), 2 * f32(n))
    # scale = 2^-8: 1 + 2^-8 is a bf16 tie and rounds to the even 1, so the
    # output is n (an unrounded 1 + scale would move most of them up).
    out = orc.rms_modulate_seg(d["x"], d["weight"], full(2.0 ** -8), full(0), d["seg"], EPS)[0]
    assert np.array_equal(out, n)
    unrounded = inputs.to_bf16_bits(f32(n) * np.float32(1 + 2.0 ** -8))
    assert np.mean(unrounded != n) > 0.5


def test_product_is_rounded_before_the_shift(orc):
    # n = t = 1 + 2^-7: n * t = 1 + 2^-6 + 2^-14 rounds to 1 + 2^-6.  Adding the
    # shift 2^-8 then lands exactly between 1 + 2^-6 and 1 + 3 * 2^-7 and goes to
    # the even 1 + 2^-6; without the bf16 step the 2^-14 would carry the sum
    # up to 1 + 3 * 2^-7.
    b = lambda v: inputs.to_bf16_bits(np.array([v], np.float32))
    y = orc.bf16_modulate(b(1 + 2.0 ** -7), b(2.0 ** -7), b(2.0 ** -8))
    assert f32(y)[0] == np.float32(1 + 2.0 ** -6)
    assert inputs.to_bf16_bits(np.array([(1 + 2.0 ** -7) ** 2 + 2.0 ** -8], np.float32))[0] != y[0]


def test_segment_routing(orc):
    rows, dim, segments = 12, 32, 5
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=7, segments=segments)
    sc = inputs.to_bf16_bits(np.full((segments, dim), -1.0, np.float32))
    sh = inputs.to_bf16_bits(np.repeat(0.5 * (np.arange(segments, dtype=np.float32) + 1)[:, None],
                                       dim, axis=1))
    out = orc.rms_modulate_seg(d["x"], d["weight"], sc, sh, d["seg"], EPS)[0]
    assert np.array_equal(f32(out), np.repeat((0.5 * (d["seg"] + 1))[:, None], dim, axis=1))


def test_out_of_range_segment_gives_nan_row(orc):
    rows, dim = 4, 48
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=8)
    seg = np.array([0, -1, 3, 2], np.int32)   # 3 tables rows: -1 and 3 are outside
    out, rstd, _ = orc.rms_modulate_seg(d["x"], d["weight"], d["scale"], d["shift"], seg, EPS)
    assert np.all(out[1] == 0x7FC0) and np.all(out[2] == 0x7FC0)
    good = orc.rms_modulate_seg(d["x"][[0, 3]], d["weight"], d["scale"], d["shift"],
                                seg[[0, 3]], EPS)[0]
    assert np.array_equal(out[[0, 3]], good)
    assert np.all(np.isfinite(rstd))
