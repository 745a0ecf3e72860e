"""Pins for the oracle's FP4 producer (LayerNorm -> bf16 stage -> e2m1 with
one e4m3 scale per 16 elements).

The block rule (scale = e4m3(amax / 6), clamp at 448, E2M1 round to nearest
even) is the one in the h3-blackwell-runtime compare page,
benchmarks/gb10-cute-p1-stream-a-summary.json, "numerical_contract", taken
with a global scale of 1; the bf16 staging of the normalized row is the
"staged BF16-norm" of the "adaptive-layernorm-producers" README,
"Validation".  Blocks are hand-built so the expected codes follow from the
e2m1 and e4m3 tables alone.
"""
import numpy as np
import torch

from dit_adaptive_layernorm_amd import inputs

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def e4m3_code(v):
    return int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_block_amax_six_is_identity(orc):
    """amax = 6 -> scale 1.0 (code 0x38) -> codes are the values' own codes."""
    b = np.concatenate([GRID, -GRID]).astype(np.float32)
    codes, sc = orc.fp4_block_quant(b)
    assert sc[0] == 0x38
    assert list(codes) == list(range(8)) + [8 + c for c in range(8)]


def test_block_power_of_two_scale(orc):
    for e in (-6, -3, 0, 2, 5):
        s = 2.0**e
        b = np.concatenate([GRID, GRID[::-1]]).astype(np.float32) * np.float32(s)
        codes, sc = orc.fp4_block_quant(b)
        assert sc[0] == e4m3_code(s)
        assert list(codes) == list(range(8)) + list(range(7, -1, -1))


def test_block_scale_rounds_to_nearest_e4m3(orc):
    """amax 7 -> 7/6 = 1.1667 -> nearest e4m3 is 1.125 (code 0x39);
    then 7 / 1.125 = 6.22 -> 6, and 3 / 1.125 = 2.67 -> 3."""
    b = np.zeros(16, np.float32)
    b[0], b[1], b[2] = 7.0, 3.0, -1.0
    codes, sc = orc.fp4_block_quant(b)
    assert sc[0] == 0x39
    # -1/1.125 = -0.889 -> -1 (code 0xA)
    assert list(codes[:3]) == [7, 5, 0xA] and not np.any(codes[3:])


def test_block_outlier(orc):
    """One x20 outlier sets the scale; small neighbours fall to 0 or 0.5."""
    b = np.array([20.0] + [0.3, -0.7, 0.05, -0.05, 0.9, 1.0, -2.0] * 2 + [0.0],
                 np.float32)
    codes, sc = orc.fp4_block_quant(b)
    s = 3.25                               # e4m3 nearest to 20/6 = 3.333
    assert sc[0] == e4m3_code(s) == 0x45
    enc = np.float32(1.0) / np.float32(s)
    ref = []
    for v in b:                            # nearest grid value, by hand
        a = abs(float(np.float32(v) * enc))
        ref.append(int(np.argmin(np.abs(GRID - a))) | (8 if v < 0 else 0))
    assert list(codes) == ref
    assert codes[0] == 7


def test_block_all_zero(orc):
    codes, sc = orc.fp4_block_quant(np.zeros(16, np.float32))
    assert sc[0] == 0 and not np.any(codes)
    # A block too small for the smallest scale also gives a zero scale.
    codes, sc = orc.fp4_block_quant(np.full(16, 2.0**-14, np.float32))
    assert sc[0] == 0 and not np.any(codes)


def test_block_scale_saturates(orc):
    b = np.full(16, 3000.0, np.float32)
    codes, sc = orc.fp4_block_quant(b)
    assert sc[0] == 0x7E          # 3000/6 = 500 > 448 -> 448
    assert np.all(codes == 7)     # 3000/448 = 6.7 -> 6


def test_ln_fp4_alternating_row(orc):
    """Row +-a: xhat = +-a/sqrt(a^2+eps) = +-0.99999 -> bf16 +-1.0;
    amax 1 -> scale e4m3(1/6) = 0.171875 (0x23) -> 1/0.171875 = 5.82 -> 6
    (code 7); packed low nibble first: 0xF7 (7 | 0xF << 4)."""
    x = inputs.to_bf16_bits(np.tile(np.array([1.5, -1.5], np.float32), 64)[None])
    packed, sf, mean, rstd, b = orc.ln_fp4(x, want_b=True)
    assert np.all(np.abs(b) == 1.0)
    assert np.all(sf == 0x23)
    assert np.all(packed == 0xF7)


def test_ln_fp4_constant_row_is_zero(orc):
    x = inputs.to_bf16_bits(np.full((2, 64), 0.75, np.float32))
    packed, sf, _, _, _ = orc.ln_fp4(x)
    assert not np.any(packed) and not np.any(sf)


def test_ln_fp4_composes_stages(orc):
    """LN->FP4 equals: the FP8 path's modulation-off normalized row, rounded to
    bf16 (torch's conversion), then block quantization and packing."""
    d = inputs.make("fp4", rows=24, dim=512, seed=6)
    packed, sf, mean, rstd, b = orc.ln_fp4(d["x"], want_b=True)
    _, mean2, rstd2, y = orc.ln_fp8(d["x"], 1.0, want_y=True)
    assert np.array_equal(mean, mean2) and np.array_equal(rstd, rstd2)
    staged = torch.from_numpy(y).to(torch.bfloat16).float().numpy()
    assert np.array_equal(b, staged)
    codes, sc = orc.fp4_block_quant(staged)
    assert np.array_equal(sf, sc)
    assert np.array_equal(packed, orc.fp4_pack(codes))


def test_ln_fp4_dequant_error_bound(orc):
    """Each dequantized value lies within half a grid step (x scale) of the
    staged value, or at +-6*scale when it exceeds the grid."""
    d = inputs.make("fp4", rows=32, dim=1024, seed=8)
    packed, sf, _, _, b = orc.ln_fp4(d["x"], want_b=True)
    codes = np.empty((32, 1024), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    s = np.repeat(orc.e4m3_decode(sf), 16, axis=1)
    deq = orc.e2m1_decode(codes) * s
    step = np.where(np.abs(deq) / np.maximum(s, 1e-30) >= 4, 2.0, np.where(np.abs(deq) / np.maximum(s, 1e-30) >= 2, 1.0, 0.5))
    err = np.abs(deq - b.astype(np.float64))
    assert np.all(err <= step * s / 2 + 1e-12)


def test_ln_fp4_batch_invariance(orc):
    d = inputs.make("fp4", rows=65, dim=256, seed=9)
    full = orc.ln_fp4(d["x"])
    for r0, r1 in ((0, 1), (7, 14), (64, 65), (3, 60)):
        part = orc.ln_fp4(d["x"][r0:r1])
        assert np.array_equal(part[0], full[0][r0:r1])
        assert np.array_equal(part[1], full[1][r0:r1])
    thr = orc.ln_fp4(d["x"], threads=3)
    assert np.array_equal(thr[0], full[0]) and np.array_equal(thr[1], full[1])
