"""Pin of the oracle's fp32 modulation sequence.

The h3-blackwell-runtime page ("NVFP4 Modulation Producer Fusion" ->
"Exactness Contract") fixes the order (x * (scale + 1)) + shift; the FP8
path evaluates it in fp32 with each operation rounded and no fused
multiply-add.  Scale -1, 0 and 1 (the other oracle tests) are exact under
every order, so they cannot tell it from a fused or re-associated one.  Here:

- hand-built cases, one per plausible slip (tests/exact32.py), each with a
  different e4m3 code under the right order and under the slip, are fed to
  the oracle, whose y and codes must follow the right order;
- random per-token rows, whose pre-quantization y must equal numpy's
  float32 evaluation of the sequence bit for bit, from the oracle's own
  (separately pinned) row statistics.

The hand-built rows have mean 0 and variance 16 exactly, and eps = 0, so
rstd = 1/4 and xhat = x / 4 exactly, on any correct implementation: the
statistics add no rounding of their own and the cases reach the modulation
unchanged.
"""
import math

import numpy as np
import pytest

from dit_adaptive_layernorm_amd import inputs
from exact32 import (ACT_SCALE, WRONG_ORDERS, add32, e4m3_code, find_case, fma32, mul32,
                     right_order)

# One 32-element block: sum 0, sum of squares 2 * (169 + 81 + 4 + 1 + 1) =
# 512, so mean 0 and biased variance 512 / 32 = 16; xhat = x / 4 takes the
# values +-3.25, +-2.25, +-0.5, +-0.25 and 0.
BLOCK = np.array([13, -13, 9, -9, 2, -2, 1, -1, 1, -1] + [0] * 22, np.float32)


def bf16(f):
    return inputs.to_bf16_bits(np.asarray(f, np.float32))


def f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


@pytest.fixture(scope="module")
def cases():
    found = {name: find_case(fn) for name, fn in WRONG_ORDERS.items()}
    missing = [n for n, c in found.items() if c is None]
    assert not missing, f"no discriminating case found for {missing}"
    return found


def case_row(cases):
    """x (1, 32 * K) of K blocks and fp32 scale / shift (1, 32 * K): case k
    sits in block k at the column whose xhat is the case's; every other
    column has scale = shift = 0."""
    names = sorted(cases)
    x = np.tile(BLOCK, len(names))
    sc = np.zeros_like(x)
    sh = np.zeros_like(x)
    cols = {}
    for k, name in enumerate(names):
        c, s, h = cases[name]
        j = 32 * k + int(np.flatnonzero(BLOCK / 4 == c)[0])
        sc[j], sh[j] = s, h
        cols[name] = j
    return bf16(x)[None], sc[None], sh[None], cols


def test_exact_helpers_are_ieee_binary32():
    """The rational model rounds as numpy's float32 does (IEEE), including
    subnormal results, exact zeros and ties."""
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    b = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    a[:40] = np.float32(2.0**-120) * np.arange(40, dtype=np.float32)   # subnormal products
    b[40:80] = -a[40:80]                                               # exact zero sums
    a[80:100] = np.float32(1.0)
    b[80:100] = np.float32(2.0**-24) * np.arange(1, 21, dtype=np.float32)  # ties at 1 + ulp/2
    with np.errstate(all="ignore"):
        s, p = a + b, a * b
    for i in range(len(a)):
        assert np.float32(add32(float(a[i]), float(b[i]))).tobytes() == s[i].tobytes()
        assert np.float32(mul32(float(a[i]), float(b[i]))).tobytes() == p[i].tobytes()
    # A fused multiply-add rounds once: (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24
    # is a binary32 value, while the rounded square (a tie at 2^-24) loses
    # the 2^-24.
    e = 1 + 2.0**-12
    assert fma32(e, e, -1.0) == 2.0**-11 + 2.0**-24
    assert add32(mul32(e, e), -1.0) == 2.0**-11


def test_cases_discriminate_each_slip(cases):
    for name, (c, s, h) in cases.items():
        right = right_order(c, s, h)
        wrong = WRONG_ORDERS[name](c, s, h)
        assert e4m3_code(right) != e4m3_code(wrong), name
        assert c in (3.25, -2.25, 2.25, -3.25)


def test_oracle_follows_the_order_on_hand_built_cases(orc, cases):
    x, sc, sh, cols = case_row(cases)
    out, mean, rstd, y = orc.adaln_fp8_f32ops(x, sc, sh, ACT_SCALE, eps=0.0, want_y=True)
    assert mean[0] == 0.0 and rstd[0] == 0.25
    # Every column follows the exact model, bit for bit.
    xhat = f32(x[0]) / np.float32(4.0)
    for j in range(x.shape[1]):
        want = right_order(float(xhat[j]), float(sc[0, j]), float(sh[0, j]))
        assert np.float32(want).tobytes() == y[0, j].tobytes(), j
        assert out[0, j] == e4m3_code(want), j
    # At each case's column the code is not the slip's.
    for name, j in cols.items():
        c, s, h = cases[name]
        assert out[0, j] != e4m3_code(WRONG_ORDERS[name](c, s, h)), name


def test_table_form_follows_the_order(orc, cases):
    """The table form's operand is temb chunk + table row (one fp32 add); with
    a zero temb it is the table row itself, so the same cases pass through
    the table entry unchanged."""
    x, sc, sh, _ = case_row(cases)
    dim = x.shape[1]
    temb = np.zeros((1, 2, dim), np.uint16)
    table = np.stack([sh[0], sc[0]]).astype(np.float32)    # shift_idx 0, scale_idx 1
    a = orc.adaln_fp8_table(x, temb, table, 0, 1, ACT_SCALE, eps=0.0, want_y=True)
    b = orc.adaln_fp8_f32ops(x, sc, sh, ACT_SCALE, eps=0.0, want_y=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_random_rows_follow_the_order(orc):
    """Per-token rows: the oracle's y equals numpy's float32 sequence (one
    rounding per ufunc), from the oracle's mean and rstd.  The data are
    sensitive: a fused last step changes y in many elements."""
    d = inputs.make("ptok", rows=48, dim=3072, seed=21)
    out, mean, rstd, y = orc.adaln_fp8_ptok(d["x"], d["scale"], d["shift"], ACT_SCALE,
                                            want_y=True)
    xf, scf, shf = f32(d["x"]), f32(d["scale"]), f32(d["shift"])
    xhat = (xf - mean[:, None]) * rstd[:, None]
    t = np.float32(1.0) + scf
    u = xhat * t
    want = u + shf
    assert want.dtype == np.float32
    assert np.array_equal(want.view(np.uint32), y.view(np.uint32))
    # u + shift with one rounding: the product is exact in float64, so the
    # fused value is float32(u_exact + shift) up to float64's own rounding.
    fused = (xhat.astype(np.float64) * t.astype(np.float64) + shf.astype(np.float64)).astype(np.float32)
    assert np.count_nonzero(fused != want) > 1000
    # And the codes are the e4m3 conversion of y * 40.
    v = y * np.float32(40.0)
    inr = np.abs(v) < 448
    import torch
    codes = torch.from_numpy(np.ascontiguousarray(v[inr])).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(out[inr], codes)


def test_block_statistics_are_exact():
    """The hand-built block's closed forms: mean 0, biased variance 16."""
    assert BLOCK.sum() == 0
    assert float((BLOCK.astype(np.float64) ** 2).mean()) == 16.0
    assert 1.0 / math.sqrt(16.0) == 0.25
