"""Exact binary32 arithmetic for pinning the modulation sequence.

Each operation is computed exactly on rationals (fractions.Fraction) and
rounded once to the nearest binary32 value, ties to the even significand,
with IEEE 754's sign rules for exact zeros.  This is the textbook definition
of a correctly rounded fp32 operation, written independently of both the
oracle and the HIP kernels; `tests/test_oracle_modulation_order.py` checks
it against numpy's float32 arithmetic.

The modulation order to pin is (xhat * (scale + 1)) + shift, every step one
rounded fp32 operation (h3-blackwell-runtime page, "NVFP4 Modulation
Producer Fusion" -> "Exactness Contract"; the FP8 path keeps the value in
fp32 until the e4m3 conversion).  `WRONG_ORDERS` lists plausible slips in
that sequence, and `find_case` builds, for one of them, an (xhat, scale,
shift) triple whose e4m3 code under act_scale 0.025 differs between the
right order and the slip.  A random search almost never finds such a case
(a one-ulp change of y moves the code with probability ~2^-20), so the
search aims at it: it puts xhat * t right beside an fp32 value y0 whose code
differs from its neighbour's, then tries small shifts.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction as Q

import numpy as np
import torch

ACT_SCALE = 0.025   # 1 / 0.025f is exactly 40.0f


def rn32(q: Q) -> float:
    """Nearest binary32 value to the non-zero rational q, ties to even;
    +-inf past the largest finite value."""
    assert q != 0
    sign = -1.0 if q < 0 else 1.0
    m = abs(q)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if m < Q(2) ** e:
        e -= 1                                   # 2^e <= m < 2^(e+1)
    quantum = Q(2) ** (max(e, -126) - 23)        # subnormal spacing below 2^-126
    k = m / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Q(1, 2) or (rem == Q(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Q(2) ** 128:
        return sign * math.inf
    return sign * float(v)                       # exact: v is a binary32 value


def _neg(v: float) -> bool:
    return math.copysign(1.0, v) < 0


def add32(a: float, b: float) -> float:
    s = Q(a) + Q(b)
    if s == 0:       # round to nearest: +0 unless both operands are -0
        return -0.0 if (_neg(a) and _neg(b)) else 0.0
    return rn32(s)


def mul32(a: float, b: float) -> float:
    p = Q(a) * Q(b)
    if p == 0:
        return -0.0 if _neg(a) != _neg(b) else 0.0
    return rn32(p)


def fma32(a: float, b: float, c: float) -> float:
    """a * b + c with one rounding (the fused form the contract excludes)."""
    s = Q(a) * Q(b) + Q(c)
    if s == 0:
        return -0.0 if ((_neg(a) != _neg(b)) and _neg(c)) else 0.0
    return rn32(s)


def bf16_round(v: float) -> float:
    """Nearest bf16 value (8-bit significand), ties to even, of a finite
    binary32 value: rn32's rule at a coarser quantum."""
    if v == 0:
        return v
    q = Q(v)
    sign = -1.0 if q < 0 else 1.0
    m = abs(q)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if m < Q(2) ** e:
        e -= 1
    quantum = Q(2) ** (max(e, -126) - 7)
    k = m / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Q(1, 2) or (rem == Q(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * quantum)


def right_order(xhat: float, sc: float, sh: float) -> float:
    """y = (xhat * (1 + sc)) + sh, three rounded fp32 operations."""
    return add32(mul32(xhat, add32(1.0, sc)), sh)


WRONG_ORDERS = {
    # u + shift fused into one rounding with the product
    "fused_multiply_add": lambda c, sc, sh: fma32(c, add32(1.0, sc), sh),
    # xhat + xhat * scale + shift, each rounded
    "expanded": lambda c, sc, sh: add32(add32(c, mul32(c, sc)), sh),
    # xhat + xhat * scale as one fused operation, then + shift
    "expanded_fused": lambda c, sc, sh: add32(fma32(c, sc, c), sh),
    # 1 + scale not rounded before the product
    "unrounded_one_plus_scale": lambda c, sc, sh: add32(rn32(Q(c) * (1 + Q(sc))), sh),
    # the product rounded to bf16 before the shift (a bf16 tensor step)
    "bf16_product": lambda c, sc, sh: add32(bf16_round(mul32(c, add32(1.0, sc))), sh),
    # shift applied before the scale
    "shift_then_scale": lambda c, sc, sh: mul32(add32(c, sh), add32(1.0, sc)),
}


def e4m3_code(y: float) -> int:
    """Code of y * (1 / act_scale) = y * 40 (one fp32 multiplication) by
    torch's float8_e4m3fn conversion (round to nearest even)."""
    v = np.float32(mul32(y, 40.0))
    t = torch.from_numpy(np.array([v], np.float32)).to(torch.float8_e4m3fn)
    return int(t.view(torch.uint8)[0])


def _f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def _bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _code_boundaries(v_lo: float, v_hi: float):
    """Pairs (y0, y1) of adjacent positive fp32 values whose codes differ,
    one per e4m3 rounding midpoint m with v_lo <= m <= v_hi."""
    vals = sorted(float(torch.tensor([i], dtype=torch.uint8).view(torch.float8_e4m3fn).float())
                  for i in range(0x7F))
    out = []
    for a, b in zip(vals, vals[1:]):
        m = (a + b) / 2
        if not v_lo <= m <= v_hi:
            continue
        lo = _f32_bits(float(np.float32(m / 40.0))) - 64
        c0 = e4m3_code(_bits_f32(lo))
        while e4m3_code(_bits_f32(lo + 1)) == c0:
            lo += 1
        out.append((_bits_f32(lo), _bits_f32(lo + 1)))
    return out


def find_case(wrong, xhats=(3.25, -2.25, 2.25, -3.25)):
    """(xhat, scale, shift) with xhat from `xhats` whose code differs between
    right_order and `wrong`, or None.  Deterministic.  For each code boundary
    (y0, y1) and each xhat, t = 1 + scale runs over the fp32 grid near
    y/xhat (scale also one to three ulps off the exact t - 1, so that 1 +
    scale itself rounds), and shift over eighths of y's ulp."""
    for c in xhats:
        for y0, y1 in _code_boundaries(60.0, 440.0):
            for target in (y0, y1):
                target = math.copysign(target, c)
                tc = target / c
                if not 0.5 < tc < 2.0:
                    continue
                ut = 2.0 ** (math.floor(math.log2(tc)) - 23)
                base = round(tc / ut)
                for dj in range(-4, 5):
                    sc0 = add32((base + dj) * ut, -1.0)
                    us = 2.0 ** (math.floor(math.log2(abs(sc0))) - 23)
                    for ks in (0, -1, 1, -2, 2, -3, 3):
                        sc = sc0 + ks * us
                        uy = 2.0 ** (math.floor(math.log2(abs(target))) - 23)
                        for k in range(-12, 13):
                            sh = k * uy / 8
                            if e4m3_code(right_order(c, sc, sh)) != e4m3_code(wrong(c, sc, sh)):
                                return c, sc, sh
    return None
