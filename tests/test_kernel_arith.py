"""Host-side checks of arithmetic substitutions the HIP kernels make, each
proved against the oracle's definition over every input it can see.

The FP4 block scale is defined as s = e4m3(amax / 6) with an IEEE division
(block-scale rule of the h3-blackwell-runtime page,
benchmarks/gb10-cute-p1-stream-a-summary.json, "numerical_contract"; global
scale 1).  The kernel multiplies by RN(1/6) instead.  amax is the largest
magnitude of bf16-staged values, so it is itself a bf16 value: checking all
32,768 non-negative bf16 patterns covers every case.
"""
import numpy as np


def test_fp4_scale_multiply_equals_division_for_every_bf16_amax(orc):
    b = np.arange(0x8000, dtype=np.uint32)
    amax = (b << 16).view(np.float32)
    amax = amax[np.isfinite(amax)]
    by_div = orc.e4m3_encode_sat(np.minimum(amax / np.float32(6.0), np.float32(448.0)))
    by_mul = orc.e4m3_encode_sat(np.minimum(amax * (np.float32(1.0) / np.float32(6.0)),
                                            np.float32(448.0)))
    assert np.array_equal(by_div, by_mul)
    # The quotients themselves do differ, so the check is not vacuous.
    assert np.any(amax / np.float32(6.0) != amax * (np.float32(1.0) / np.float32(6.0)))


def test_fp4_reciprocal_table_is_ieee_division(orc):
    """The kernel tabulates 1/s per e4m3 code at compile time (constant
    evaluation divides in IEEE binary32, round to nearest even), the division
    the oracle performs per block; s values are exact in fp32.  On the GPU,
    an input reaching every scale code checks the table against the oracle."""
    codes = np.arange(1, 127, dtype=np.uint8)
    s = orc.e4m3_decode(codes)
    assert np.array_equal(s.astype(np.float32).astype(np.float64), s)
    inv = np.float32(1.0) / s.astype(np.float32)
    assert np.all(np.isfinite(inv)) and inv.max() == 512.0
