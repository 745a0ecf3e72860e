"""Parity of the LN -> FP4 producer with the oracle through the C ABI: packed
e2m1 codes and e4m3 block scales, small and ragged shapes, the full
4096 x 3072 outlier workload on every row, the fallback kernel, and
batch invariance."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import (assert_codes_close, assert_stats_close, dev_bf16, e2m1_ordinal,
                    e4m3_ordinal, host_u8, misaligned_like, unpack_e2m1)

pytestmark = pytest.mark.gpu


def run_gpu(xb, rows, dim, x=None):
    x = dev_bf16(xb) if x is None else x
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x, row_mean=mean, row_rstd=rstd)
    return host_u8(packed), host_u8(sf), mean.cpu().numpy(), rstd.cpu().numpy()


def check(got, ref, what):
    gp, gs, gm, gr = got
    rp, rs, rm, rr = ref[:4]
    assert_codes_close(unpack_e2m1(gp), unpack_e2m1(rp), e2m1_ordinal, what + " codes")
    assert_codes_close(gs, rs, e4m3_ordinal, what + " scales")
    assert_stats_close(gm, gr, rm, rr)


@pytest.mark.parametrize("rows,dim", [(1, 3072), (7, 16), (16, 2048), (65, 1536), (63, 1152),
                                      (9, 5376), (3, 8192), (5, 48), (3, 8208), (2, 12016),
                                      (2, 20480), (1, 32768), (2, 32784)])
def test_small_shapes(orc, rows, dim):
    print(f"fp4 rows={rows} dim={dim}", flush=True)
    d = inputs.make("fp4", rows=rows, dim=dim, seed=rows + dim)
    check(run_gpu(d["x"], rows, dim), orc.ln_fp4(d["x"]), f"{rows}x{dim}")


def test_full_size_workload(orc):
    d = inputs.workload("ln_fp4_4096x3072")
    rows, dim = d["x"].shape
    got = run_gpu(d["x"], rows, dim)
    ref = orc.ln_fp4(d["x"], threads=8)  # every row
    check(got, ref, "ln_fp4_4096x3072")


def test_unaligned_uses_fallback(orc):
    rows, dim = 11, 3072
    d = inputs.make("fp4", rows=rows, dim=dim, seed=3)
    x = misaligned_like((rows, dim), torch.bfloat16)
    x.copy_(dev_bf16(d["x"]))
    check(run_gpu(d["x"], rows, dim, x=x), orc.ln_fp4(d["x"]), "unaligned")


def test_degenerate_rows(orc):
    rows, dim = 3, 256
    x = np.zeros((rows, dim), np.float32)
    x[1] = 0.75                                   # constant -> all zero
    x[2, ::2], x[2, 1::2] = 1.5, -1.5             # +-1 -> 0xF7 bytes
    xb = inputs.to_bf16_bits(x)
    got = run_gpu(xb, rows, dim)
    ref = orc.ln_fp4(xb)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    assert np.all(got[0][2] == 0xF7) and np.all(got[1][2] == 0x23)


def test_batch_invariance_and_determinism():
    d = inputs.make("fp4", rows=1024, dim=3072, seed=4)
    x = dev_bf16(d["x"])
    p1, s1 = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x)
    p2, s2 = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x)
    p1, s1 = host_u8(p1), host_u8(s1)
    assert np.array_equal(p1, host_u8(p2)) and np.array_equal(s1, host_u8(s2))
    for bs in (1, 5, 64, 129):
        for r0 in (0, 511, 1024 - bs):
            p, s = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x[r0:r0 + bs])
            assert np.array_equal(host_u8(p), p1[r0:r0 + bs])
            assert np.array_equal(host_u8(s), s1[r0:r0 + bs])


def test_zero_eps_constant_row(orc):
    """eps = 0 and a constant row: xhat = 0 * inf is NaN at every element, the
    staged block maximum ignores NaN and is 0, so every block scale is code 0
    and every code 0 (the zero-scale rule), on both sides bit for bit; the
    other rows as usual."""
    rows, dim = 4, 3072
    d = inputs.make("fp4", rows=rows, dim=dim, seed=22)
    x = d["x"].copy()
    x[2] = inputs.to_bf16_bits(np.full(dim, -1.25, np.float32))
    packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(dev_bf16(x), eps=0.0)
    got = (host_u8(packed), host_u8(sf))
    ref = orc.ln_fp4(x, eps=0.0)
    assert np.all(got[0][2] == 0) and np.all(got[1][2] == 0)
    assert np.array_equal(got[0][2], ref[0][2]) and np.array_equal(got[1][2], ref[1][2])
    keep = [0, 1, 3]
    assert_codes_close(unpack_e2m1(got[0][keep]), unpack_e2m1(ref[0][keep]), e2m1_ordinal,
                       "eps 0 codes")
    assert_codes_close(got[1][keep], ref[1][keep], e4m3_ordinal, "eps 0 scales")
