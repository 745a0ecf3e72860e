"""The kernels' fp32 modulation order, pinned code by code.

The hand-built cases of tests/exact32.py (each (xhat, scale, shift) gives a
different e4m3 code under the right order (xhat * (scale + 1)) + shift than
under one plausible slip: a fused multiply-add, a re-associated or
expanded form, an unrounded 1 + scale, a bf16 product, shift before scale)
go through the table-form producers, the one operand form that takes fp32
operands (temb chunk 0 + fp32 table row = the table row).  The rows have
mean 0 and variance 16 exactly and eps = 0, so rstd = 1/4 on both sides and
the GPU's codes must equal the oracle's on every element, not only 99.9% of
them (h3-blackwell-runtime page, "NVFP4 Modulation Producer Fusion" ->
"Exactness Contract", for the order).  Both table kernels are covered: the
rows kernel (up to 512 rows) and the LDS kernel (from 513), with an odd row
count for the LDS kernel's half-filled last workgroup."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from exact32 import ACT_SCALE, WRONG_ORDERS, e4m3_code, find_case
from parity import act, dev_bf16, dev_f32, host_u8
from test_oracle_modulation_order import case_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cases():
    found = {name: find_case(fn) for name, fn in WRONG_ORDERS.items()}
    assert all(c is not None for c in found.values())
    return found


def table_inputs(cases, rows):
    x1, sc, sh, cols = case_row(cases)
    dim = x1.shape[1]
    x = np.ascontiguousarray(np.broadcast_to(x1, (rows, dim)))
    temb = np.zeros((rows, 2, dim), np.uint16)
    table = np.stack([sh[0], sc[0]]).astype(np.float32)   # shift_idx 0, scale_idx 1
    return x, temb, table, cols


@pytest.mark.parametrize("rows", [3, 512, 601])
def test_fp8_table_codes_exact(orc, cases, rows):
    x, temb, table, cols = table_inputs(cases, rows)
    dim = x.shape[1]
    print(f"modulation order fp8 table rows={rows} dim={dim}", flush=True)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    out = alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(
        dev_bf16(x), dev_bf16(temb), dev_f32(table), act(ACT_SCALE), 0, 1, eps=0.0,
        row_mean=mean, row_rstd=rstd)
    got = host_u8(out)
    assert np.all(mean.cpu().numpy() == 0.0)
    assert np.all(rstd.cpu().numpy() == 0.25)
    ref = orc.adaln_fp8_table(x, temb, table, 0, 1, ACT_SCALE, eps=0.0)[0]
    assert np.array_equal(got, ref)
    for name, j in cols.items():
        c, s, h = cases[name]
        assert np.all(got[:, j] != e4m3_code(WRONG_ORDERS[name](c, s, h))), name


@pytest.mark.parametrize("rows", [3, 601])
def test_mxfp8_table_codes_exact(orc, cases, rows):
    """The MXFP8 table producer evaluates the same y; with exact statistics
    its codes and block scales equal the oracle's everywhere."""
    x, temb, table, _ = table_inputs(cases, rows)
    dim = x.shape[1]
    print(f"modulation order mxfp8 table rows={rows} dim={dim}", flush=True)
    out, scales = alnp.ada_layer_norm_quant_mxfp8_ptok_table_bf16(
        dev_bf16(x), dev_bf16(temb), dev_f32(table), 0, 1, eps=0.0)
    ref, ref_sc = orc.adaln_mxfp8_table(x, temb, table, 0, 1, eps=0.0)[:2]
    assert np.array_equal(host_u8(out), ref)
    assert np.array_equal(host_u8(scales), ref_sc)
