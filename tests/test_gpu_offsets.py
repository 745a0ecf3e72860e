"""Calls past 2^31 and 2^32 elements, where every offset a kernel forms from
a row or token index must be 64-bit: LN->FP8, per-token and table AdaLN->FP8,
LN->NVFP4 and LN->MXFP8 at 1 398 102 x 3072 (4.29e9 elements; the table
form's temb holds 8.6e9), RMSNorm modulation at 798 916 x 5376, the six-way
producer at 233 017 tokens (4.29e9 fp32 parameters) and the residual gate at
1 398 102 x 3072.  The inputs are drawn on the GPU (inputs.device_normal);
the rows that hold elements 2^31 and 2^32, their neighbours, and the first
and last rows are copied to the host and checked against the oracle, at the
tolerances of the other parity tests.  Each case needs 13-35 GB of device
memory and frees it before the next."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import act, assert_codes_close, assert_stats_close, e2m1_ordinal, e4m3_ordinal, unpack_e2m1
from test_gpu_mx import assert_mx_close

pytestmark = pytest.mark.gpu

DIM = 3072
ROWS = (1 << 32) // DIM + 1          # 1 398 102 rows: element 2^32 sits in the last row
RMS_DIM = 5376
RMS_ROWS = (1 << 32) // RMS_DIM + 1  # 798 916 rows
SEED = 31


def offset_rows(rows, dim):
    """Rows holding elements 2^31 and 2^32 (of a (rows, dim) tensor), their
    neighbours, and the first and last rows."""
    picks = [0, 1, rows - 2, rows - 1]
    for e in (1 << 31, 1 << 32):
        r = e // dim
        picks += [r - 1, r, r + 1]
    return np.unique([r for r in picks if 0 <= r < rows])


def host_rows(t, sel, np_dtype):
    """Rows `sel` of a device tensor, as host numpy with the given bit view."""
    idx = torch.from_numpy(sel).to(t.device)
    v = t.index_select(0, idx).contiguous()
    if v.dtype == torch.bfloat16:
        return v.view(torch.int16).cpu().numpy().view(np.uint16)
    if v.dtype in (torch.float8_e4m3fn, torch.uint8):
        return v.view(torch.uint8).cpu().numpy()
    return v.cpu().numpy().astype(np_dtype)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(autouse=True)
def _release():
    yield
    free()


def stats(rows):
    return (torch.empty(rows, dtype=torch.float32, device="cuda"),
            torch.empty(rows, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("form", ["ln", "ptok", "table"])
def test_fp8_past_2_pow_32_elements(orc, form):
    print(f"fp8 {form} rows={ROWS} dim={DIM}", flush=True)
    sel = offset_rows(ROWS, DIM)
    x = inputs.device_normal((ROWS, DIM), 1.0, SEED, inputs.STREAM["x"])
    a = act(inputs.ACT_SCALE)
    mean, rstd = stats(ROWS)
    xs = host_rows(x, sel, None)
    if form == "ln":
        out = alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, a, row_mean=mean, row_rstd=rstd)
        ref = orc.ln_fp8(xs, inputs.ACT_SCALE)
    elif form == "ptok":
        sc = inputs.device_normal((ROWS, DIM), 0.1, SEED, inputs.STREAM["scale"])
        sh = inputs.device_normal((ROWS, DIM), 0.1, SEED, inputs.STREAM["shift"])
        out = alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, sc, sh, a, row_mean=mean, row_rstd=rstd)
        ref = orc.adaln_fp8_ptok(xs, host_rows(sc, sel, None), host_rows(sh, sel, None),
                                 inputs.ACT_SCALE)
        del sc, sh
    else:
        # Two temb chunks keep the call at 17 GB of temb; the kernel is the
        # two-row LDS table kernel (more than 512 rows).
        temb = inputs.device_normal((ROWS, 2, DIM), 0.5, SEED, inputs.STREAM["temb"])
        table = inputs.normal_f32((2, DIM), 0.1, SEED, inputs.STREAM["table"])
        out = alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(
            x, temb, torch.from_numpy(table).cuda(), a, 0, 1, row_mean=mean, row_rstd=rstd)
        ref = orc.adaln_fp8_table(xs, host_rows(temb, sel, None), table, 0, 1, inputs.ACT_SCALE)
        del temb
    got = host_rows(out, sel, None)
    assert_codes_close(got, ref[0], e4m3_ordinal, f"{form} {ROWS}x{DIM}")
    assert_stats_close(host_rows(mean, sel, np.float32), host_rows(rstd, sel, np.float32),
                       ref[1], ref[2])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp8"])
def test_block_formats_past_2_pow_32_elements(orc, fmt):
    print(f"{fmt} rows={ROWS} dim={DIM}", flush=True)
    sel = offset_rows(ROWS, DIM)
    x = inputs.device_normal((ROWS, DIM), 1.0, SEED, inputs.STREAM["x"])
    xs = host_rows(x, sel, None)
    if fmt == "nvfp4":
        packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x)
        rp, rs = orc.ln_fp4(xs)[:2]
        assert_codes_close(unpack_e2m1(host_rows(packed, sel, None)), unpack_e2m1(rp),
                           e2m1_ordinal, "nvfp4 codes")
        assert_codes_close(host_rows(sf, sel, None), rs, e4m3_ordinal, "nvfp4 scales")
    else:
        out, scales = alnp.layer_norm_no_affine_quant_mxfp8_bf16(x)
        rc, rsc, _, _, ry = orc.adaln_mxfp8(xs, want_y=True)
        assert_mx_close(host_rows(out, sel, None), host_rows(scales.view(ROWS, DIM // 32), sel, None),
                        rc, rsc, ry, e4m3_ordinal, "mxfp8")


def test_rmsmod_past_2_pow_32_elements(orc):
    print(f"rmsmod rows={RMS_ROWS} dim={RMS_DIM}", flush=True)
    sel = offset_rows(RMS_ROWS, RMS_DIM)
    small = inputs.make("rmsmod", rows=4, dim=RMS_DIM, seed=SEED)
    x = inputs.device_normal((RMS_ROWS, RMS_DIM), 1.0, SEED, inputs.STREAM["x"])
    seg = inputs.segment_ids(RMS_ROWS, 3, "h3", SEED)
    out = alnp.rms_norm_modulate_seg_bf16(
        x, torch.from_numpy(small["weight"].view(np.int16)).cuda().view(torch.bfloat16),
        torch.from_numpy(small["scale"].view(np.int16)).cuda().view(torch.bfloat16),
        torch.from_numpy(small["shift"].view(np.int16)).cuda().view(torch.bfloat16),
        torch.from_numpy(seg).cuda())
    ref = orc.rms_modulate_seg(host_rows(x, sel, None), small["weight"], small["scale"],
                               small["shift"], seg[sel])[0]
    assert np.mean(host_rows(out, sel, None) == ref) >= 0.999


def test_modulation6_past_2_pow_32_parameters(orc):
    tokens = (1 << 32) // (6 * DIM) + 1   # 233 017 tokens, 4.29e9 fp32 parameters
    print(f"mod6 tokens={tokens} dim={DIM}", flush=True)
    params = inputs.device_normal((1, tokens, 6, DIM), 1.0, SEED, inputs.STREAM["params"],
                                  dtype=torch.float32)
    mod = inputs.normal_f32((6, DIM), 0.1, SEED, inputs.STREAM["mod"])
    outs = alnp.adaln_modulation6_bf16(params, torch.from_numpy(mod).cuda())
    sel = offset_rows(tokens, 6 * DIM)
    ps = host_rows(params[0], sel, np.float32)[None]
    ref = orc.modulation6(ps, mod)
    got = np.stack([host_rows(o[0], sel, None) for o in outs])
    assert np.array_equal(got, ref.reshape(got.shape))


def test_gated_residual_past_2_pow_32_elements(orc):
    print(f"gated residual rows={ROWS} dim={DIM}", flush=True)
    sel = offset_rows(ROWS, DIM)
    res = inputs.device_normal((ROWS, DIM), 1.0, SEED, 1)
    gate = inputs.device_normal((ROWS, DIM), 0.5, SEED, 2)
    proj = inputs.device_normal((ROWS, DIM), 2.0, SEED, 3)
    out = alnp.gated_residual_bf16(res, gate, proj)
    ref = orc.gated_residual(host_rows(res, sel, None), host_rows(gate, sel, None),
                             host_rows(proj, sel, None))
    assert np.array_equal(host_rows(out, sel, None), ref)
