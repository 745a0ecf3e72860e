"""Extents of the launch mapping, against the oracle through the C ABI: row
counts past the 65535 workgroups one grid dimension holds (the row kernels
then use a second grid dimension; the table form and the RMSNorm producer's
span kernel hold two rows per workgroup); token and row counts past 4 x 65535
for the six-way producer and the residual gate, which map four per thread
onto two grid dimensions and then need the third; and rows of 2^20 elements,
which go to the workgroup-per-row fallback.  Rows on both sides of each
boundary are checked."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import (act, assert_codes_close, assert_stats_close, dev_bf16, dev_f32, e2m1_ordinal,
                    e4m3_ordinal, host_u8, host_u16, unpack_e2m1)

pytestmark = pytest.mark.gpu

GRID_X = 65535


def boundary_rows(rows, per_group=1):
    """Rows at the first grid-row boundary (in workgroups of per_group rows),
    the first and the last rows."""
    edge = GRID_X * per_group
    picks = [0, 1, edge - 2, edge - 1, edge, edge + 1, rows - 2, rows - 1]
    return np.unique([r for r in picks if 0 <= r < rows])


@pytest.mark.parametrize("kind,rows", [("ptok", 70001), ("table", 140003), ("ln", 70001)])
def test_fp8_rows_past_one_grid_dimension(orc, kind, rows):
    dim = 64
    print(f"fp8 {kind} rows={rows} dim={dim}", flush=True)
    d = inputs.make(kind, rows=rows, dim=dim, seed=5)
    x = dev_bf16(d["x"])
    a = act(d["act_scale"])
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    if kind == "ptok":
        o = alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]),
                                                    a, row_mean=mean, row_rstd=rstd)
        sel = boundary_rows(rows)
        ref = orc.adaln_fp8_ptok(d["x"][sel], d["scale"][sel], d["shift"][sel], d["act_scale"])
    elif kind == "table":
        o = alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(
            x, dev_bf16(d["temb"]), dev_f32(d["table"]), a, d["shift_idx"], d["scale_idx"],
            row_mean=mean, row_rstd=rstd)
        sel = boundary_rows(rows, per_group=2)
        ref = orc.adaln_fp8_table(d["x"][sel], d["temb"][sel], d["table"], d["shift_idx"],
                                  d["scale_idx"], d["act_scale"])
    else:
        o = alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, a, row_mean=mean, row_rstd=rstd)
        sel = boundary_rows(rows)
        ref = orc.ln_fp8(d["x"][sel], d["act_scale"])
    got = host_u8(o)
    assert_codes_close(got[sel], ref[0], e4m3_ordinal, f"{kind} {rows} rows")
    assert_stats_close(mean.cpu().numpy()[sel], rstd.cpu().numpy()[sel], ref[1], ref[2])


def test_fp4_rows_past_one_grid_dimension(orc):
    rows, dim = 70001, 64
    d = inputs.make("fp4", rows=rows, dim=dim, seed=6)
    packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(dev_bf16(d["x"]))
    sel = boundary_rows(rows)
    rp, rs = orc.ln_fp4(d["x"][sel])[:2]
    assert_codes_close(unpack_e2m1(host_u8(packed)[sel]), unpack_e2m1(rp), e2m1_ordinal, "fp4 codes")
    assert_codes_close(host_u8(sf)[sel], rs, e4m3_ordinal, "fp4 scales")


@pytest.mark.parametrize("rows", [70001, 140003])
def test_rmsmod_rows_past_one_grid_dimension(orc, rows):
    # Two rows per workgroup from 4096 rows: 140003 rows need a second grid
    # dimension, 70001 rows do not.
    dim = 64
    print(f"rmsmod rows={rows} dim={dim}", flush=True)
    d = inputs.make("rmsmod", rows=rows, dim=dim, seed=7)
    o = alnp.rms_norm_modulate_seg_bf16(dev_bf16(d["x"]), dev_bf16(d["weight"]),
                                        dev_bf16(d["scale"]), dev_bf16(d["shift"]),
                                        torch.from_numpy(d["seg"]).cuda())
    sel = boundary_rows(rows, per_group=2)
    ref = orc.rms_modulate_seg(d["x"][sel], d["weight"], d["scale"], d["shift"], d["seg"][sel])[0]
    got = host_u16(o)[sel]
    assert np.mean(got == ref) >= 0.999


@pytest.mark.parametrize("kind", ["ptok", "ln"])
def test_fp8_rows_of_2_pow_20(orc, kind):
    rows, dim = 2, 1 << 20
    d = inputs.make(kind, rows=rows, dim=dim, seed=8)
    x = dev_bf16(d["x"])
    a = act(d["act_scale"])
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    if kind == "ptok":
        o = alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]),
                                                    a, row_mean=mean, row_rstd=rstd)
        ref = orc.adaln_fp8_ptok(d["x"], d["scale"], d["shift"], d["act_scale"])
    else:
        o = alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, a, row_mean=mean, row_rstd=rstd)
        ref = orc.ln_fp8(d["x"], d["act_scale"])
    assert_codes_close(host_u8(o), ref[0], e4m3_ordinal, f"{kind} 2 x 2^20")
    assert_stats_close(mean.cpu().numpy(), rstd.cpu().numpy(), ref[1], ref[2])


def test_fp4_and_rmsmod_rows_of_2_pow_20(orc):
    rows, dim = 2, 1 << 20
    f = inputs.make("fp4", rows=rows, dim=dim, seed=9)
    packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(dev_bf16(f["x"]))
    rp, rs = orc.ln_fp4(f["x"])[:2]
    assert_codes_close(unpack_e2m1(host_u8(packed)), unpack_e2m1(rp), e2m1_ordinal, "fp4 2^20")
    assert_codes_close(host_u8(sf), rs, e4m3_ordinal, "fp4 scales 2^20")
    r = inputs.make("rmsmod", rows=rows, dim=dim, seed=10)
    o = alnp.rms_norm_modulate_seg_bf16(dev_bf16(r["x"]), dev_bf16(r["weight"]),
                                        dev_bf16(r["scale"]), dev_bf16(r["shift"]),
                                        torch.from_numpy(r["seg"]).cuda())
    ref = orc.rms_modulate_seg(r["x"], r["weight"], r["scale"], r["shift"], r["seg"])[0]
    assert np.mean(host_u16(o) == ref) >= 0.999


# Six-way modulation and the residual gate give each thread four tokens
# (rows) and spread the groups over (blockIdx.y, blockIdx.z): from 4 * 65535
# = 262140 tokens the third grid dimension is used.  262147: a second z
# slice holding one partial group.  Bit-exact, compared in full.
def test_modulation6_tokens_past_two_grid_dimensions(orc):
    B, S, D = 1, 262147, 16
    print(f"mod6 B={B} S={S} D={D}", flush=True)
    d = inputs.make("mod6", batch=B, seq=S, dim=D, seed=10)
    outs = alnp.adaln_modulation6_bf16(dev_f32(d["params"]), dev_f32(d["mod"]))
    got = np.stack([host_u16(o) for o in outs])
    assert np.array_equal(got, orc.modulation6(d["params"], d["mod"]))


@pytest.mark.parametrize("bcast", [False, True])
def test_gated_residual_rows_past_two_grid_dimensions(orc, bcast):
    rows, dim = 262147, 16
    print(f"gated residual rows={rows} dim={dim} bcast={bcast}", flush=True)
    res = inputs.normal_bf16((rows, dim), 1.0, 11, 1)
    gate = inputs.normal_bf16((dim,) if bcast else (rows, dim), 0.5, 11, 2)
    proj = inputs.normal_bf16((rows, dim), 2.0, 11, 3)
    out = alnp.gated_residual_bf16(dev_bf16(res), dev_bf16(gate), dev_bf16(proj))
    assert np.array_equal(host_u16(out), orc.gated_residual(res, gate, proj))


def test_standalone_quantizer_at_its_limit(orc):
    """quant_fp8_static_f32 takes up to 2^31 values (one thread each, 2^23
    workgroups): the values past 2^31 - 2^8 and a sample of the rest against
    the oracle's encoder.  The input is drawn on the GPU (8 GiB)."""
    n = 1 << 31
    print(f"quant fp8 n={n}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(12)
    v = torch.randn(n, generator=g, device="cuda") * 4.0
    a = act(0.025)
    out = alnp.quant_fp8_static_f32(v, a)
    rng = np.random.default_rng(12)
    idx = np.unique(np.concatenate([rng.integers(0, n, 4096), np.arange(n - 256, n), [0, 1]]))
    it = torch.from_numpy(idx).cuda()
    vs = v[it].cpu().numpy()
    got = out.view(torch.uint8)[it].cpu().numpy()
    del v, out
    torch.cuda.empty_cache()
    ref = orc.e4m3_encode_sat(vs * np.float32(1.0 / np.float32(0.025)))
    assert np.array_equal(got, ref)


def test_empty_calls_leave_outputs_untouched():
    """rows = 0 (tokens = 0, n = 0) is a no-op through the C ABI: status 0,
    and output buffers sized for one row keep their sentinel bytes."""
    import ctypes
    L = alnp.lib()
    dim = 3072
    print("empty calls through the C ABI", flush=True)
    dev = lambda n, dt: torch.zeros(n, dtype=dt, device="cuda")
    x = dev(dim, torch.bfloat16)
    sc = dev(dim, torch.bfloat16)
    sh = dev(dim, torch.bfloat16)
    temb = dev(6 * dim, torch.bfloat16)
    table = dev(6 * dim, torch.float32)
    act = torch.tensor([0.025], dtype=torch.float32, device="cuda")
    seg = torch.zeros(1, dtype=torch.int32, device="cuda")
    sentinel = lambda n: torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    out8, packed, sf, mxs = sentinel(dim), sentinel(dim // 2), sentinel(512), sentinel(dim // 32)
    out16 = sentinel(2 * dim)
    stats = sentinel(8)
    m6 = [sentinel(2 * dim) for _ in range(6)]
    arr = (ctypes.c_void_p * 6)(*[o.data_ptr() for o in m6])
    p = lambda t: t.data_ptr()
    h = torch.cuda.current_stream().cuda_stream
    calls = [
        L.alnp_ada_layer_norm_quant_fp8_bf16(p(x), p(sc), p(sh), p(act), 1e-5, 0, dim, p(out8),
                                             p(stats), p(stats), h),
        L.alnp_ada_layer_norm_quant_fp8_ptok_bf16(p(x), p(sc), p(sh), p(act), 1e-5, 0, dim,
                                                  p(out8), p(stats), p(stats), h),
        L.alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(p(x), p(temb), p(table), 6, 0, 1, p(act),
                                                        1e-5, 0, dim, p(out8), p(stats),
                                                        p(stats), h),
        L.alnp_layer_norm_no_affine_quant_fp8_static_bf16(p(x), p(act), 1e-5, 0, dim, p(out8),
                                                          p(stats), p(stats), h),
        L.alnp_layer_norm_no_affine_quant_nvfp4_bf16(p(x), 1e-5, 0, dim, p(packed), p(sf),
                                                     p(stats), p(stats), h),
        L.alnp_layer_norm_no_affine_quant_mxfp8_bf16(p(x), 1e-5, 0, dim, p(out8), p(mxs),
                                                     p(stats), p(stats), h),
        L.alnp_layer_norm_no_affine_quant_mxfp4_bf16(p(x), 1e-5, 0, dim, p(packed), p(mxs),
                                                     p(stats), p(stats), h),
        L.alnp_adaln_modulation6_bf16(p(table), p(table), 1, 0, dim, arr, h),
        L.alnp_gated_residual_bf16(p(x), p(x), p(x), 0, dim, 1, p(out16), h),
        L.alnp_rms_norm_modulate_seg_bf16(p(x), p(x), p(sc), p(sh), p(seg), 1, 1e-5, 0, dim,
                                          p(out16), p(stats), h),
        L.alnp_quant_fp8_static_f32(p(table), p(act), 0, p(out8), h),
    ]
    torch.cuda.synchronize()
    assert calls == [0] * len(calls), calls
    for buf in (out8, packed, sf, mxs, out16, stats, *m6):
        assert bool((buf == 0xA5).all())
