"""Parity of the FP8 variants (modfp8, AWQ) and the FP4 variants (AdaLN->FP4,
128x4 tiled scales) with the oracle, through the C ABI: small and ragged
shapes (fast and fallback kernels), full Wan-size shapes on every row,
every finite e4m3 operand code, and the tiled layout's padding rules."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import (act, assert_codes_close, assert_stats_close, dev_bf16, e2m1_ordinal,
                    e4m3_ordinal, host_u8, misaligned_like, unpack_e2m1)

pytestmark = pytest.mark.gpu

SHAPES = [(1, 2048), (7, 3072), (63, 1536), (65, 1152), (9, 5376), (3, 8192), (5, 8),
          (4, 2), (5, 1030), (2, 12000), (2, 32768), (1, 40000)]
FP4_SHAPES = [(1, 3072), (7, 16), (65, 1536), (63, 1152), (9, 5376), (3, 8192), (5, 48),
              (3, 8208), (2, 20480), (2, 32784), (130, 3072), (129, 80)]


def e4m3_codes(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def dev_u8_as_fp8(u8):
    return torch.from_numpy(np.ascontiguousarray(u8)).cuda().view(torch.float8_e4m3fn)


def scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


# ---- modfp8 -------------------------------------------------------------------

def modfp8_inputs(rows, dim, seed):
    d = inputs.make("bcast", rows=rows, dim=dim, seed=seed)
    d["scale_fp8"] = e4m3_codes(inputs.normal_f32((dim,), 0.3, seed, 9))
    d["shift_fp8"] = e4m3_codes(inputs.normal_f32((dim,), 0.3, seed, 10))
    return d


def run_modfp8(d, sdeq, hdeq, x=None):
    rows, dim = d["x"].shape
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    o = alnp.ada_layer_norm_quant_fp8_modfp8_bf16(
        dev_bf16(d["x"]) if x is None else x, dev_u8_as_fp8(d["scale_fp8"]),
        dev_u8_as_fp8(d["shift_fp8"]), scalar(sdeq), scalar(hdeq), act(0.025),
        row_mean=mean, row_rstd=rstd)
    return host_u8(o), mean.cpu().numpy(), rstd.cpu().numpy()


@pytest.mark.parametrize("rows,dim", SHAPES)
def test_modfp8_shapes(orc, rows, dim):
    print(f"modfp8 rows={rows} dim={dim}", flush=True)
    d = modfp8_inputs(rows, dim, rows + dim)
    got, m, r = run_modfp8(d, 0.75, 1.5)
    ref, rm, rr, _ = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5, 0.025)
    assert_codes_close(got, ref, e4m3_ordinal, f"modfp8 {rows}x{dim}")
    assert_stats_close(m, r, rm, rr)


def test_modfp8_every_finite_operand_code(orc):
    dim = 2048
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    d = inputs.make("bcast", rows=16, dim=dim, seed=31)
    d["scale_fp8"] = np.resize(codes, dim).astype(np.uint8)
    d["shift_fp8"] = np.resize(codes[::-1], dim).astype(np.uint8)
    for sdeq, hdeq in ((1.0, 1.0), (0.01, 0.37), (2.0, 0.5)):
        got, _, _ = run_modfp8(d, sdeq, hdeq)
        ref = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], sdeq, hdeq, 0.025)[0]
        assert_codes_close(got, ref, e4m3_ordinal, f"modfp8 codes deq {sdeq}/{hdeq}")


def test_modfp8_full_size(orc):
    d = modfp8_inputs(2520, 3072, 32)
    got, m, r = run_modfp8(d, 1.0, 1.0)
    ref, rm, rr, _ = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 1.0, 1.0, 0.025,
                                          threads=8)  # every row
    assert_codes_close(got, ref, e4m3_ordinal, "modfp8 2520x3072")
    assert_stats_close(m, r, rm, rr)


def test_modfp8_unaligned_fallback(orc):
    d = modfp8_inputs(9, 3072, 33)
    x = misaligned_like((9, 3072), torch.bfloat16)
    x.copy_(dev_bf16(d["x"]))
    got, _, _ = run_modfp8(d, 0.5, 2.0, x=x)
    ref = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.5, 2.0, 0.025)[0]
    assert_codes_close(got, ref, e4m3_ordinal, "modfp8 unaligned")


# ---- AWQ --------------------------------------------------------------------------

def awq_inputs(rows, dim, seed):
    d = inputs.make("bcast", rows=rows, dim=dim, seed=seed)
    d["inv_s"] = inputs.to_bf16_bits(np.abs(inputs.normal_f32((dim,), 0.5, seed, 11)) + 0.5)
    return d


def run_awq(d, x=None):
    rows, dim = d["x"].shape
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    o = alnp.awq_ada_layer_norm_quant_fp8_bf16(
        dev_bf16(d["x"]) if x is None else x, dev_bf16(d["scale"]), dev_bf16(d["shift"]),
        dev_bf16(d["inv_s"]), act(0.025), row_mean=mean, row_rstd=rstd)
    return host_u8(o), mean.cpu().numpy(), rstd.cpu().numpy()


@pytest.mark.parametrize("rows,dim", SHAPES)
def test_awq_shapes(orc, rows, dim):
    print(f"awq rows={rows} dim={dim}", flush=True)
    d = awq_inputs(rows, dim, 3 * rows + dim)
    got, m, r = run_awq(d)
    ref, rm, rr, _ = orc.awq_adaln_fp8(d["x"], d["scale"], d["shift"], d["inv_s"], 0.025)
    assert_codes_close(got, ref, e4m3_ordinal, f"awq {rows}x{dim}")
    assert_stats_close(m, r, rm, rr)


def test_awq_unit_inv_s_equals_broadcast_bitwise():
    d = inputs.make("bcast", rows=300, dim=3072, seed=34)
    x, s, h = dev_bf16(d["x"]), dev_bf16(d["scale"]), dev_bf16(d["shift"])
    one = torch.ones(3072, dtype=torch.bfloat16, device="cuda")
    a = host_u8(alnp.awq_ada_layer_norm_quant_fp8_bf16(x, s, h, one, act()))
    b = host_u8(alnp.ada_layer_norm_quant_fp8_bf16(x, s, h, act()))
    assert np.array_equal(a, b)


# ---- AdaLN -> FP4 and tiled scales ---------------------------------------------------

def fp4_check(got_packed, got_sf, ref_packed, ref_sf, what):
    assert_codes_close(unpack_e2m1(got_packed), unpack_e2m1(ref_packed), e2m1_ordinal, what + " codes")
    assert_codes_close(got_sf, ref_sf, e4m3_ordinal, what + " scales")


def swizzled_positions(orc, rows, cols):
    return np.array([[orc.sf_swizzled_offset(r, c, cols) for c in range(cols)]
                     for r in range(rows)], np.int64)


@pytest.mark.parametrize("rows,dim", FP4_SHAPES)
def test_adaln_fp4_rowmajor_shapes(orc, rows, dim):
    print(f"adaln fp4 rows={rows} dim={dim}", flush=True)
    d = inputs.make("bcast", rows=rows, dim=dim, seed=rows + 5 * dim)
    packed, sf = alnp.ada_layer_norm_quant_nvfp4_bf16(dev_bf16(d["x"]), dev_bf16(d["scale"]),
                                                      dev_bf16(d["shift"]))
    rp, rs, _, _, _ = orc.adaln_fp4(d["x"], d["scale"], d["shift"])
    fp4_check(host_u8(packed), host_u8(sf), rp, rs, f"adaln fp4 {rows}x{dim}")


def test_adaln_fp4_every_scale_code(orc):
    # Per-block modulation factors 1 + scale log-spaced over 2^-8 .. 2^10 spread
    # the block maxima so that every e4m3 scale code 0..126 occurs (asserted on
    # the oracle's output), which exercises the kernel's 1/s for each code.
    rows, dim = 64, 4096
    d = inputs.make("bcast", rows=rows, dim=dim, seed=11)
    nb = dim // 16
    u = -8.0 + 18.0 * np.arange(nb) / (nb - 1)
    scale = inputs.to_bf16_bits(np.repeat(2.0 ** u - 1.0, 16).astype(np.float32))
    shift = np.zeros(dim, np.uint16)
    rp, rs, _, _, _ = orc.adaln_fp4(d["x"], scale, shift)
    assert set(np.unique(rs).tolist()) == set(range(127))
    packed, sf = alnp.ada_layer_norm_quant_nvfp4_bf16(dev_bf16(d["x"]), dev_bf16(scale), dev_bf16(shift))
    fp4_check(host_u8(packed), host_u8(sf), rp, rs, "every scale code")


def test_fp4_non_finite_rows(orc):
    # A NaN or an infinity in a row makes its statistics NaN; every block
    # maximum then ignores the NaN values, so the row gets zero scales and
    # zero codes, as in the oracle.  The other rows are unaffected.
    rows, dim = 4, 3072
    d = inputs.make("fp4", rows=rows, dim=dim, seed=12)
    xb = d["x"].copy()
    xb[1, 100] = 0x7FC0   # NaN
    xb[2, 7] = 0x7F80     # +inf
    xb[3, 3000] = 0xFF80  # -inf
    packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_bf16(dev_bf16(xb))
    rp, rs, _, _, _ = orc.ln_fp4(xb)
    gp, gs = host_u8(packed), host_u8(sf)
    assert np.all(rp[1:] == 0) and np.all(rs[1:] == 0)
    assert np.array_equal(gp[1:], rp[1:]) and np.array_equal(gs[1:], rs[1:])
    fp4_check(gp[:1], gs[:1], rp[:1], rs[:1], "finite row")


@pytest.mark.parametrize("mod", [False, True])
@pytest.mark.parametrize("rows,dim", [(1, 3072), (130, 3072), (129, 80), (7, 48), (2, 32784),
                                      (300, 1536)])
def test_fp4_swizzled_layout(orc, mod, rows, dim):
    print(f"fp4 swizzled mod={mod} rows={rows} dim={dim}", flush=True)
    d = inputs.make("bcast", rows=rows, dim=dim, seed=7 * rows + dim)
    cols = dim // 16
    size = alnp.swizzled_sf_size(rows, dim)
    sentinel = 0xA5
    sf = torch.full((size,), sentinel, dtype=torch.uint8, device="cuda")
    x = dev_bf16(d["x"])
    if mod:
        packed, sf = alnp.ada_layer_norm_quant_nvfp4_swizzled_bf16(
            x, dev_bf16(d["scale"]), dev_bf16(d["shift"]), sf_swizzled=sf)
        rp, rs, _, _, _ = orc.adaln_fp4(d["x"], d["scale"], d["shift"])
    else:
        packed, sf = alnp.layer_norm_no_affine_quant_nvfp4_swizzled_bf16(x, sf_swizzled=sf)
        rp, rs, _, _, _ = orc.ln_fp4(d["x"])
    got = host_u8(sf)
    pos = swizzled_positions(orc, rows, cols)
    fp4_check(host_u8(packed), got[pos], rp, rs, f"swizzled {rows}x{dim}")
    # Padding columns of written rows are zero; padding rows are untouched.
    pc = -(-cols // 4) * 4
    for r in range(rows):
        for c in range(cols, pc):
            assert got[orc.sf_swizzled_offset(r, c, cols)] == 0
    pr = -(-rows // 128) * 128
    for r in range(rows, pr):
        for c in range(pc):
            assert got[orc.sf_swizzled_offset(r, c, cols)] == sentinel
    # The same scales as the row-major entry, moved.
    if mod:
        _, sf_rm = alnp.ada_layer_norm_quant_nvfp4_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]))
    else:
        _, sf_rm = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x)
    assert np.array_equal(got[pos], host_u8(sf_rm))


# ---- AdaLN -> FP4 with modfp8 operands (tiled scales) ------------------------------

def run_fp4_modfp8(d, sdeq, hdeq, x=None, sentinel=None):
    rows, dim = d["x"].shape
    sf = None
    if sentinel is not None:
        sf = torch.full((alnp.swizzled_sf_size(rows, dim),), sentinel, dtype=torch.uint8,
                        device="cuda")
    packed, sf = alnp.ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
        dev_bf16(d["x"]) if x is None else x, dev_u8_as_fp8(d["scale_fp8"]),
        dev_u8_as_fp8(d["shift_fp8"]), scalar(sdeq), scalar(hdeq), sf_swizzled=sf)
    return host_u8(packed), host_u8(sf)


@pytest.mark.parametrize("rows,dim", FP4_SHAPES)
def test_adaln_fp4_modfp8_shapes(orc, rows, dim):
    print(f"adaln fp4 modfp8 rows={rows} dim={dim}", flush=True)
    d = modfp8_inputs(rows, dim, seed=rows + 11 * dim)
    gp, gs = run_fp4_modfp8(d, 0.75, 1.5, sentinel=0xA5)
    rp, rs, _, _, _ = orc.adaln_fp4_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5)
    cols = dim // 16
    fp4_check(gp, gs[swizzled_positions(orc, rows, cols)], rp, rs, f"fp4 modfp8 {rows}x{dim}")
    pc = -(-cols // 4) * 4
    for r in range(rows):
        for c in range(cols, pc):
            assert gs[orc.sf_swizzled_offset(r, c, cols)] == 0
    for r in range(rows, -(-rows // 128) * 128):
        for c in range(pc):
            assert gs[orc.sf_swizzled_offset(r, c, cols)] == 0xA5


def test_adaln_fp4_modfp8_unit_dequant_equals_broadcast_bitwise():
    # e4m3 values are exact in bf16: unit scalars give the broadcast entry's bytes.
    rows, dim = 257, 3072
    d = modfp8_inputs(rows, dim, seed=38)
    sc = torch.from_numpy(d["scale_fp8"]).view(torch.float8_e4m3fn).float().to(torch.bfloat16).cuda()
    sh = torch.from_numpy(d["shift_fp8"]).view(torch.float8_e4m3fn).float().to(torch.bfloat16).cuda()
    gp, gs = run_fp4_modfp8(d, 1.0, 1.0, sentinel=0x3C)
    # Same fill: padding rows of the tiled buffer are not written.
    s2 = torch.full((alnp.swizzled_sf_size(rows, dim),), 0x3C, dtype=torch.uint8, device="cuda")
    p2, s2 = alnp.ada_layer_norm_quant_nvfp4_swizzled_bf16(dev_bf16(d["x"]), sc, sh, sf_swizzled=s2)
    assert np.array_equal(gp, host_u8(p2)) and np.array_equal(gs, host_u8(s2))


def test_adaln_fp4_modfp8_full_size(orc):
    rows, dim = 4096, 3072
    d = modfp8_inputs(rows, dim, seed=39)
    gp, gs = run_fp4_modfp8(d, 0.5, 2.0)
    rp, rs, _, _, _ = orc.adaln_fp4_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.5, 2.0,
                                           threads=8)  # every row
    pos = swizzled_positions(orc, rows, dim // 16)
    fp4_check(gp, gs[pos], rp, rs, "fp4 modfp8 4096x3072")


def test_adaln_fp4_modfp8_unaligned_fallback(orc):
    rows, dim = 11, 3072
    d = modfp8_inputs(rows, dim, seed=40)
    x = misaligned_like((rows, dim), torch.bfloat16)
    x.copy_(dev_bf16(d["x"]))
    gp, gs = run_fp4_modfp8(d, 0.75, 1.5, x=x)
    rp, rs, _, _, _ = orc.adaln_fp4_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5)
    fp4_check(gp, gs[swizzled_positions(orc, rows, dim // 16)], rp, rs, "fp4 modfp8 unaligned")


def test_adaln_fp4_zero_modulation_equals_ln_fp4_bitwise():
    d = inputs.make("fp4", rows=512, dim=3072, seed=35)
    x = dev_bf16(d["x"])
    z = torch.zeros(3072, dtype=torch.bfloat16, device="cuda")
    p1, s1 = alnp.ada_layer_norm_quant_nvfp4_bf16(x, z, z)
    p2, s2 = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x)
    assert np.array_equal(host_u8(p1), host_u8(p2)) and np.array_equal(host_u8(s1), host_u8(s2))


def test_adaln_fp4_full_size(orc):
    d = inputs.make("bcast", rows=4096, dim=3072, seed=36)
    packed, sf = alnp.ada_layer_norm_quant_nvfp4_bf16(dev_bf16(d["x"]), dev_bf16(d["scale"]),
                                                      dev_bf16(d["shift"]))
    rp, rs, _, _, _ = orc.adaln_fp4(d["x"], d["scale"], d["shift"], threads=8)  # every row
    fp4_check(host_u8(packed), host_u8(sf), rp, rs, "adaln fp4 4096x3072")


def test_adaln_fp4_unaligned_fallback(orc):
    d = inputs.make("bcast", rows=11, dim=3072, seed=37)
    x = misaligned_like((11, 3072), torch.bfloat16)
    x.copy_(dev_bf16(d["x"]))
    packed, sf = alnp.ada_layer_norm_quant_nvfp4_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]))
    rp, rs, _, _, _ = orc.adaln_fp4(d["x"], d["scale"], d["shift"])
    fp4_check(host_u8(packed), host_u8(sf), rp, rs, "adaln fp4 unaligned")


# ---- launch-time choices that must not change bytes ----------------------------------

def _shared_operand_call(kind, mx, x, d):
    """One call of a shared-operand form; returns (codes, mx scales or None,
    row_mean, row_rstd) on the host."""
    rows = x.shape[0]
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    sc, sh = dev_bf16(d["scale"]), dev_bf16(d["shift"])
    s8, h8 = dev_u8_as_fp8(d["scale_fp8"]), dev_u8_as_fp8(d["shift_fp8"])
    inv_s = dev_bf16(d["inv_s"])
    st = dict(row_mean=mean, row_rstd=rstd)
    if mx:
        if kind == "bcast":
            o, s = alnp.ada_layer_norm_quant_mxfp8_bf16(x, sc, sh, **st)
        elif kind == "modfp8":
            o, s = alnp.ada_layer_norm_quant_mxfp8_modfp8_bf16(x, s8, h8, scalar(0.75), scalar(1.5), **st)
        else:
            o, s = alnp.awq_ada_layer_norm_quant_mxfp8_bf16(x, sc, sh, inv_s, **st)
        return host_u8(o), host_u8(s), mean.cpu().numpy(), rstd.cpu().numpy()
    if kind == "bcast":
        o = alnp.ada_layer_norm_quant_fp8_bf16(x, sc, sh, act(), **st)
    elif kind == "modfp8":
        o = alnp.ada_layer_norm_quant_fp8_modfp8_bf16(x, s8, h8, scalar(0.75), scalar(1.5), act(), **st)
    else:
        o = alnp.awq_ada_layer_norm_quant_fp8_bf16(x, sc, sh, inv_s, act(), **st)
    return host_u8(o), None, mean.cpu().numpy(), rstd.cpu().numpy()


@pytest.mark.parametrize("dim", [2048, 3072])
def test_modfp8_operands_on_8_byte_boundaries(orc, dim):
    """Rows that fill every slot, from 512 rows: the FP8 modfp8 form loads its
    e4m3 operands in lane pairs (16 bytes per lane) when both are 16-byte
    aligned, and eight bytes per lane otherwise.  Operands that start 8 bytes
    past a 16-byte boundary give the same codes and row statistics as
    aligned ones."""
    print(f"modfp8 operand alignment dim={dim}", flush=True)
    rows = 1030
    d = modfp8_inputs(rows, dim, seed=43)
    x = dev_bf16(d["x"])
    outs = []
    for off in (0, 8):
        s8 = torch.zeros(dim + 16, dtype=torch.uint8, device="cuda")
        h8 = torch.zeros(dim + 16, dtype=torch.uint8, device="cuda")
        s8[off:off + dim] = torch.from_numpy(d["scale_fp8"]).cuda()
        h8[off:off + dim] = torch.from_numpy(d["shift_fp8"]).cuda()
        sv, hv = s8[off:off + dim].view(torch.float8_e4m3fn), h8[off:off + dim].view(torch.float8_e4m3fn)
        assert (sv.data_ptr() % 16 == 0) == (off == 0)
        mean = torch.empty(rows, dtype=torch.float32, device="cuda")
        rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
        o = alnp.ada_layer_norm_quant_fp8_modfp8_bf16(x, sv, hv, scalar(0.75), scalar(1.5), act(),
                                                     row_mean=mean, row_rstd=rstd)
        outs.append((host_u8(o), mean.cpu().numpy(), rstd.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ref = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5, 0.025)[0]
    assert_codes_close(outs[0][0], ref, e4m3_ordinal, f"modfp8 lane pairs {rows}x{dim}")


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("kind", ["bcast", "modfp8", "awq"])
def test_shared_operand_forms_same_bytes_across_the_row_threshold(kind, mx):
    """From 512 rows the broadcast, modfp8 and AWQ forms form (1 + scale) and
    shift before the row arrives; smaller calls keep x first.  A 1030-row
    call and calls of at most 511 rows give the same codes, scales and row
    statistics."""
    print(f"shared-operand threshold kind={kind} mx={mx}", flush=True)
    rows, dim = 1030, 3072
    d = modfp8_inputs(rows, dim, seed=41)
    d["inv_s"] = inputs.to_bf16_bits(np.abs(inputs.normal_f32((dim,), 0.5, 41, 11)) + 0.5)
    x = dev_bf16(d["x"])
    full = _shared_operand_call(kind, mx, x, d)
    for r0, bs in ((0, 511), (511, 511), (1022, 8), (300, 1)):
        part = _shared_operand_call(kind, mx, x[r0:r0 + bs], d)
        for p, f in zip(part, full):
            if p is None:
                continue
            if p.ndim == 2:
                assert np.array_equal(p, f[r0:r0 + bs]), (kind, mx, r0, bs)
            else:
                assert np.array_equal(p, f[r0:r0 + bs]), (kind, mx, r0, bs, "stats")


@pytest.mark.parametrize("mod", ["ln", "bcast", "modfp8"])
@pytest.mark.parametrize("rows,dim", [(512, 3072), (768, 1536), (256, 80)])
def test_fp4_swizzled_row_grouping(orc, mod, rows, dim):
    """With rows a multiple of 256 the tiled-scale entries hand rows to
    workgroups in an XCD-grouped order; codes, tiled scales and row
    statistics must match the oracle and the row-major entries byte for
    byte."""
    print(f"fp4 swizzled grouping mod={mod} rows={rows} dim={dim}", flush=True)
    d = modfp8_inputs(rows, dim, seed=rows + dim)
    cols = dim // 16
    x = dev_bf16(d["x"])
    st = lambda: (torch.empty(rows, dtype=torch.float32, device="cuda"),
                  torch.empty(rows, dtype=torch.float32, device="cuda"))
    (m1, r1), (m2, r2) = st(), st()
    if mod == "ln":
        p1, s1 = alnp.layer_norm_no_affine_quant_nvfp4_swizzled_bf16(x, row_mean=m1, row_rstd=r1)
        p2, s2 = alnp.layer_norm_no_affine_quant_nvfp4_bf16(x, row_mean=m2, row_rstd=r2)
        rp, rs, rm, rr, _ = orc.ln_fp4(d["x"])
    elif mod == "bcast":
        sc, sh = dev_bf16(d["scale"]), dev_bf16(d["shift"])
        p1, s1 = alnp.ada_layer_norm_quant_nvfp4_swizzled_bf16(x, sc, sh, row_mean=m1, row_rstd=r1)
        p2, s2 = alnp.ada_layer_norm_quant_nvfp4_bf16(x, sc, sh, row_mean=m2, row_rstd=r2)
        rp, rs, rm, rr, _ = orc.adaln_fp4(d["x"], d["scale"], d["shift"])
    else:
        p1, s1 = alnp.ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
            x, dev_u8_as_fp8(d["scale_fp8"]), dev_u8_as_fp8(d["shift_fp8"]), scalar(0.75),
            scalar(1.5), row_mean=m1, row_rstd=r1)
        p2, s2 = None, None
        rp, rs, rm, rr, _ = orc.adaln_fp4_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5)
    got = host_u8(s1)
    pos = swizzled_positions(orc, rows, cols)
    fp4_check(host_u8(p1), got[pos], rp, rs, f"grouped swizzled {mod} {rows}x{dim}")
    for r in range(rows):
        for c in range(cols, -(-cols // 4) * 4):
            assert got[orc.sf_swizzled_offset(r, c, cols)] == 0
    assert_stats_close(m1.cpu().numpy(), r1.cpu().numpy(), rm, rr)
    if p2 is not None:
        assert np.array_equal(host_u8(p1), host_u8(p2))
        assert np.array_equal(got[pos], host_u8(s2))
        assert np.array_equal(m1.cpu().numpy(), m2.cpu().numpy())
        assert np.array_equal(r1.cpu().numpy(), r2.cpu().numpy())


@pytest.mark.parametrize("kind", ["bcast", "modfp8", "awq"])
@pytest.mark.parametrize("dim", [8, 1152, 1536, 2048, 5376, 6144, 12000])
def test_shared_operand_forms_ahead_of_the_row_shapes(orc, kind, dim):
    """600 rows: the operands-ahead path at every row shape it takes (up to
    three vectors per thread, partial last slots) and the plain path above
    it, against the oracle."""
    rows = 600
    print(f"shared-operand forms ahead kind={kind} dim={dim}", flush=True)
    d = modfp8_inputs(rows, dim, seed=7 * dim + 5)
    d["inv_s"] = inputs.to_bf16_bits(np.abs(inputs.normal_f32((dim,), 0.5, dim, 11)) + 0.5)
    got, _, m, r = _shared_operand_call(kind, False, dev_bf16(d["x"]), d)
    if kind == "bcast":
        ref, rm, rr, _ = orc.adaln_fp8_bcast(d["x"], d["scale"], d["shift"], 0.025, threads=8)
    elif kind == "modfp8":
        ref, rm, rr, _ = orc.adaln_fp8_modfp8(d["x"], d["scale_fp8"], d["shift_fp8"], 0.75, 1.5,
                                              0.025, threads=8)
    else:
        ref, rm, rr, _ = orc.awq_adaln_fp8(d["x"], d["scale"], d["shift"], d["inv_s"], 0.025,
                                           threads=8)
    assert_codes_close(got, ref, e4m3_ordinal, f"{kind} {rows}x{dim}")
    assert_stats_close(m, r, rm, rr)
