"""Parity of the FP8 producers (LN, broadcast, per-token, table) with the
oracle, through the C ABI: small and ragged shapes compared element by
element, the full-size workloads on every row, the edge cases (one row,
tails of a partial wave, the workgroup-per-row fallback for dims that are
not a multiple of 8 or above 32768 and for unaligned pointers), and the
identities between forms, batch invariance and determinism on the GPU."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import (act, assert_codes_close, assert_stats_close, dev_bf16, dev_f32, e4m3_ordinal,
                    host_u8, misaligned_like)

pytestmark = pytest.mark.gpu

SHAPES = [(1, 2048), (7, 3072), (16, 2048), (63, 1536), (65, 1152), (257, 512), (5, 8),
          (9, 5376), (3, 8192), (4, 2), (6, 6), (5, 1030), (3, 8200), (2, 12000),
          (3, 10240), (2, 16384), (2, 20480), (1, 24576), (1, 28672), (2, 32768),
          (2, 32776), (1, 40000)]


def run_gpu(kind, d, rows, dim, x=None, out=None):
    x = dev_bf16(d["x"]) if x is None else x
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    a = act(d["act_scale"])
    if kind == "ln":
        o = alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, a, out=out, row_mean=mean, row_rstd=rstd)
    elif kind == "bcast":
        o = alnp.ada_layer_norm_quant_fp8_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]), a,
                                               out=out, row_mean=mean, row_rstd=rstd)
    elif kind == "ptok":
        o = alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, dev_bf16(d["scale"]), dev_bf16(d["shift"]), a,
                                                    out=out, row_mean=mean, row_rstd=rstd)
    else:
        o = alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(
            x, dev_bf16(d["temb"]), dev_f32(d["table"]), a, d["shift_idx"], d["scale_idx"],
            out=out, row_mean=mean, row_rstd=rstd)
    return host_u8(o), mean.cpu().numpy(), rstd.cpu().numpy()


def run_oracle(orc, kind, d, rows_sel=None, threads=8):
    sel = (lambda a: a) if rows_sel is None else (lambda a: np.ascontiguousarray(a[rows_sel]))
    x = sel(d["x"])
    if kind == "ln":
        return orc.ln_fp8(x, d["act_scale"], threads=threads)[:3]
    if kind == "bcast":
        return orc.adaln_fp8_bcast(x, d["scale"], d["shift"], d["act_scale"], threads=threads)[:3]
    if kind == "ptok":
        return orc.adaln_fp8_ptok(x, sel(d["scale"]), sel(d["shift"]), d["act_scale"],
                                  threads=threads)[:3]
    return orc.adaln_fp8_table(x, sel(d["temb"]), d["table"], d["shift_idx"], d["scale_idx"],
                               d["act_scale"], threads=threads)[:3]


@pytest.mark.parametrize("kind", ["ln", "bcast", "ptok", "table"])
@pytest.mark.parametrize("rows,dim", SHAPES)
def test_small_shapes(orc, kind, rows, dim):
    d = inputs.make(kind, rows=rows, dim=dim, seed=rows * 7 + dim)
    print(f"fp8 {kind} rows={rows} dim={dim}", flush=True)
    got, mean, rstd = run_gpu(kind, d, rows, dim)
    ref, rmean, rrstd = run_oracle(orc, kind, d)
    assert_codes_close(got, ref, e4m3_ordinal, f"{kind} {rows}x{dim}")
    assert_stats_close(mean, rstd, rmean, rrstd)


@pytest.mark.parametrize("name", ["bcast_fp8_16x2048", "ptok_fp8_2520x3072", "table_fp8_2520x3072"])
def test_full_size_workloads(orc, name):
    d = inputs.workload(name)
    kind = d["kind"]
    rows, dim = d["x"].shape
    print(f"fp8 workload {name}", flush=True)
    got, mean, rstd = run_gpu(kind, d, rows, dim)
    ref, rmean, rrstd = run_oracle(orc, kind, d)  # every row
    assert_codes_close(got, ref, e4m3_ordinal, name)
    assert_stats_close(mean, rstd, rmean, rrstd)
    # Properties at every row: modulation-off statistics agree with float64.
    xf = (d["x"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(mean, xf.mean(1), rtol=0, atol=1e-5 * xf.std(1).max())
    assert np.allclose(rstd, 1 / np.sqrt(xf.var(1) + 1e-5), rtol=1e-5, atol=0)


# From 513 rows the table form runs its LDS-staged kernel (two rows per
# workgroup, both fp32 table rows in LDS) for rows of up to 4 waves.  Row
# shapes of 1, 2 and 4 waves with 1 to 7 vectors per thread; 3080 has a
# partial last vector slot; 7168 (2 waves x 7 vectors, 57344 bytes of tables
# in LDS) is the largest dim it takes: 7176, 8192 and 8200 have 8-wave rows
# and run the rows kernel.  601 rows: the last workgroup's second row lies
# past the end.
@pytest.mark.parametrize("dim", [512, 1152, 1536, 2048, 3080, 4096, 5376, 6144, 7168, 7176,
                                 8192, 8200])
def test_table_lds_kernel_dims(orc, dim):
    rows = 601
    d = inputs.make("table", rows=rows, dim=dim, seed=dim, shift_idx=4, scale_idx=1)
    print(f"fp8 table rows={rows} dim={dim}", flush=True)
    got, mean, rstd = run_gpu("table", d, rows, dim)
    ref, rmean, rrstd = run_oracle(orc, "table", d)
    assert_codes_close(got, ref, e4m3_ordinal, f"table {rows}x{dim}")
    assert_stats_close(mean, rstd, rmean, rrstd)


@pytest.mark.parametrize("kind", ["ln", "bcast", "ptok", "table"])
def test_unaligned_pointers_use_fallback(orc, kind):
    rows, dim = 9, 3072
    d = inputs.make(kind, rows=rows, dim=dim, seed=77)
    x = misaligned_like((rows, dim), torch.bfloat16)
    x.copy_(dev_bf16(d["x"]))
    out = misaligned_like((rows, dim), torch.float8_e4m3fn, elem_offset=3)
    got, mean, rstd = run_gpu(kind, d, rows, dim, x=x, out=out)
    ref, rmean, rrstd = run_oracle(orc, kind, d)
    assert_codes_close(got, ref, e4m3_ordinal, f"unaligned {kind}")
    assert_stats_close(mean, rstd, rmean, rrstd)


def test_zero_modulation_equals_ln_bitwise():
    d = inputs.make("bcast", rows=300, dim=3072, seed=5)
    zero = torch.zeros(3072, dtype=torch.bfloat16, device="cuda")
    x = dev_bf16(d["x"])
    a = act()
    o1 = host_u8(alnp.ada_layer_norm_quant_fp8_bf16(x, zero, zero, a))
    o2 = host_u8(alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, a))
    assert np.array_equal(o1, o2)


def test_broadcast_equals_replicated_per_token_bitwise():
    d = inputs.make("bcast", rows=129, dim=2048, seed=6)
    x, s, h, a = dev_bf16(d["x"]), dev_bf16(d["scale"]), dev_bf16(d["shift"]), act()
    o1 = host_u8(alnp.ada_layer_norm_quant_fp8_bf16(x, s, h, a))
    o2 = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_bf16(
        x, s.expand(129, 2048).contiguous(), h.expand(129, 2048).contiguous(), a))
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("rows", [70, 600])
def test_table_zero_equals_per_token_chunks_bitwise(rows):
    # 70 rows: the table form on the rows kernel; 600 rows: on the LDS kernel.
    d = inputs.make("table", rows=rows, dim=3072, seed=7, shift_idx=5, scale_idx=3)
    x, temb, a = dev_bf16(d["x"]), dev_bf16(d["temb"]), act()
    zero = torch.zeros(6, 3072, dtype=torch.float32, device="cuda")
    o1 = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(x, temb, zero, a, 5, 3))
    o2 = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_bf16(
        x, temb[:, 3].contiguous(), temb[:, 5].contiguous(), a))
    assert np.array_equal(o1, o2)


def test_batch_invariance_and_determinism():
    """Full batch vs sub-batches (the batch-invariance protocol of the
    RL-Kernel norm_modulate page): byte-identical; two runs identical."""
    d = inputs.make("ptok", rows=2048, dim=3072, seed=8)
    x, s, h, a = dev_bf16(d["x"]), dev_bf16(d["scale"]), dev_bf16(d["shift"]), act()
    full = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, s, h, a))
    again = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, s, h, a))
    assert np.array_equal(full, again)
    for bs in (1, 2, 3, 7, 63, 64, 65, 257, 1025):
        for r0 in (0, 259, 2047 - bs + 1):
            r1 = r0 + bs
            part = host_u8(alnp.ada_layer_norm_quant_fp8_ptok_bf16(
                x[r0:r1], s[r0:r1], h[r0:r1], a))
            assert np.array_equal(part, full[r0:r1]), (bs, r0)


def test_table_batch_invariance_across_kernels():
    """The table form runs the rows kernel up to 512 rows and the LDS-staged
    kernel above: one 1030-row call and calls of at most 512 rows give the
    same bytes and row statistics."""
    d = inputs.make("table", rows=1030, dim=3072, seed=9, shift_idx=2, scale_idx=4)
    full = run_gpu("table", d, 1030, 3072)
    for r0, bs in ((0, 512), (512, 511), (1023, 7), (300, 1)):
        sub = {k: (v[r0:r0 + bs] if k in ("x", "temb") else v) for k, v in d.items()}
        part = run_gpu("table", sub, bs, 3072)
        for p, f in zip(part, full):
            assert np.array_equal(p, f[r0:r0 + bs]), (r0, bs)


def test_empty_rows_is_noop():
    x = torch.empty((0, 3072), dtype=torch.bfloat16, device="cuda")
    out = alnp.layer_norm_no_affine_quant_fp8_static_bf16(x, act())
    assert out.shape == (0, 3072)


def test_constant_and_saturating_rows(orc):
    """Degenerate rows: constant (variance 0 -> xhat 0, y = shift), and
    huge shifts that saturate at +-448."""
    rows, dim = 4, 3072
    x = np.zeros((rows, dim), np.float32)
    x[1] = 3.0
    x[2, ::2], x[2, 1::2] = 1e4, -1e4
    xb = inputs.to_bf16_bits(x)
    shift = inputs.to_bf16_bits(np.linspace(-30, 30, dim).astype(np.float32))
    scale = inputs.to_bf16_bits(np.full(dim, 0.5, np.float32))
    d = dict(x=xb, scale=scale, shift=shift, act_scale=0.025)
    got, _, _ = run_gpu("bcast", d, rows, dim)
    ref = orc.adaln_fp8_bcast(xb, scale, shift, 0.025)[0]
    assert np.array_equal(got, ref)


def test_zero_eps_constant_rows(orc):
    """eps = 0 is accepted: a constant row then has variance 0 and rstd
    1/sqrt(0) = inf, so xhat = 0 * inf is NaN and every code of the row is a
    NaN code (its sign is whatever the platform's default NaN carries, so
    only NaN-ness is compared there); the other rows match the oracle with
    eps = 0 to the usual tolerance, statistics included."""
    rows, dim = 6, 3072
    d = inputs.make("ptok", rows=rows, dim=dim, seed=21)
    x = d["x"].copy()
    x[[1, 4]] = inputs.to_bf16_bits(np.full((2, dim), 0.625, np.float32))
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    o = alnp.ada_layer_norm_quant_fp8_ptok_bf16(dev_bf16(x), dev_bf16(d["scale"]),
                                                dev_bf16(d["shift"]), act(d["act_scale"]),
                                                eps=0.0, row_mean=mean, row_rstd=rstd)
    got = host_u8(o)
    ref, rmean, rrstd = orc.adaln_fp8_ptok(x, d["scale"], d["shift"], d["act_scale"], eps=0.0)[:3]
    const = np.zeros(rows, bool)
    const[[1, 4]] = True
    assert np.all((got[const] & 0x7F) == 0x7F) and np.all((ref[const] & 0x7F) == 0x7F)
    assert_codes_close(got[~const], ref[~const], e4m3_ordinal, "eps 0")
    assert np.all(np.isinf(rstd.cpu().numpy()[const])) and np.all(np.isinf(rrstd[const]))
    assert_stats_close(mean.cpu().numpy()[~const], rstd.cpu().numpy()[~const], rmean[~const],
                       rrstd[~const])
