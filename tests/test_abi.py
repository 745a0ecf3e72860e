"""The C ABI without a GPU: libalnp.so loads, exports every entry point that
include/alnp.h declares, and rejects bad arguments on the host with the
documented status, before any launch (no call here reaches a kernel)."""
import ctypes
import math
import os
import re

import pytest

import dit_adaptive_layernorm_amd as alnp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "alnp.h")

OK, NULL, SHAPE, DIM, INDEX, ALIGN, LAUNCH, ARG = 0, -1, -2, -3, -4, -5, -6, -7

# Fake, never dereferenced device addresses (validation only looks at them).
A = 0x7F0000000000
B = 0x7F0000100000
C = 0x7F0000200000
D = 0x7F0000300000


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(alnp_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return alnp.lib()


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) == 29
    for n in names:
        assert hasattr(L, n), n
    assert sorted(alnp.SIGNATURES) == names


def test_status_strings(L):
    assert L.alnp_abi_version() == 1
    for s in (OK, NULL, SHAPE, DIM, INDEX, ALIGN, LAUNCH, ARG, 99):
        assert isinstance(L.alnp_status_string(s), bytes)


def test_fp8_validation(L):
    f = L.alnp_ada_layer_norm_quant_fp8_ptok_bf16
    assert f(A, B, C, D, 1e-5, -1, 64, A, None, None, None) == SHAPE
    assert f(A, B, C, D, 1e-5, 4, 0, A, None, None, None) == SHAPE
    assert f(A, B, C, D, 1e-5, 4, 1 << 25, A, None, None, None) == SHAPE
    assert f(A, B, C, D, 1e-5, 1 << 24, 64, A, None, None, None) == SHAPE
    assert f(A, B, C, D, 1e-5, 4, 63, A, None, None, None) == DIM
    assert f(None, B, C, D, 1e-5, 4, 64, A, None, None, None) == NULL
    assert f(A, None, C, D, 1e-5, 4, 64, A, None, None, None) == NULL
    assert f(A, B, C, None, 1e-5, 4, 64, A, None, None, None) == NULL
    assert f(A, B, C, D, 1e-5, 4, 64, None, None, None, None) == NULL
    assert f(A + 1, B, C, D, 1e-5, 4, 64, A, None, None, None) == ALIGN
    assert f(A, B, C, D + 2, 1e-5, 4, 64, A, None, None, None) == ALIGN
    assert f(A, B, C, D, 1e-5, 4, 64, A, B + 2, None, None) == ALIGN
    assert f(A, B, C, D, -1.0, 4, 64, A, None, None, None) == ARG
    assert f(A, B, C, D, math.nan, 4, 64, A, None, None, None) == ARG
    assert f(A, B, C, D, math.inf, 4, 64, A, None, None, None) == ARG
    # rows == 0 is a no-op, even with null pointers.
    assert f(None, None, None, None, 1e-5, 0, 64, None, None, None, None) == OK
    g = L.alnp_ada_layer_norm_quant_fp8_bf16
    assert g(A, None, C, D, 1e-5, 4, 64, A, None, None, None) == NULL
    assert g(A, B, C, D, 1e-5, 4, 7, A, None, None, None) == DIM
    h = L.alnp_layer_norm_no_affine_quant_fp8_static_bf16
    assert h(A, None, 1e-5, 4, 64, A, None, None, None) == NULL
    assert h(A, D, 1e-5, -5, 64, A, None, None, None) == SHAPE


def test_table_validation(L):
    f = L.alnp_ada_layer_norm_quant_fp8_ptok_table_bf16

    def call(x=A, temb=B, table=C, chunks=6, si=0, ci=1, act=D, eps=1e-5, rows=4, dim=64, out=A):
        return f(x, temb, table, chunks, si, ci, act, eps, rows, dim, out, None, None, None)
    assert call(si=6) == INDEX
    assert call(ci=-1) == INDEX
    assert call(chunks=0) == SHAPE
    assert call(table=None) == NULL
    assert call(temb=None) == NULL
    assert call(table=C + 2) == ALIGN
    assert call(dim=9) == DIM


def test_fp4_validation(L):
    f = L.alnp_layer_norm_no_affine_quant_nvfp4_bf16
    assert f(A, 1e-5, 4, 72, B, C, None, None, None) == DIM
    assert f(A, 1e-5, 4, 64, None, C, None, None, None) == NULL
    assert f(A, 1e-5, 4, 64, B, None, None, None, None) == NULL
    assert f(A + 1, 1e-5, 4, 64, B, C, None, None, None) == ALIGN
    assert f(A, -1e-5, 4, 64, B, C, None, None, None) == ARG
    assert f(None, 1e-5, 0, 64, None, None, None, None, None) == OK
    assert L.alnp_sf_size(4096, 3072) == 4096 * 192
    assert L.alnp_sf_size(4096, 3000) == DIM
    assert L.alnp_sf_size(-1, 3072) == SHAPE
    assert alnp.sf_size(2, 32) == 4


def test_variant_validation(L):
    m = L.alnp_ada_layer_norm_quant_fp8_modfp8_bf16
    assert m(A, B, C, None, D, D, 1e-5, 4, 64, A, None, None, None) == NULL
    assert m(A, B, C, D, D + 2, D, 1e-5, 4, 64, A, None, None, None) == ALIGN
    assert m(A, B, C, D, D, D, 1e-5, 4, 63, A, None, None, None) == DIM
    assert m(None, None, None, None, None, None, 1e-5, 0, 64, None, None, None, None) == OK
    w = L.alnp_awq_ada_layer_norm_quant_fp8_bf16
    assert w(A, B, C, None, D, 1e-5, 4, 64, A, None, None, None) == NULL
    assert w(A, B, C, D + 1, D, 1e-5, 4, 64, A, None, None, None) == ALIGN
    f = L.alnp_ada_layer_norm_quant_nvfp4_bf16
    assert f(A, None, C, 1e-5, 4, 64, B, C, None, None, None) == NULL
    assert f(A, B, C, 1e-5, 4, 40, B, C, None, None, None) == DIM
    g = L.alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16
    assert g(A, B, C + 2 - 1, 1e-5, 4, 64, B, C, None, None, None) == ALIGN
    h = L.alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16
    assert h(A, 1e-5, 4, 64, B, None, None, None, None) == NULL
    q = L.alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16

    def call(x=A, s8=B, h8=C, sd=D, hd=D, eps=1e-5, rows=4, dim=64, pk=B, sf=C):
        return q(x, s8, h8, sd, hd, eps, rows, dim, pk, sf, None, None, None)
    assert call(s8=None) == NULL
    assert call(hd=None) == NULL
    assert call(sd=D + 2) == ALIGN
    assert call(dim=40) == DIM
    assert call(eps=math.nan) == ARG
    assert call(x=None, s8=None, h8=None, sd=None, hd=None, rows=0, pk=None, sf=None) == OK
    assert L.alnp_swizzled_sf_size(4096, 3072) == 4096 * 192
    assert L.alnp_swizzled_sf_size(130, 48) == 256 * 4
    assert L.alnp_swizzled_sf_size(1, 16) == 128 * 4
    assert L.alnp_swizzled_sf_size(5, 24) == DIM
    assert alnp.swizzled_sf_size(300, 3072) == 384 * 192


def test_modulation6_validation(L):
    f = L.alnp_adaln_modulation6_bf16
    P6 = ctypes.c_void_p * 6
    outs = P6(A, B, C, D, A + 64, B + 64)
    assert f(A, B, -1, 5, 64, outs, None) == SHAPE
    assert f(A, B, 1, 5, 0, outs, None) == SHAPE
    assert f(A, B, 1 << 12, 1 << 12, 64, outs, None) == SHAPE
    assert f(None, B, 1, 5, 64, outs, None) == NULL
    assert f(A, B, 1, 5, 64, None, None) == NULL
    assert f(A, B, 1, 5, 64, P6(A, B, C, None, A, B), None) == NULL
    assert f(A, B, 1, 5, 64, P6(A, B, C, D + 1, A, B), None) == ALIGN
    assert f(A + 2, B, 1, 5, 64, outs, None) == ALIGN
    assert f(None, None, 0, 5, 64, None, None) == OK


def test_gated_residual_validation(L):
    f = L.alnp_gated_residual_bf16
    assert f(A, B, C, 4, 64, 2, D, None) == SHAPE
    assert f(A, B, C, -1, 64, 1, D, None) == SHAPE
    assert f(A, B, C, 4, 0, 1, D, None) == SHAPE
    assert f(A, None, C, 4, 64, 4, D, None) == NULL
    assert f(A, B, C, 4, 64, 1, D + 1, None) == ALIGN
    assert f(None, None, None, 0, 64, 0, None, None) == OK


def test_quant_validation(L):
    f = L.alnp_quant_fp8_static_f32
    assert f(A, B, -1, C, None) == SHAPE
    assert f(A, B, (1 << 31) + 1, C, None) == SHAPE
    assert f(None, B, 4, C, None) == NULL
    assert f(A + 2, B, 4, C, None) == ALIGN
    assert f(None, None, 0, None, None) == OK


def test_rms_modulate_validation(L):
    f = L.alnp_rms_norm_modulate_seg_bf16

    def call(x=A, w=B, sc=C, sh=D, seg=B, segments=3, eps=1e-5, rows=4, dim=64, out=A, rstd=None):
        return f(x, w, sc, sh, seg, segments, eps, rows, dim, out, rstd, None)
    assert call(segments=0) == SHAPE
    assert call(segments=1 << 31) == SHAPE
    assert call(rows=-1) == SHAPE
    assert call(dim=0) == SHAPE
    assert call(x=None) == NULL
    assert call(sc=None) == NULL
    assert call(sh=None) == NULL
    assert call(seg=None) == NULL
    assert call(out=None) == NULL
    assert call(w=B + 1) == ALIGN
    assert call(seg=B + 2) == ALIGN
    assert call(rstd=C + 2) == ALIGN
    assert call(eps=-1.0) == ARG
    assert call(x=None, sc=None, sh=None, seg=None, out=None, rows=0) == OK


def test_mx_validation(L):
    f8 = L.alnp_ada_layer_norm_quant_mxfp8_ptok_bf16
    assert f8(A, B, C, 1e-5, 4, 48, A, D, None, None, None) == DIM
    assert f8(A, None, C, 1e-5, 4, 64, A, D, None, None, None) == NULL
    assert f8(A, B, C, 1e-5, 4, 64, A, None, None, None, None) == NULL
    assert f8(A + 1, B, C, 1e-5, 4, 64, A, D, None, None, None) == ALIGN
    assert f8(A, B, C, -1.0, 4, 64, A, D, None, None, None) == ARG
    assert f8(None, None, None, 1e-5, 0, 64, None, None, None, None, None) == OK
    ln8 = L.alnp_layer_norm_no_affine_quant_mxfp8_bf16
    assert ln8(A, 1e-5, 4, 64, None, D, None, None, None) == NULL
    f4 = L.alnp_ada_layer_norm_quant_mxfp4_bf16
    assert f4(A, B, C, 1e-5, 4, 48, B, C, None, None, None) == DIM
    assert f4(A, None, C, 1e-5, 4, 64, B, C, None, None, None) == NULL
    ln4 = L.alnp_layer_norm_no_affine_quant_mxfp4_bf16
    assert ln4(A, 1e-5, 4, 64, B, None, None, None, None) == NULL
    assert ln4(A, 1e-5, 4, 80, B, C, None, None, None) == DIM
    t8 = L.alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16

    def call(x=A, temb=B, table=C, chunks=6, si=0, ci=1, eps=1e-5, rows=4, dim=64, out=A, sc=D):
        return t8(x, temb, table, chunks, si, ci, eps, rows, dim, out, sc, None, None, None)
    assert call(si=6) == INDEX
    assert call(chunks=0) == SHAPE
    assert call(table=None) == NULL
    assert call(sc=None) == NULL
    assert call(table=C + 2) == ALIGN
    assert call(dim=48) == DIM
    assert call(x=None, temb=None, table=None, chunks=0, rows=0, out=None, sc=None) == OK
    # modfp8 and AWQ forms: their operands are required and aligned.
    m8 = L.alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16

    def mcall(x=A, sf=B, hf=B + 64, sd=C, hd=C + 4, eps=1e-5, rows=4, dim=64, out=A, sc=D):
        return m8(x, sf, hf, sd, hd, eps, rows, dim, out, sc, None, None, None)
    assert mcall(sf=None) == NULL
    assert mcall(hd=None) == NULL
    assert mcall(sd=C + 2) == ALIGN
    assert mcall(dim=48) == DIM
    assert mcall(eps=float("nan")) == ARG
    aw = L.alnp_awq_ada_layer_norm_quant_mxfp8_bf16
    assert aw(A, B, C, None, 1e-5, 4, 64, A, D, None, None, None) == NULL
    assert aw(A, B, C, D + 1, 1e-5, 4, 64, A, D, None, None, None) == ALIGN
    assert aw(A, B, C, D, 1e-5, 4, 48, A, D, None, None, None) == DIM
    m4 = L.alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16
    assert m4(A, B, B + 64, C, None, 1e-5, 4, 64, B, C, None, None, None) == NULL
    assert m4(A, B, B + 64, C, C + 4, 1e-5, 4, 80, B, C, None, None, None) == DIM
    assert m4(None, None, None, None, None, 1e-5, 0, 64, None, None, None, None, None) == OK
    assert L.alnp_mx_scale_size(4096, 3072) == 4096 * 96
    assert L.alnp_mx_scale_size(4, 48) == DIM
    assert alnp.mx_scale_size(2, 64) == 4

