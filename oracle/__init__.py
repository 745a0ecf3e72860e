"""numpy front end of the plain C oracle (oracle/alnp_oracle.c).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; the product package never imports it and shares
no code with it.

Arrays are numpy: bf16 as uint16 bit patterns, e4m3 / packed e2m1 as uint8,
fp32 as float32.  Large row loops can be split over threads (`threads=`); the
C calls release the GIL, each thread owns a disjoint block of rows, and the
per-row arithmetic is unchanged, so the result does not depend on `threads`.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "orc_bf16_to_f32_n": [_P, _I64, _P],
    "orc_f32_to_bf16_n": [_P, _I64, _P],
    "orc_e4m3_decode_n": [_P, _I64, _P],
    "orc_e4m3_encode_sat_n": [_P, _I64, _P],
    "orc_e2m1_decode_n": [_P, _I64, _P],
    "orc_e2m1_encode_n": [_P, _I64, _P],
    "orc_ln_stats": [_P, _I64, _I64, _F, _P, _P],
    "orc_ln_fp8": [_P, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_adaln_fp8_bcast": [_P, _P, _P, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_adaln_fp8_ptok": [_P, _P, _P, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_adaln_fp8_table": [_P, _P, _P, _I64, _I64, _I64, _F, _F, _I64, _I64,
                            _P, _P, _P, _P],
    "orc_adaln_fp8_f32ops": [_P, _P, _P, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_fp4_block_quant_n": [_P, _I64, _P, _P],
    "orc_fp4_pack": [_P, _I64, _P],
    "orc_ln_fp4": [_P, _F, _I64, _I64, _P, _P, _P, _P, _P],
    "orc_modulation6": [_P, _P, _I64, _I64, _P],
    "orc_adaln_fp8_modfp8": [_P, _P, _P, _F, _F, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_awq_adaln_fp8": [_P, _P, _P, _P, _F, _F, _I64, _I64, _P, _P, _P, _P],
    "orc_adaln_fp4": [_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P],
    "orc_adaln_fp4_modfp8": [_P, _P, _P, _F, _F, _F, _I64, _I64, _P, _P, _P, _P, _P],
    "orc_sf_swizzle": [_P, _I64, _I64, _P],
    "orc_gated_residual": [_P, _P, _P, _I64, _I64, _I64, _P],
    "orc_bf16_modulate_n": [_P, _P, _P, _I64, _P],
    "orc_rms_modulate_seg": [_P, _P, _P, _P, _P, _I64, _F, _I64, _I64, _P, _P, _P],
    "orc_mx_block_quant_n": [_P, _I64, ctypes.c_int, _P, _P],
    "orc_adaln_mxfp4": [_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P],
    "orc_adaln_mxfp8": [_P, _P, _P, ctypes.c_int, _F, _I64, _I64, _P, _P, _P, _P, _P],
    "orc_adaln_mxfp8_table": [_P, _P, _P, _I64, _I64, _I64, _F, _I64, _I64, _P, _P, _P, _P, _P],
}

_RESTYPES = {"orc_e8m0_scale": ([_F, ctypes.c_int], ctypes.c_uint8),
             "orc_e8m0_decode": ([ctypes.c_uint8], ctypes.c_double),
             "orc_sf_swizzled_size": ([_I64, _I64], _I64),
             "orc_sf_swizzled_offset": ([_I64, _I64, _I64], _I64)}

_lib = None


def lib():
    """Load liboracle.so (build it first with oracle/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build  # noqa: WPS433
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None
        for name, (args, res) in _RESTYPES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _row_blocks(rows, threads):
    threads = max(1, min(int(threads), rows)) if rows else 1
    step = -(-rows // threads) if rows else 0
    return [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)] if rows else []


def _parallel(rows, threads, fn):
    blocks = _row_blocks(rows, threads)
    if len(blocks) <= 1:
        for r0, r1 in blocks:
            fn(r0, r1)
        return
    with ThreadPoolExecutor(len(blocks)) as ex:
        list(ex.map(lambda b: fn(*b), blocks))


# ---- number formats -------------------------------------------------------

def bf16_to_f32(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_f32_n(_ptr(b), b.size, _ptr(out))
    return out


def f32_to_bf16(f):
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(f), f.size, _ptr(out))
    return out


def e4m3_decode(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode_sat(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_sat_n(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_decode(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e2m1_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e2m1_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e2m1_encode_n(_ptr(v), v.size, _ptr(out))
    return out


# ---- row statistics -------------------------------------------------------

def ln_stats(x, eps=1e-5):
    x = _c(x, np.uint16)
    rows, dim = x.shape
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    lib().orc_ln_stats(_ptr(x), rows, dim, eps, _ptr(mean), _ptr(rstd))
    return mean, rstd


# ---- FP8 producers --------------------------------------------------------

def _fp8_outputs(rows, dim, want_y):
    out = np.empty((rows, dim), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    y = np.empty((rows, dim), np.float32) if want_y else None
    return out, mean, rstd, y


def _rowptr(a, r0, row_elems):
    return None if a is None else a.ctypes.data + r0 * row_elems * a.itemsize


def ln_fp8(x, act_scale, eps=1e-5, want_y=False, threads=1):
    """LayerNorm (no affine) -> static-scale e4m3; returns (out, mean, rstd, y)."""
    x = _c(x, np.uint16)
    rows, dim = x.shape
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_ln_fp8(_rowptr(x, r0, dim), act_scale, eps, r1 - r0, dim,
                         _rowptr(out, r0, dim), _rowptr(mean, r0, 1),
                         _rowptr(rstd, r0, 1), _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


def adaln_fp8_bcast(x, scale, shift, act_scale, eps=1e-5, want_y=False, threads=1):
    x = _c(x, np.uint16)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    rows, dim = x.shape
    assert scale.shape == (dim,) and shift.shape == (dim,)
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_adaln_fp8_bcast(_rowptr(x, r0, dim), _ptr(scale), _ptr(shift),
                                  act_scale, eps, r1 - r0, dim,
                                  _rowptr(out, r0, dim), _rowptr(mean, r0, 1),
                                  _rowptr(rstd, r0, 1), _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


def adaln_fp8_ptok(x, scale, shift, act_scale, eps=1e-5, want_y=False, threads=1):
    x = _c(x, np.uint16)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    rows, dim = x.shape
    assert scale.shape == (rows, dim) and shift.shape == (rows, dim)
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_adaln_fp8_ptok(_rowptr(x, r0, dim), _rowptr(scale, r0, dim),
                                 _rowptr(shift, r0, dim), act_scale, eps,
                                 r1 - r0, dim, _rowptr(out, r0, dim),
                                 _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1),
                                 _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


def adaln_fp8_table(x, temb, table, shift_idx, scale_idx, act_scale, eps=1e-5,
                    want_y=False, threads=1):
    x = _c(x, np.uint16)
    temb = _c(temb, np.uint16)
    table = _c(table, np.float32)
    rows, dim = x.shape
    chunks = temb.shape[1]
    assert temb.shape == (rows, chunks, dim) and table.shape == (chunks, dim)
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_adaln_fp8_table(_rowptr(x, r0, dim), _rowptr(temb, r0, chunks * dim),
                                  _ptr(table), chunks, shift_idx, scale_idx,
                                  act_scale, eps, r1 - r0, dim,
                                  _rowptr(out, r0, dim), _rowptr(mean, r0, 1),
                                  _rowptr(rstd, r0, 1), _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


def adaln_fp8_f32ops(x, scale_f32, shift_f32, act_scale, eps=1e-5, want_y=False):
    """Per-token core fed fp32 operands (rows, dim) directly."""
    x = _c(x, np.uint16)
    sc = _c(scale_f32, np.float32)
    sh = _c(shift_f32, np.float32)
    rows, dim = x.shape
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)
    lib().orc_adaln_fp8_f32ops(_ptr(x), _ptr(sc), _ptr(sh), act_scale, eps, rows,
                               dim, _ptr(out), _ptr(mean), _ptr(rstd), _ptr(y))
    return out, mean, rstd, y


def adaln_fp8_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, act_scale, eps=1e-5,
                     want_y=False, threads=1):
    """Broadcast AdaLN -> FP8 with e4m3 (dim,) operands times fp32 scalars."""
    x = _c(x, np.uint16)
    sf = _c(scale_fp8, np.uint8)
    hf = _c(shift_fp8, np.uint8)
    rows, dim = x.shape
    assert sf.shape == (dim,) and hf.shape == (dim,)
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_adaln_fp8_modfp8(_rowptr(x, r0, dim), _ptr(sf), _ptr(hf), scale_deq,
                                   shift_deq, act_scale, eps, r1 - r0, dim,
                                   _rowptr(out, r0, dim), _rowptr(mean, r0, 1),
                                   _rowptr(rstd, r0, 1), _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


def awq_adaln_fp8(x, scale, shift, inv_s, act_scale, eps=1e-5, want_y=False, threads=1):
    """Broadcast AdaLN -> per-channel inv_s smoothing -> FP8."""
    x = _c(x, np.uint16)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    inv_s = _c(inv_s, np.uint16)
    rows, dim = x.shape
    assert scale.shape == shift.shape == inv_s.shape == (dim,)
    out, mean, rstd, y = _fp8_outputs(rows, dim, want_y)

    def run(r0, r1):
        lib().orc_awq_adaln_fp8(_rowptr(x, r0, dim), _ptr(scale), _ptr(shift), _ptr(inv_s),
                                act_scale, eps, r1 - r0, dim, _rowptr(out, r0, dim),
                                _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1),
                                _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, mean, rstd, y


# ---- FP4 producer ---------------------------------------------------------

def fp4_block_quant(b):
    """b: (..., 16k) fp32 -> (codes uint8 per element, scale codes per block)."""
    b = _c(b, np.float32)
    assert b.size % 16 == 0
    codes = np.empty(b.shape, np.uint8)
    scales = np.empty(b.shape[:-1] + (b.shape[-1] // 16,), np.uint8)
    lib().orc_fp4_block_quant_n(_ptr(b), b.size // 16, _ptr(codes), _ptr(scales))
    return codes, scales


def fp4_pack(codes):
    c = _c(codes, np.uint8)
    assert c.shape[-1] % 2 == 0
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 2,), np.uint8)
    lib().orc_fp4_pack(_ptr(c), c.size, _ptr(out))
    return out


def ln_fp4(x, eps=1e-5, want_b=False, threads=1):
    """LayerNorm (no affine) -> bf16 stage -> e2m1 packed + e4m3 block scales.

    Returns (packed (rows, dim/2), sf (rows, dim/16), mean, rstd, b)."""
    x = _c(x, np.uint16)
    rows, dim = x.shape
    assert dim % 16 == 0
    packed = np.empty((rows, dim // 2), np.uint8)
    sf = np.empty((rows, dim // 16), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    b = np.empty((rows, dim), np.float32) if want_b else None

    def run(r0, r1):
        lib().orc_ln_fp4(_rowptr(x, r0, dim), eps, r1 - r0, dim,
                         _rowptr(packed, r0, dim // 2), _rowptr(sf, r0, dim // 16),
                         _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1),
                         _rowptr(b, r0, dim))
    _parallel(rows, threads, run)
    return packed, sf, mean, rstd, b


def adaln_fp4(x, scale, shift, eps=1e-5, want_b=False, threads=1):
    """Broadcast AdaLN -> bf16 stage -> e2m1 packed + e4m3 block scales
    (row-major).  Returns (packed, sf, mean, rstd, b)."""
    x = _c(x, np.uint16)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    rows, dim = x.shape
    assert dim % 16 == 0 and scale.shape == shift.shape == (dim,)
    packed = np.empty((rows, dim // 2), np.uint8)
    sf = np.empty((rows, dim // 16), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    b = np.empty((rows, dim), np.float32) if want_b else None

    def run(r0, r1):
        lib().orc_adaln_fp4(_rowptr(x, r0, dim), _ptr(scale), _ptr(shift), eps, r1 - r0, dim,
                            _rowptr(packed, r0, dim // 2), _rowptr(sf, r0, dim // 16),
                            _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1), _rowptr(b, r0, dim))
    _parallel(rows, threads, run)
    return packed, sf, mean, rstd, b


def adaln_fp4_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, eps=1e-5, want_b=False,
                     threads=1):
    """modfp8 operands (e4m3 (dim,) codes times fp32 scalars) -> AdaLN -> bf16
    stage -> e2m1 packed + e4m3 block scales (row-major).  Returns (packed, sf,
    mean, rstd, b)."""
    x = _c(x, np.uint16)
    scale_fp8 = _c(scale_fp8, np.uint8)
    shift_fp8 = _c(shift_fp8, np.uint8)
    rows, dim = x.shape
    assert dim % 16 == 0 and scale_fp8.shape == shift_fp8.shape == (dim,)
    packed = np.empty((rows, dim // 2), np.uint8)
    sf = np.empty((rows, dim // 16), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    b = np.empty((rows, dim), np.float32) if want_b else None

    def run(r0, r1):
        lib().orc_adaln_fp4_modfp8(_rowptr(x, r0, dim), _ptr(scale_fp8), _ptr(shift_fp8),
                                   scale_deq, shift_deq, eps, r1 - r0, dim,
                                   _rowptr(packed, r0, dim // 2), _rowptr(sf, r0, dim // 16),
                                   _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1),
                                   _rowptr(b, r0, dim))
    _parallel(rows, threads, run)
    return packed, sf, mean, rstd, b


def sf_swizzled_size(rows, cols):
    return int(lib().orc_sf_swizzled_size(rows, cols))


def sf_swizzled_offset(r, c, cols):
    return int(lib().orc_sf_swizzled_offset(r, c, cols))


def sf_swizzle(sf_rowmajor):
    """Row-major (rows, cols) e4m3 scales -> 128x4 tiled buffer (padding 0)."""
    sf = _c(sf_rowmajor, np.uint8)
    rows, cols = sf.shape
    out = np.empty(sf_swizzled_size(rows, cols), np.uint8)
    lib().orc_sf_swizzle(_ptr(sf), rows, cols, _ptr(out))
    return out


# ---- residual gate ----------------------------------------------------------

def gated_residual(residual, gate, proj):
    """bf16(residual + bf16(gate * proj)); gate (dim,) or (rows, dim)."""
    res = _c(residual, np.uint16)
    g = _c(gate, np.uint16)
    pr = _c(proj, np.uint16)
    rows, dim = res.shape
    assert pr.shape == (rows, dim)
    gate_rows = 1 if g.shape == (dim,) else rows
    assert g.size == gate_rows * dim
    out = np.empty((rows, dim), np.uint16)
    lib().orc_gated_residual(_ptr(res), _ptr(g), _ptr(pr), rows, dim, gate_rows, _ptr(out))
    return out


# ---- RMSNorm with segment-selected modulation (R14) -------------------------

def bf16_modulate(n, scale, shift):
    """Elementwise bf16((bf16(n * bf16(scale + 1))) + shift) on bf16 bits of one shape."""
    n = _c(n, np.uint16)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    assert n.shape == scale.shape == shift.shape
    out = np.empty(n.shape, np.uint16)
    lib().orc_bf16_modulate_n(_ptr(n), _ptr(scale), _ptr(shift), n.size, _ptr(out))
    return out


def rms_modulate_seg(x, weight, scale, shift, seg, eps=1e-5, want_n=False, threads=1):
    """RMSNorm (weight (dim,) or None) then (n * (scale[seg] + 1)) + shift[seg]
    in bf16 operations.  scale, shift (segments, dim) bf16; seg (rows,) int32.
    Returns (out (rows, dim) bf16 bits, rstd (rows,), n or None)."""
    x = _c(x, np.uint16)
    rows, dim = x.shape
    w = None if weight is None else _c(weight, np.uint16)
    assert w is None or w.shape == (dim,)
    scale = _c(scale, np.uint16)
    shift = _c(shift, np.uint16)
    segments = scale.shape[0]
    assert scale.shape == shift.shape == (segments, dim)
    seg = _c(seg, np.int32)
    assert seg.shape == (rows,)
    out = np.empty((rows, dim), np.uint16)
    rstd = np.empty(rows, np.float32)
    n = np.empty((rows, dim), np.uint16) if want_n else None

    def run(r0, r1):
        lib().orc_rms_modulate_seg(_rowptr(x, r0, dim), None if w is None else _ptr(w),
                                   _ptr(scale), _ptr(shift), _rowptr(seg, r0, 1), segments,
                                   eps, r1 - r0, dim, _rowptr(out, r0, dim),
                                   _rowptr(rstd, r0, 1), _rowptr(n, r0, dim))
    _parallel(rows, threads, run)
    return out, rstd, n


# ---- MX block formats (R15) -------------------------------------------------

def e8m0_scale(amax, emax):
    return int(lib().orc_e8m0_scale(float(amax), int(emax)))


def e8m0_decode(code):
    return float(lib().orc_e8m0_decode(int(code)))


def mx_block_quant(v, fp4):
    """Blocks of 32 fp32 values -> (element codes (n,), scale codes (n/32,))."""
    v = _c(v, np.float32).ravel()
    assert v.size % 32 == 0
    codes = np.empty(v.size, np.uint8)
    scales = np.empty(v.size // 32, np.uint8)
    lib().orc_mx_block_quant_n(_ptr(v), v.size // 32, 1 if fp4 else 0, _ptr(codes), _ptr(scales))
    return codes, scales


def adaln_mxfp4(x, scale=None, shift=None, eps=1e-5, want_b=False, threads=1):
    """LN (scale = shift = None) or broadcast AdaLN -> bf16 stage -> MXFP4.
    Returns (packed (rows, dim/2), scales (rows, dim/32), mean, rstd, b)."""
    x = _c(x, np.uint16)
    rows, dim = x.shape
    assert dim % 32 == 0
    sc = None if scale is None else _c(scale, np.uint16)
    sh = None if shift is None else _c(shift, np.uint16)
    packed = np.empty((rows, dim // 2), np.uint8)
    scales = np.empty((rows, dim // 32), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    b = np.empty((rows, dim), np.float32) if want_b else None

    def run(r0, r1):
        lib().orc_adaln_mxfp4(_rowptr(x, r0, dim), _ptr(sc), _ptr(sh), eps, r1 - r0, dim,
                              _rowptr(packed, r0, dim // 2), _rowptr(scales, r0, dim // 32),
                              _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1), _rowptr(b, r0, dim))
    _parallel(rows, threads, run)
    return packed, scales, mean, rstd, b


def adaln_mxfp4_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, eps=1e-5, threads=1):
    """modfp8 AdaLN -> bf16 stage -> MXFP4: the MX block rule applied to the
    modfp8 FP4 path's bf16-staged values.  Returns (packed, scales, mean, rstd,
    b)."""
    _, _, mean, rstd, b = adaln_fp4_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, eps,
                                           want_b=True, threads=threads)
    rows, dim = b.shape
    codes, scales = mx_block_quant(b, fp4=True)
    return (fp4_pack(codes).reshape(rows, dim // 2), scales.reshape(rows, dim // 32), mean, rstd,
            b)


def adaln_mxfp8(x, scale=None, shift=None, eps=1e-5, want_y=False, threads=1):
    """LN (None operands), broadcast ((dim,)) or per-token ((rows, dim)) AdaLN ->
    MXFP8.  Returns (out (rows, dim) e4m3, scales (rows, dim/32), mean, rstd, y)."""
    x = _c(x, np.uint16)
    rows, dim = x.shape
    assert dim % 32 == 0
    sc = None if scale is None else _c(scale, np.uint16)
    sh = None if shift is None else _c(shift, np.uint16)
    per_token = sc is not None and sc.shape == (rows, dim)
    out = np.empty((rows, dim), np.uint8)
    scales = np.empty((rows, dim // 32), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    y = np.empty((rows, dim), np.float32) if want_y else None

    def run(r0, r1):
        lib().orc_adaln_mxfp8(_rowptr(x, r0, dim), _rowptr(sc, r0, dim) if per_token else _ptr(sc),
                              _rowptr(sh, r0, dim) if per_token else _ptr(sh),
                              1 if per_token else 0, eps, r1 - r0, dim, _rowptr(out, r0, dim),
                              _rowptr(scales, r0, dim // 32), _rowptr(mean, r0, 1),
                              _rowptr(rstd, r0, 1), _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, scales, mean, rstd, y


def _mxfp8_of(y):
    rows, dim = y.shape
    codes, scales = mx_block_quant(y, fp4=False)
    return codes.reshape(rows, dim), scales.reshape(rows, dim // 32)


def adaln_mxfp8_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, eps=1e-5, threads=1):
    """modfp8 AdaLN -> MXFP8: the MX block rule applied to the modfp8 FP8 path's
    fp32 y (which does not depend on act_scale).  Returns (out, scales, mean,
    rstd, y)."""
    _, mean, rstd, y = adaln_fp8_modfp8(x, scale_fp8, shift_fp8, scale_deq, shift_deq, 1.0, eps,
                                        want_y=True, threads=threads)
    out, scales = _mxfp8_of(y)
    return out, scales, mean, rstd, y


def awq_adaln_mxfp8(x, scale, shift, inv_s, eps=1e-5, threads=1):
    """AWQ AdaLN -> MXFP8: the broadcast y times inv_s[j] (one fp32 product, the
    value the FP8 AWQ path scales by 1 / act_scale), then the MX block rule.
    Returns (out, scales, mean, rstd, smoothed y)."""
    _, mean, rstd, y = awq_adaln_fp8(x, scale, shift, inv_s, 1.0, eps, want_y=True,
                                     threads=threads)
    smoothed = (y * bf16_to_f32(_c(inv_s, np.uint16))[None, :]).astype(np.float32)
    out, scales = _mxfp8_of(smoothed)
    return out, scales, mean, rstd, smoothed


def adaln_mxfp8_table(x, temb, table, shift_idx, scale_idx, eps=1e-5, want_y=False, threads=1):
    """Table form -> MXFP8.  Returns (out, scales, mean, rstd, y)."""
    x = _c(x, np.uint16)
    temb = _c(temb, np.uint16)
    table = _c(table, np.float32)
    rows, dim = x.shape
    chunks = temb.shape[1]
    assert dim % 32 == 0 and temb.shape == (rows, chunks, dim) and table.shape == (chunks, dim)
    out = np.empty((rows, dim), np.uint8)
    scales = np.empty((rows, dim // 32), np.uint8)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    y = np.empty((rows, dim), np.float32) if want_y else None

    def run(r0, r1):
        lib().orc_adaln_mxfp8_table(_rowptr(x, r0, dim), _rowptr(temb, r0, chunks * dim),
                                    _ptr(table), chunks, shift_idx, scale_idx, eps, r1 - r0, dim,
                                    _rowptr(out, r0, dim), _rowptr(scales, r0, dim // 32),
                                    _rowptr(mean, r0, 1), _rowptr(rstd, r0, 1),
                                    _rowptr(y, r0, dim))
    _parallel(rows, threads, run)
    return out, scales, mean, rstd, y


# ---- six-way modulation ---------------------------------------------------

def modulation6(params, mod, threads=1):
    """params (B, S, 6, D) fp32 + mod (6, D) fp32 -> (6, B, S, D) bf16 bits."""
    params = _c(params, np.float32)
    mod = _c(mod, np.float32)
    B, S, six, D = params.shape
    assert six == 6 and mod.shape == (6, D)
    tokens = B * S
    out = np.empty((6, tokens, D), np.uint16)
    if threads <= 1 or tokens < 2:
        lib().orc_modulation6(_ptr(params), _ptr(mod), tokens, D, _ptr(out))
    else:
        # Each block of tokens writes its own token range of every plane.
        parts = {}

        def run(t0, t1):
            o = np.empty((6, t1 - t0, D), np.uint16)
            lib().orc_modulation6(_rowptr(params, t0, 6 * D), _ptr(mod), t1 - t0,
                                  D, _ptr(o))
            parts[t0] = (t1, o)
        _parallel(tokens, threads, run)
        for t0, (t1, o) in parts.items():
            out[:, t0:t1] = o
    return out.reshape(6, B, S, D)
