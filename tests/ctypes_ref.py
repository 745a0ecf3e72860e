"""An independent ctypes marshalling of the package's functions.

Test infrastructure only.  The package's functions are its compiled binding
(csrc/torch_binding.cpp).  This module makes the same tensor checks and the
same C-ABI calls (include/alnp.h) in Python, through ctypes, so that the
tests can compare the two marshallings byte for byte and error for error.
Every function runs on the device of its first tensor, as the compiled one
does.  Nothing here computes: every step runs in libalnp.so's kernels.
"""
from __future__ import annotations

import ctypes
import functools

import torch

from dit_adaptive_layernorm_amd import AlnpError, lib, mx_scale_size, sf_size, swizzled_sf_size

_P = ctypes.c_void_p

def _check(fn: str, status: int) -> None:
    if status != 0:
        raise AlnpError(fn, status)


# The raw current stream of the current device, read without building a
# torch.cuda.Stream object (which costs microseconds per call).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


_device_index = _cur_device if _cur_device is not None else torch.cuda.current_device


def _stream() -> int:
    if _raw_stream is not None:
        return _raw_stream(_device_index())
    return torch.cuda.current_stream().cuda_stream


def _on_call_device(fn):
    """Run `fn` on the device of its first argument, a GPU tensor, as torch's
    own operators do: switch the current device only when it differs.  Every
    other tensor of the call must be on that device (checked by _dev)."""
    @functools.wraps(fn)
    def run(first, *args, **kwargs):
        if isinstance(first, torch.Tensor) and first.is_cuda and first.get_device() != _device_index():
            with torch.cuda.device(first.device):
                return fn(first, *args, **kwargs)
        return fn(first, *args, **kwargs)
    return run


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> int:
    """Device pointer of a contiguous tensor of the given dtype (and shape) on
    the call's GPU (the current device); raises with the reason otherwise."""
    try:
        if (t.dtype is dtype and t.is_cuda and t.get_device() == _device_index()
                and t.is_contiguous() and (shape is None or t.shape == shape)):
            return t.data_ptr()
    except AttributeError:
        pass
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.get_device() != _device_index():
        raise ValueError(f"{name} must be on cuda:{_device_index()}, the device of the call, "
                         f"got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name, shape):
    return None if t is None else _dev(t, name, torch.float32, shape)


def _x(x):
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, dim)")
    return x.shape


def _act(act_scale):
    p = _dev(act_scale, "act_scale", torch.float32)
    if act_scale.numel() != 1:
        raise ValueError("act_scale must hold one fp32 value")
    return p


def _fp8_out(out, x):
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    _dev(out, "out", torch.float8_e4m3fn, x.shape)
    return out


# ---- FP8 producers ----------------------------------------------------------

def ada_layer_norm_quant_fp8_bf16(x, scale, shift, act_scale, eps=1e-5, out=None,
                                  row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> FP8: scale, shift (dim,) bf16."""
    rows, dim = _x(x)
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_fp8_bf16", lib().alnp_ada_layer_norm_quant_fp8_bf16(
        x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (dim,)),
        _dev(shift, "shift", torch.bfloat16, (dim,)), _act(act_scale), eps, rows, dim,
        out.data_ptr(), _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
        _stream()))
    return out


def ada_layer_norm_quant_fp8_ptok_bf16(x, scale, shift, act_scale, eps=1e-5, out=None,
                                       row_mean=None, row_rstd=None):
    """Per-token AdaLN -> FP8: scale, shift (rows, dim) bf16."""
    rows, dim = _x(x)
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_fp8_ptok_bf16", lib().alnp_ada_layer_norm_quant_fp8_ptok_bf16(
        x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (rows, dim)),
        _dev(shift, "shift", torch.bfloat16, (rows, dim)), _act(act_scale), eps, rows, dim,
        out.data_ptr(), _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
        _stream()))
    return out


def ada_layer_norm_quant_fp8_ptok_table_bf16(x, temb, table, act_scale, shift_idx, scale_idx,
                                             eps=1e-5, out=None, row_mean=None, row_rstd=None):
    """Table-form per-token AdaLN -> FP8: temb (rows, chunks, dim) bf16, table
    (chunks, dim) fp32; operands temb[:, idx] + table[idx]."""
    rows, dim = _x(x)
    if temb.dim() != 3:
        raise ValueError("temb must be (rows, chunks, dim)")
    chunks = temb.shape[1]
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_fp8_ptok_table_bf16",
           lib().alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(
               x.data_ptr(), _dev(temb, "temb", torch.bfloat16, (rows, chunks, dim)),
               _dev(table, "table", torch.float32, (chunks, dim)), chunks, int(shift_idx),
               int(scale_idx), _act(act_scale), eps, rows, dim, out.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return out


def _scalar(t, name):
    p = _dev(t, name, torch.float32)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold one fp32 value")
    return p


def ada_layer_norm_quant_fp8_modfp8_bf16(x, scale_fp8, shift_fp8, scale_deq, shift_deq,
                                         act_scale, eps=1e-5, out=None, row_mean=None,
                                         row_rstd=None):
    """Broadcast AdaLN -> FP8 with e4m3 (dim,) scale/shift and fp32 device
    dequantization scalars."""
    rows, dim = _x(x)
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_fp8_modfp8_bf16",
           lib().alnp_ada_layer_norm_quant_fp8_modfp8_bf16(
               x.data_ptr(), _dev(scale_fp8, "scale_fp8", torch.float8_e4m3fn, (dim,)),
               _dev(shift_fp8, "shift_fp8", torch.float8_e4m3fn, (dim,)),
               _scalar(scale_deq, "scale_deq"), _scalar(shift_deq, "shift_deq"),
               _act(act_scale), eps, rows, dim, out.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return out


def awq_ada_layer_norm_quant_fp8_bf16(x, scale, shift, inv_s, act_scale, eps=1e-5, out=None,
                                      row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> per-channel inv_s (dim,) bf16 -> FP8."""
    rows, dim = _x(x)
    out = _fp8_out(out, x)
    _check("alnp_awq_ada_layer_norm_quant_fp8_bf16", lib().alnp_awq_ada_layer_norm_quant_fp8_bf16(
        x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (dim,)),
        _dev(shift, "shift", torch.bfloat16, (dim,)), _dev(inv_s, "inv_s", torch.bfloat16, (dim,)),
        _act(act_scale), eps, rows, dim, out.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
        _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return out


def layer_norm_no_affine_quant_fp8_static_bf16(x, act_scale, eps=1e-5, out=None,
                                               row_mean=None, row_rstd=None):
    """LayerNorm (no affine) -> FP8."""
    rows, dim = _x(x)
    out = _fp8_out(out, x)
    _check("alnp_layer_norm_no_affine_quant_fp8_static_bf16",
           lib().alnp_layer_norm_no_affine_quant_fp8_static_bf16(
               x.data_ptr(), _act(act_scale), eps, rows, dim, out.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return out


# ---- FP4 producer ------------------------------------------------------------



def layer_norm_no_affine_quant_nvfp4_bf16(x, eps=1e-5, packed=None, sf=None,
                                          row_mean=None, row_rstd=None):
    """LayerNorm (no affine) -> e2m1 packed (rows, dim // 2) uint8 (low nibble
    first) + e4m3 block scales (rows, dim // 16), row-major."""
    rows, dim = _x(x)
    if dim % 16:
        raise ValueError("dim must be a multiple of 16")
    if packed is None:
        packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rows, dim // 16), dtype=torch.float8_e4m3fn, device=x.device)
    _dev(packed, "packed", torch.uint8, (rows, dim // 2))
    if sf.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("sf must be uint8 or float8_e4m3fn")
    _dev(sf, "sf", sf.dtype, (rows, dim // 16))
    _check("alnp_layer_norm_no_affine_quant_nvfp4_bf16",
           lib().alnp_layer_norm_no_affine_quant_nvfp4_bf16(
               x.data_ptr(), eps, rows, dim, packed.data_ptr(), sf.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return packed, sf




def _fp4_outputs(x, rows, dim, packed, sf, swizzled):
    if dim % 16:
        raise ValueError("dim must be a multiple of 16")
    if packed is None:
        packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=x.device)
    n_sf = swizzled_sf_size(rows, dim) if swizzled else sf_size(rows, dim)
    if sf is None:
        sf = torch.empty((n_sf,) if swizzled else (rows, dim // 16), dtype=torch.uint8,
                         device=x.device)
    _dev(packed, "packed", torch.uint8, (rows, dim // 2))
    if sf.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("sf must be uint8 or float8_e4m3fn")
    _dev(sf, "sf", sf.dtype)
    if sf.numel() != n_sf:
        raise ValueError(f"sf must hold {n_sf} bytes, got {sf.numel()}")
    return packed, sf


def layer_norm_no_affine_quant_nvfp4_swizzled_bf16(x, eps=1e-5, packed=None, sf_swizzled=None,
                                                   row_mean=None, row_rstd=None):
    """LayerNorm (no affine) -> e2m1 packed + e4m3 block scales in the 128x4
    tiled layout."""
    rows, dim = _x(x)
    packed, sf = _fp4_outputs(x, rows, dim, packed, sf_swizzled, True)
    _check("alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16",
           lib().alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16(
               x.data_ptr(), eps, rows, dim, packed.data_ptr(), sf.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return packed, sf


def ada_layer_norm_quant_nvfp4_bf16(x, scale, shift, eps=1e-5, packed=None, sf=None,
                                    row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> e2m1 packed + row-major e4m3 block scales."""
    rows, dim = _x(x)
    packed, sf = _fp4_outputs(x, rows, dim, packed, sf, False)
    _check("alnp_ada_layer_norm_quant_nvfp4_bf16", lib().alnp_ada_layer_norm_quant_nvfp4_bf16(
        x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (dim,)),
        _dev(shift, "shift", torch.bfloat16, (dim,)), eps, rows, dim, packed.data_ptr(),
        sf.data_ptr(), _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
        _stream()))
    return packed, sf


def ada_layer_norm_quant_nvfp4_swizzled_bf16(x, scale, shift, eps=1e-5, packed=None,
                                             sf_swizzled=None, row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> e2m1 packed + e4m3 block scales in the 128x4 tiled
    layout."""
    rows, dim = _x(x)
    packed, sf = _fp4_outputs(x, rows, dim, packed, sf_swizzled, True)
    _check("alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16",
           lib().alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16(
               x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (dim,)),
               _dev(shift, "shift", torch.bfloat16, (dim,)), eps, rows, dim, packed.data_ptr(),
               sf.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
               _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return packed, sf


def ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(x, scale_fp8, shift_fp8, scale_deq, shift_deq,
                                                    eps=1e-5, packed=None, sf_swizzled=None,
                                                    row_mean=None, row_rstd=None):
    """AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars
    -> e2m1 packed + e4m3 block scales in the 128x4 tiled layout."""
    rows, dim = _x(x)
    packed, sf = _fp4_outputs(x, rows, dim, packed, sf_swizzled, True)
    _check("alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16",
           lib().alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
               x.data_ptr(), _dev(scale_fp8, "scale_fp8", torch.float8_e4m3fn, (dim,)),
               _dev(shift_fp8, "shift_fp8", torch.float8_e4m3fn, (dim,)),
               _scalar(scale_deq, "scale_deq"), _scalar(shift_deq, "shift_deq"), eps, rows, dim,
               packed.data_ptr(), sf.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
               _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return packed, sf


# ---- MX block formats (E8M0 scale per 32 elements) --------------------------------

_E8M0 = tuple(t for t in (torch.uint8, getattr(torch, "float8_e8m0fnu", None)) if t is not None)




def _mx_scales(x, rows, dim, scales):
    if dim % 32:
        raise ValueError("dim must be a multiple of 32")
    if scales is None:
        scales = torch.empty((rows, dim // 32), dtype=torch.uint8, device=x.device)
    if scales.dtype not in _E8M0:
        raise TypeError("scales must be uint8 (E8M0 bytes)")
    _dev(scales, "scales", scales.dtype, (rows, dim // 32))
    return scales


def _mxfp8(name, x, scale, shift, eps, out, scales, row_mean, row_rstd, op_shape):
    rows, dim = _x(x)
    scales = _mx_scales(x, rows, dim, scales)
    out = _fp8_out(out, x)
    ops = []
    if op_shape is not None:
        shp = op_shape(rows, dim)
        ops = [_dev(scale, "scale", torch.bfloat16, shp), _dev(shift, "shift", torch.bfloat16, shp)]
    _check(name, getattr(lib(), name)(
        x.data_ptr(), *ops, eps, rows, dim, out.data_ptr(), scales.data_ptr(),
        _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return out, scales


def layer_norm_no_affine_quant_mxfp8_bf16(x, eps=1e-5, out=None, scales=None, row_mean=None,
                                          row_rstd=None):
    """LayerNorm (no affine) -> MXFP8: e4m3 (rows, dim) + E8M0 (rows, dim // 32)."""
    return _mxfp8("alnp_layer_norm_no_affine_quant_mxfp8_bf16", x, None, None, eps, out, scales,
                  row_mean, row_rstd, None)


def ada_layer_norm_quant_mxfp8_bf16(x, scale, shift, eps=1e-5, out=None, scales=None,
                                    row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> MXFP8; scale, shift (dim,) bf16."""
    return _mxfp8("alnp_ada_layer_norm_quant_mxfp8_bf16", x, scale, shift, eps, out, scales,
                  row_mean, row_rstd, lambda r, d: (d,))


def ada_layer_norm_quant_mxfp8_ptok_bf16(x, scale, shift, eps=1e-5, out=None, scales=None,
                                         row_mean=None, row_rstd=None):
    """Per-token AdaLN -> MXFP8; scale, shift (rows, dim) bf16."""
    return _mxfp8("alnp_ada_layer_norm_quant_mxfp8_ptok_bf16", x, scale, shift, eps, out, scales,
                  row_mean, row_rstd, lambda r, d: (r, d))


def ada_layer_norm_quant_mxfp8_ptok_table_bf16(x, temb, table, shift_idx, scale_idx, eps=1e-5,
                                               out=None, scales=None, row_mean=None,
                                               row_rstd=None):
    """Table-form AdaLN -> MXFP8: temb (rows, chunks, dim) bf16, table (chunks, dim)
    fp32; operands temb[:, idx] + table[idx]."""
    rows, dim = _x(x)
    if temb.dim() != 3:
        raise ValueError("temb must be (rows, chunks, dim)")
    chunks = temb.shape[1]
    scales = _mx_scales(x, rows, dim, scales)
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16",
           lib().alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(
               x.data_ptr(), _dev(temb, "temb", torch.bfloat16, (rows, chunks, dim)),
               _dev(table, "table", torch.float32, (chunks, dim)), chunks, int(shift_idx),
               int(scale_idx), eps, rows, dim, out.data_ptr(), scales.data_ptr(),
               _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)),
               _stream()))
    return out, scales


def ada_layer_norm_quant_mxfp8_modfp8_bf16(x, scale_fp8, shift_fp8, scale_deq, shift_deq,
                                           eps=1e-5, out=None, scales=None, row_mean=None,
                                           row_rstd=None):
    """AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars
    -> MXFP8."""
    rows, dim = _x(x)
    scales = _mx_scales(x, rows, dim, scales)
    out = _fp8_out(out, x)
    _check("alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16",
           lib().alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16(
               x.data_ptr(), _dev(scale_fp8, "scale_fp8", torch.float8_e4m3fn, (dim,)),
               _dev(shift_fp8, "shift_fp8", torch.float8_e4m3fn, (dim,)),
               _scalar(scale_deq, "scale_deq"), _scalar(shift_deq, "shift_deq"), eps, rows, dim,
               out.data_ptr(), scales.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
               _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return out, scales


def awq_ada_layer_norm_quant_mxfp8_bf16(x, scale, shift, inv_s, eps=1e-5, out=None, scales=None,
                                        row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> per-channel inv_s (dim,) bf16 -> MXFP8."""
    rows, dim = _x(x)
    scales = _mx_scales(x, rows, dim, scales)
    out = _fp8_out(out, x)
    _check("alnp_awq_ada_layer_norm_quant_mxfp8_bf16",
           lib().alnp_awq_ada_layer_norm_quant_mxfp8_bf16(
               x.data_ptr(), _dev(scale, "scale", torch.bfloat16, (dim,)),
               _dev(shift, "shift", torch.bfloat16, (dim,)),
               _dev(inv_s, "inv_s", torch.bfloat16, (dim,)), eps, rows, dim, out.data_ptr(),
               scales.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
               _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return out, scales


def _mxfp4(name, x, scale, shift, eps, packed, scales, row_mean, row_rstd):
    rows, dim = _x(x)
    scales = _mx_scales(x, rows, dim, scales)
    if packed is None:
        packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=x.device)
    _dev(packed, "packed", torch.uint8, (rows, dim // 2))
    ops = [] if scale is None else [_dev(scale, "scale", torch.bfloat16, (dim,)),
                                    _dev(shift, "shift", torch.bfloat16, (dim,))]
    _check(name, getattr(lib(), name)(
        x.data_ptr(), *ops, eps, rows, dim, packed.data_ptr(), scales.data_ptr(),
        _opt(row_mean, "row_mean", (rows,)), _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return packed, scales


def layer_norm_no_affine_quant_mxfp4_bf16(x, eps=1e-5, packed=None, scales=None, row_mean=None,
                                          row_rstd=None):
    """LayerNorm (no affine) -> bf16 stage -> MXFP4: packed e2m1 (rows, dim // 2)
    + E8M0 (rows, dim // 32)."""
    return _mxfp4("alnp_layer_norm_no_affine_quant_mxfp4_bf16", x, None, None, eps, packed,
                  scales, row_mean, row_rstd)


def ada_layer_norm_quant_mxfp4_bf16(x, scale, shift, eps=1e-5, packed=None, scales=None,
                                    row_mean=None, row_rstd=None):
    """Broadcast AdaLN -> bf16 stage -> MXFP4; scale, shift (dim,) bf16."""
    return _mxfp4("alnp_ada_layer_norm_quant_mxfp4_bf16", x, scale, shift, eps, packed, scales,
                  row_mean, row_rstd)


def ada_layer_norm_quant_mxfp4_modfp8_bf16(x, scale_fp8, shift_fp8, scale_deq, shift_deq,
                                           eps=1e-5, packed=None, scales=None, row_mean=None,
                                           row_rstd=None):
    """AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars
    -> bf16 stage -> MXFP4."""
    rows, dim = _x(x)
    scales = _mx_scales(x, rows, dim, scales)
    if packed is None:
        packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=x.device)
    _dev(packed, "packed", torch.uint8, (rows, dim // 2))
    _check("alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16",
           lib().alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16(
               x.data_ptr(), _dev(scale_fp8, "scale_fp8", torch.float8_e4m3fn, (dim,)),
               _dev(shift_fp8, "shift_fp8", torch.float8_e4m3fn, (dim,)),
               _scalar(scale_deq, "scale_deq"), _scalar(shift_deq, "shift_deq"), eps, rows, dim,
               packed.data_ptr(), scales.data_ptr(), _opt(row_mean, "row_mean", (rows,)),
               _opt(row_rstd, "row_rstd", (rows,)), _stream()))
    return packed, scales


# ---- six-way modulation --------------------------------------------------------

def adaln_modulation6_bf16(adaln_params, layer_modulation, out=None):
    """fp32 (batch, seq, 6, dim) + fp32 (6, dim) -> six bf16 (batch, seq, dim)."""
    if adaln_params.dim() != 4 or adaln_params.shape[2] != 6:
        raise ValueError("adaln_params must be (batch, seq, 6, dim)")
    B, S, _, D = adaln_params.shape
    _dev(adaln_params, "adaln_params", torch.float32)
    _dev(layer_modulation, "layer_modulation", torch.float32, (6, D))
    if out is None:
        out = [torch.empty((B, S, D), dtype=torch.bfloat16, device=adaln_params.device)
               for _ in range(6)]
    if len(out) != 6:
        raise ValueError("out must hold six tensors")
    ptrs = (_P * 6)(*[_dev(o, f"out[{k}]", torch.bfloat16, (B, S, D)) for k, o in enumerate(out)])
    _check("alnp_adaln_modulation6_bf16", lib().alnp_adaln_modulation6_bf16(
        adaln_params.data_ptr(), layer_modulation.data_ptr(), B, S, D, ptrs, _stream()))
    return tuple(out)


# ---- residual gate ---------------------------------------------------------------

def gated_residual_bf16(residual, gate, proj, out=None):
    """out = bf16(residual + bf16(gate * proj)); gate (rows, dim) or (dim,).
    Pass out=residual to update the residual stream in place."""
    if residual.dim() != 2:
        raise ValueError("residual must be 2-D (rows, dim)")
    rows, dim = residual.shape
    _dev(residual, "residual", torch.bfloat16)
    _dev(proj, "proj", torch.bfloat16, (rows, dim))
    if tuple(gate.shape) == (dim,):
        gate_rows = 1
    elif tuple(gate.shape) == (rows, dim):
        gate_rows = rows
    else:
        raise ValueError(f"gate must be ({dim},) or ({rows}, {dim})")
    _dev(gate, "gate", torch.bfloat16)
    if out is None:
        out = torch.empty_like(residual)
    _dev(out, "out", torch.bfloat16, (rows, dim))
    _check("alnp_gated_residual_bf16", lib().alnp_gated_residual_bf16(
        residual.data_ptr(), gate.data_ptr(), proj.data_ptr(), rows, dim, gate_rows,
        out.data_ptr(), _stream()))
    return out


# ---- RMSNorm with segment-selected modulation -------------------------------------

def rms_norm_modulate_seg_bf16(x, weight, scale, shift, seg, eps=1e-5, out=None, row_rstd=None):
    """RMSNorm (weight (dim,) bf16 or None) then (n * (scale[seg] + 1)) + shift[seg]
    in bf16 operations.  scale, shift (segments, dim) bf16; seg (rows,) int32
    table row per row (outside [0, segments): NaN row).  Returns out (rows, dim)
    bf16."""
    rows, dim = _x(x)
    if scale.dim() != 2:
        raise ValueError("scale must be (segments, dim)")
    segments = scale.shape[0]
    wp = None if weight is None else _dev(weight, "weight", torch.bfloat16, (dim,))
    if out is None:
        out = torch.empty_like(x)
    _check("alnp_rms_norm_modulate_seg_bf16", lib().alnp_rms_norm_modulate_seg_bf16(
        x.data_ptr(), wp, _dev(scale, "scale", torch.bfloat16, (segments, dim)),
        _dev(shift, "shift", torch.bfloat16, (segments, dim)),
        _dev(seg, "seg", torch.int32, (rows,)), segments, eps, rows, dim,
        _dev(out, "out", torch.bfloat16, (rows, dim)), _opt(row_rstd, "row_rstd", (rows,)),
        _stream()))
    return out


# ---- standalone quantizer --------------------------------------------------------

def quant_fp8_static_f32(v, act_scale, out=None):
    """e4m3(v * (1 / act_scale)), saturating; v fp32 of any shape."""
    _dev(v, "v", torch.float32)
    if out is None:
        out = torch.empty(v.shape, dtype=torch.float8_e4m3fn, device=v.device)
    _dev(out, "out", torch.float8_e4m3fn, v.shape)
    _check("alnp_quant_fp8_static_f32", lib().alnp_quant_fp8_static_f32(
        v.data_ptr(), _act(act_scale), v.numel(), out.data_ptr(), _stream()))
    return out


NAMES = (
    "ada_layer_norm_quant_fp8_bf16", "ada_layer_norm_quant_fp8_ptok_bf16",
    "ada_layer_norm_quant_fp8_ptok_table_bf16", "ada_layer_norm_quant_fp8_modfp8_bf16",
    "awq_ada_layer_norm_quant_fp8_bf16", "layer_norm_no_affine_quant_fp8_static_bf16",
    "quant_fp8_static_f32", "layer_norm_no_affine_quant_nvfp4_bf16",
    "layer_norm_no_affine_quant_nvfp4_swizzled_bf16", "ada_layer_norm_quant_nvfp4_bf16",
    "ada_layer_norm_quant_nvfp4_swizzled_bf16", "ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16",
    "layer_norm_no_affine_quant_mxfp8_bf16", "ada_layer_norm_quant_mxfp8_bf16",
    "ada_layer_norm_quant_mxfp8_ptok_bf16", "ada_layer_norm_quant_mxfp8_ptok_table_bf16",
    "layer_norm_no_affine_quant_mxfp4_bf16", "ada_layer_norm_quant_mxfp4_bf16",
    "ada_layer_norm_quant_mxfp8_modfp8_bf16", "awq_ada_layer_norm_quant_mxfp8_bf16",
    "ada_layer_norm_quant_mxfp4_modfp8_bf16",
    "adaln_modulation6_bf16", "gated_residual_bf16", "rms_norm_modulate_seg_bf16",
)

# Each function runs on the device of its first tensor.
for _n in NAMES:
    globals()[_n] = _on_call_device(globals()[_n])
