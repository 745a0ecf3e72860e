"""Adaptive-LayerNorm producers for AMD MI355X (gfx950).

A thin binding over libalnp.so, the HIP library built from csrc/ (C ABI in
include/alnp.h).  The functions carry the names of the
"adaptive-layernorm-producers" README ("Available Functions") and follow its
"Tensor Contract": bf16 activations (rows, dim), broadcast / per-token /
table modulation operands, an fp32 device scalar act_scale, FP8 e4m3 or
packed FP4 e2m1 outputs, and optional caller-owned `out=` buffers for graph
capture.

The functions are the compiled binding _torch_binding (from
csrc/torch_binding.cpp): it checks the tensors and marshals pointers to the
C ABI in C++, on the current torch stream of the call's device.  Every step
runs in the HIP kernels.  If libalnp.so or the binding is missing, or the
binding is older than this package, the functions raise; there is no CPU
fallback.  `lib()` is the C ABI itself, through ctypes, with the signatures
of include/alnp.h.

FP4 block scales come in two layouts: the README's *_swizzled_* functions
write the 128x4 tiled layout (buffer size swizzled_sf_size(rows, dim)); the
functions without "swizzled" write plain row-major (rows, dim // 16) scales
(size sf_size(rows, dim)).
"""
from __future__ import annotations

import ctypes
import os
import sysconfig

import torch  # loads libtorch, which the compiled binding links against

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libalnp.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_I = ctypes.c_int

# name -> (argtypes, restype); mirrors include/alnp.h.
SIGNATURES = {
    "alnp_abi_version": ([], _I),
    "alnp_status_string": ([_I], ctypes.c_char_p),
    "alnp_ada_layer_norm_quant_fp8_bf16": ([_P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_fp8_ptok_bf16": ([_P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_fp8_ptok_table_bf16": (
        [_P, _P, _P, _I64, _I64, _I64, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_layer_norm_no_affine_quant_fp8_static_bf16": ([_P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_layer_norm_no_affine_quant_nvfp4_bf16": ([_P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_sf_size": ([_I64, _I64], _I64),
    "alnp_adaln_modulation6_bf16": ([_P, _P, _I64, _I64, _I64, ctypes.POINTER(_P), _P], _I),
    "alnp_quant_fp8_static_f32": ([_P, _P, _I64, _P, _P], _I),
    "alnp_ada_layer_norm_quant_fp8_modfp8_bf16": (
        [_P, _P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_awq_ada_layer_norm_quant_fp8_bf16": (
        [_P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P], _I),
    "alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16": ([_P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_nvfp4_bf16": ([_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16": (
        [_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_swizzled_sf_size": ([_I64, _I64], _I64),
    "alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16": (
        [_P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_layer_norm_no_affine_quant_mxfp8_bf16": ([_P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_mxfp8_bf16": ([_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_mxfp8_ptok_bf16": (
        [_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_layer_norm_no_affine_quant_mxfp4_bf16": ([_P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_mxfp4_bf16": ([_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_mx_scale_size": ([_I64, _I64], _I64),
    "alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16": (
        [_P, _P, _P, _I64, _I64, _I64, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16": (
        [_P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_awq_ada_layer_norm_quant_mxfp8_bf16": (
        [_P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16": (
        [_P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "alnp_gated_residual_bf16": ([_P, _P, _P, _I64, _I64, _I64, _P, _P], _I),
    "alnp_rms_norm_modulate_seg_bf16": (
        [_P, _P, _P, _P, _P, _I64, _F, _I64, _I64, _P, _P, _P], _I),
}

STATUS = {0: "ALNP_OK", -1: "ALNP_ERR_NULL", -2: "ALNP_ERR_SHAPE", -3: "ALNP_ERR_DIM",
          -4: "ALNP_ERR_INDEX", -5: "ALNP_ERR_ALIGN", -6: "ALNP_ERR_LAUNCH", -7: "ALNP_ERR_ARG"}

_lib = None


class AlnpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({lib().alnp_status_string(status).decode()})")


def lib() -> ctypes.CDLL:
    """The loaded libalnp.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m dit_adaptive_layernorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib

# ---- block-scale buffer sizes ------------------------------------------------------

def sf_size(rows: int, dim: int) -> int:
    """Bytes of the row-major e4m3 block-scale buffer: rows * dim // 16."""
    n = lib().alnp_sf_size(rows, dim)
    if n < 0:
        raise AlnpError("alnp_sf_size", int(n))
    return int(n)


def swizzled_sf_size(rows: int, dim: int) -> int:
    """Bytes of the 128x4 tiled block-scale buffer."""
    n = lib().alnp_swizzled_sf_size(rows, dim)
    if n < 0:
        raise AlnpError("alnp_swizzled_sf_size", int(n))
    return int(n)


def mx_scale_size(rows: int, dim: int) -> int:
    """Bytes of an MX scale buffer: rows * dim // 32."""
    n = lib().alnp_mx_scale_size(rows, dim)
    if n < 0:
        raise AlnpError("alnp_mx_scale_size", int(n))
    return int(n)


# ---- the functions: the compiled binding -------------------------------------------

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

_BINDING_PATH = os.path.join(_PKG, "_torch_binding" + sysconfig.get_config_var("EXT_SUFFIX"))
_compiled = None
_missing = f"{_BINDING_PATH} is missing: build it with `python -m dit_adaptive_layernorm_amd.build`"
if os.path.exists(_BINDING_PATH):
    # Built, so it must load: a binding that fails to import is an error.
    from . import _torch_binding as _loaded

    # A binding built from older sources lacks some functions: it is not
    # used, and every function raises until it is rebuilt (the build imports
    # this package before rebuilding it, so importing must still work).
    if all(hasattr(_loaded, _n) for _n in NAMES):
        _compiled = _loaded
        _compiled.set_error_class(AlnpError)
    else:
        _missing = f"{_BINDING_PATH} is older than the package: rebuild it with " \
                   "`python -m dit_adaptive_layernorm_amd.build`"


def _unbuilt(name):
    def call(*args, **kwargs):
        raise ImportError(f"{name}: {_missing}")
    call.__name__ = name
    return call


for _n in NAMES:
    globals()[_n] = getattr(_compiled, _n) if _compiled is not None else _unbuilt(_n)


def binding() -> str:
    """"compiled" when the compiled binding is loaded, "missing" otherwise
    (then every function raises ImportError)."""
    return "compiled" if _compiled is not None else "missing"


__all__ = [*NAMES, "sf_size", "swizzled_sf_size", "mx_scale_size", "lib", "AlnpError",
           "SIGNATURES", "binding"]
