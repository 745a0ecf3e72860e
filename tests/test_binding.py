"""The compiled binding without a GPU: once built, the package's functions
are its functions, and misuse caught before any GPU call (tensors not on the
GPU) raises the same exception type and message as the independent ctypes
marshalling in tests/ctypes_ref.py."""
import os

import pytest
import torch

import ctypes_ref
import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import build as hip_build


def test_compiled_binding_is_public_when_built():
    built = os.path.exists(hip_build.binding_path())
    assert alnp.binding() == ("compiled" if built else "missing")
    assert set(alnp.NAMES) == set(ctypes_ref.NAMES)
    for name in alnp.NAMES:
        if built:
            assert getattr(alnp, name) is getattr(alnp._compiled, name), name
        else:
            with pytest.raises(ImportError):
                getattr(alnp, name)()


def _cpu_cases():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    v = torch.zeros(64, dtype=torch.bfloat16)
    a = torch.tensor([0.025])
    seg = torch.zeros(4, dtype=torch.int32)
    return [
        ("ada_layer_norm_quant_fp8_bf16", (x, v, v, a)),
        ("ada_layer_norm_quant_fp8_ptok_bf16", (x, x, x, a)),
        ("layer_norm_no_affine_quant_fp8_static_bf16", (x, a)),
        ("layer_norm_no_affine_quant_nvfp4_bf16", (x,)),
        ("ada_layer_norm_quant_mxfp8_ptok_bf16", (x, x, x)),
        ("layer_norm_no_affine_quant_mxfp4_bf16", (x,)),
        ("rms_norm_modulate_seg_bf16", (x, v, x, x, seg)),
        ("gated_residual_bf16", (x, v, x)),
        ("quant_fp8_static_f32", (torch.zeros(8), a)),
    ]


@pytest.mark.skipif(alnp.binding() != "compiled", reason="compiled binding not built")
@pytest.mark.parametrize("name,args", _cpu_cases())
def test_cpu_tensors_rejected_alike(name, args):
    errs = []
    for fn in (getattr(alnp, name), getattr(ctypes_ref, name)):
        with pytest.raises(Exception) as e:
            fn(*args)
        errs.append(e.value)
    assert type(errs[0]) is type(errs[1]) is ValueError, (name, errs)
    assert str(errs[0]) == str(errs[1]), (name, errs)


def test_unbuilt_binding_raises_on_call():
    """Without the compiled binding (or with one older than the package) the
    functions exist but raise ImportError naming the build step: no fallback."""
    fn = alnp._unbuilt("ada_layer_norm_quant_fp8_ptok_bf16")
    with pytest.raises(ImportError, match="dit_adaptive_layernorm_amd.build"):
        fn(torch.zeros(2, 8, dtype=torch.bfloat16))
