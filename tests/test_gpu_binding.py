"""The compiled binding against the independent ctypes marshalling of
tests/ctypes_ref.py on the GPU: for every function, the same inputs give the same bytes (outputs, block scales, row
statistics), with outputs allocated by the call or passed in; misuse raises
the same exception type on both paths (dtype: TypeError; shape, contiguity:
ValueError; a status from the library: AlnpError with the same status)."""
import numpy as np
import pytest
import torch

import ctypes_ref
import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import act, dev_bf16, dev_f32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(alnp.binding() != "compiled", reason="compiled binding not built")]

ROWS, DIM = 37, 256


def e4m3(n, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, generator=g) * 0.3).to(torch.float8_e4m3fn).cuda()


def cases():
    """name -> positional arguments, as fresh GPU tensors."""
    f8 = inputs.make("ptok", rows=ROWS, dim=DIM, seed=1)
    bc = inputs.make("bcast", rows=ROWS, dim=DIM, seed=2)
    tb = inputs.make("table", rows=ROWS, dim=DIM, seed=3, shift_idx=4, scale_idx=2)
    fp4 = inputs.make("fp4", rows=ROWS, dim=DIM, seed=4)
    rm = inputs.make("rmsmod", rows=ROWS, dim=DIM, seed=5, segments=3)
    m6 = inputs.make("mod6", batch=1, seq=9, dim=DIM, seed=6)
    x, xb, x4 = dev_bf16(f8["x"]), dev_bf16(bc["x"]), dev_bf16(fp4["x"])
    a = act(f8["act_scale"])
    s_deq = torch.tensor([0.5], device="cuda")
    h_deq = torch.tensor([0.25], device="cuda")
    return {
        "ada_layer_norm_quant_fp8_bf16": (xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"]), a),
        "ada_layer_norm_quant_fp8_ptok_bf16": (x, dev_bf16(f8["scale"]), dev_bf16(f8["shift"]), a),
        "ada_layer_norm_quant_fp8_ptok_table_bf16": (
            dev_bf16(tb["x"]), dev_bf16(tb["temb"]), dev_f32(tb["table"]), a, 4, 2),
        "ada_layer_norm_quant_fp8_modfp8_bf16": (xb, e4m3(DIM, 7), e4m3(DIM, 8), s_deq, h_deq, a),
        "awq_ada_layer_norm_quant_fp8_bf16": (
            xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"]),
            (1.0 + 0.1 * torch.randn(DIM, device="cuda")).bfloat16(), a),
        "layer_norm_no_affine_quant_fp8_static_bf16": (x, a),
        "quant_fp8_static_f32": (torch.randn(5, 77, device="cuda") * 20, a),
        "layer_norm_no_affine_quant_nvfp4_bf16": (x4,),
        "layer_norm_no_affine_quant_nvfp4_swizzled_bf16": (x4,),
        "ada_layer_norm_quant_nvfp4_bf16": (xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"])),
        "ada_layer_norm_quant_nvfp4_swizzled_bf16": (xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"])),
        "ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16": (xb, e4m3(DIM, 9), e4m3(DIM, 10), s_deq, h_deq),
        "layer_norm_no_affine_quant_mxfp8_bf16": (x,),
        "ada_layer_norm_quant_mxfp8_bf16": (xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"])),
        "ada_layer_norm_quant_mxfp8_ptok_bf16": (x, dev_bf16(f8["scale"]), dev_bf16(f8["shift"])),
        "ada_layer_norm_quant_mxfp8_ptok_table_bf16": (
            dev_bf16(tb["x"]), dev_bf16(tb["temb"]), dev_f32(tb["table"]), 4, 2),
        "layer_norm_no_affine_quant_mxfp4_bf16": (x4,),
        "ada_layer_norm_quant_mxfp4_bf16": (xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"])),
        "ada_layer_norm_quant_mxfp8_modfp8_bf16": (xb, e4m3(DIM, 11), e4m3(DIM, 12), s_deq, h_deq),
        "awq_ada_layer_norm_quant_mxfp8_bf16": (
            xb, dev_bf16(bc["scale"]), dev_bf16(bc["shift"]),
            (1.0 + 0.1 * torch.randn(DIM, device="cuda")).bfloat16()),
        "ada_layer_norm_quant_mxfp4_modfp8_bf16": (xb, e4m3(DIM, 13), e4m3(DIM, 14), s_deq, h_deq),
        "adaln_modulation6_bf16": (dev_f32(m6["params"]), dev_f32(m6["mod"])),
        "gated_residual_bf16": (x, dev_bf16(f8["scale"]), dev_bf16(f8["shift"])),
        "rms_norm_modulate_seg_bf16": (
            dev_bf16(rm["x"]), dev_bf16(rm["weight"]), dev_bf16(rm["scale"]),
            dev_bf16(rm["shift"]), torch.from_numpy(rm["seg"]).cuda()),
    }


# Functions that also fill row statistics (row_mean and / or row_rstd).
STATS = {n: ("row_mean", "row_rstd") for n in alnp.NAMES
         if n not in ("quant_fp8_static_f32", "adaln_modulation6_bf16", "gated_residual_bf16",
                      "rms_norm_modulate_seg_bf16")}
STATS["rms_norm_modulate_seg_bf16"] = ("row_rstd",)


def as_bytes(r):
    if isinstance(r, (tuple, list)):
        return [as_bytes(t) for t in r]
    return r.contiguous().view(torch.uint8).cpu().numpy()


def run(fn, args, stats):
    kw = {k: torch.full((args[0].shape[0],), -1.0, device="cuda") for k in stats}
    r = fn(*args, **kw)
    torch.cuda.synchronize()
    return as_bytes(r), {k: v.cpu().numpy().view(np.uint32) for k, v in kw.items()}


@pytest.mark.parametrize("name", alnp.NAMES)
def test_same_bytes_as_ctypes(name):
    print(f"binding {name}", flush=True)
    args = cases()[name]
    stats = STATS.get(name, ())
    got, got_s = run(getattr(alnp, name), args, stats)
    ref, ref_s = run(getattr(ctypes_ref, name), args, stats)
    got = got if isinstance(got, list) else [got]
    ref = ref if isinstance(ref, list) else [ref]
    assert len(got) == len(ref), name
    for g, r in zip(got, ref):
        assert g.shape == r.shape and np.array_equal(g, r), name
    for k in stats:
        assert np.array_equal(got_s[k], ref_s[k]), (name, k)


def test_outputs_passed_in_are_written_and_returned():
    args = cases()
    x, sc, sh, a = args["ada_layer_norm_quant_fp8_ptok_bf16"]
    out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device="cuda")
    r = alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, sc, sh, a, out=out)
    assert r.data_ptr() == out.data_ptr()
    x4 = args["layer_norm_no_affine_quant_nvfp4_swizzled_bf16"][0]
    packed = torch.empty((ROWS, DIM // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((alnp.swizzled_sf_size(ROWS, DIM),), dtype=torch.uint8, device="cuda")
    p, s = alnp.layer_norm_no_affine_quant_nvfp4_swizzled_bf16(x4, packed=packed, sf_swizzled=sf)
    assert p.data_ptr() == packed.data_ptr() and s.data_ptr() == sf.data_ptr()
    params, mod = args["adaln_modulation6_bf16"]
    outs = [torch.empty((1, 9, DIM), dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    r6 = alnp.adaln_modulation6_bf16(params, mod, out=outs)
    assert [t.data_ptr() for t in r6] == [t.data_ptr() for t in outs]
    torch.cuda.synchronize()
    ref = ctypes_ref.adaln_modulation6_bf16(params, mod)
    for t, u in zip(r6, ref):
        assert torch.equal(t.view(torch.int16), u.view(torch.int16))


def _errors(name, args, kwargs=None):
    out = []
    for fn in (getattr(alnp, name), getattr(ctypes_ref, name)):
        with pytest.raises(Exception) as e:
            fn(*args, **(kwargs or {}))
        out.append(e.value)
    return out


def test_misuse_raises_alike():
    args = cases()
    x, sc, sh, a = args["ada_layer_norm_quant_fp8_ptok_bf16"]
    e = _errors("ada_layer_norm_quant_fp8_ptok_bf16", (x.float(), sc, sh, a))   # dtype
    assert type(e[0]) is type(e[1]) is TypeError, e
    for bad in [(x, sc[:-1], sh, a),                            # shape
                (x.t().contiguous().t(), sc, sh, a),            # not contiguous
                (x, sc, sh, torch.ones(2, device="cuda"))]:     # act_scale size
        e = _errors("ada_layer_norm_quant_fp8_ptok_bf16", bad)
        assert type(e[0]) is type(e[1]) is ValueError, e
        assert str(e[0]) == str(e[1]), e
    # A status from the library: a table index outside [0, chunks).
    xt, temb, table, at, _, _ = args["ada_layer_norm_quant_fp8_ptok_table_bf16"]
    e = _errors("ada_layer_norm_quant_fp8_ptok_table_bf16", (xt, temb, table, at, 6, 2))
    assert type(e[0]) is type(e[1]) is alnp.AlnpError and e[0].status == e[1].status == -4, e
    # Block scales of the wrong size.
    x4 = args["layer_norm_no_affine_quant_nvfp4_swizzled_bf16"][0]
    small = torch.empty((7,), dtype=torch.uint8, device="cuda")
    e = _errors("layer_norm_no_affine_quant_nvfp4_swizzled_bf16", (x4,), {"sf_swizzled": small})
    assert type(e[0]) is type(e[1]) is ValueError and str(e[0]) == str(e[1]), e


def test_tensor_off_the_call_device_is_rejected(monkeypatch):
    """Every function runs on its first tensor's device and takes no tensor
    from another.  With one GPU a second device cannot be made, so the ctypes
    path is shown a call device of cuda:1: its cuda:0 tensors must then be
    rejected (ValueError naming both devices) before anything is launched."""
    args = cases()
    res, gate, proj = args["gated_residual_bf16"]
    before = res.clone()
    monkeypatch.setattr(ctypes_ref, "_device_index", lambda: 1)
    with pytest.raises(ValueError, match=r"must be on cuda:1, the device of the call, got cuda:0"):
        ctypes_ref.gated_residual_bf16(res, gate, proj, out=res)
    monkeypatch.undo()
    torch.cuda.synchronize()
    assert torch.equal(res, before)
