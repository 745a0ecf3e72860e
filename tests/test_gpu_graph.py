"""The entry points inside a captured HIP graph: six producers captured
once into static output buffers, then replayed several times with eager work
and synchronizations in between; every replay must reproduce the eager
results byte for byte (the README's static-buffer / graph-capture usage)."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import act, dev_bf16, dev_f32, host_u8, host_u16

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    rows, dim = 257, 3072
    p = inputs.make("ptok", rows=rows, dim=dim, seed=61)
    t = inputs.make("table", rows=rows, dim=dim, seed=62)
    f = inputs.make("fp4", rows=rows, dim=dim, seed=63)
    m = inputs.make("mod6", batch=1, seq=rows, dim=dim, seed=64)
    r = inputs.make("rmsmod", rows=rows, dim=dim, seed=66)
    rx, rw, rsc, rsh = (dev_bf16(r[k]) for k in ("x", "weight", "scale", "shift"))
    rseg = torch.from_numpy(r["seg"]).cuda()
    x, sc, sh = dev_bf16(p["x"]), dev_bf16(p["scale"]), dev_bf16(p["shift"])
    tx, te, tb = dev_bf16(t["x"]), dev_bf16(t["temb"]), dev_f32(t["table"])
    fx = dev_bf16(f["x"])
    mp, mm = dev_f32(m["params"]), dev_f32(m["mod"])
    a = act()

    # Static outputs, as a captured producer would use them.
    o_ptok = torch.empty((rows, dim), dtype=torch.float8_e4m3fn, device="cuda")
    o_tab = torch.empty_like(o_ptok)
    o_pk = torch.empty((rows, dim // 2), dtype=torch.uint8, device="cuda")
    o_sf = torch.empty((alnp.swizzled_sf_size(rows, dim),), dtype=torch.uint8, device="cuda")
    o_m6 = [torch.empty((1, rows, dim), dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    o_res = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    o_rms = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    res = dev_bf16(inputs.normal_bf16((rows, dim), 1.0, 65, 1))
    proj = dev_bf16(inputs.normal_bf16((rows, dim), 1.0, 65, 2))

    def run_all():
        alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, sc, sh, a, out=o_ptok)
        alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(tx, te, tb, a, 0, 1, out=o_tab)
        alnp.layer_norm_no_affine_quant_nvfp4_swizzled_bf16(fx, packed=o_pk, sf_swizzled=o_sf)
        alnp.adaln_modulation6_bf16(mp, mm, out=o_m6)
        alnp.gated_residual_bf16(res, o_m6[2][0], proj, out=o_res)
        alnp.rms_norm_modulate_seg_bf16(rx, rw, rsc, rsh, rseg, out=o_rms)

    def scribble():
        # Fixed patterns over every output.  Bytes a producer does not own
        # (the tiled scale buffer's padding rows) keep the pattern.
        for o in (o_ptok, o_tab):
            o.view(torch.uint8).fill_(0x55)
        o_pk.fill_(0x77)
        o_sf.fill_(0x33)
        for o in o_m6 + [o_res, o_rms]:
            o.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()

    def snapshot():
        torch.cuda.synchronize()
        return [host_u8(o_ptok), host_u8(o_tab), host_u8(o_pk), host_u8(o_sf)] + \
               [host_u16(o) for o in o_m6] + [host_u16(o_res), host_u16(o_rms)]

    scribble()
    run_all()
    eager = snapshot()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_all()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()

    for replay in range(4):
        # Scribble over the outputs with eager work, then replay.
        scribble()
        g.replay()
        got = snapshot()
        for k, (u, v) in enumerate(zip(got, eager)):
            assert np.array_equal(u, v), f"replay {replay}, output {k}"
