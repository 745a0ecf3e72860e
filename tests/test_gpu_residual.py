"""Parity of the residual-gate step with the oracle, bit-exact, through the
C ABI: per-token gates (row kernel in every row shape, and the slot kernel
above the row shapes' largest dim) and broadcast gates (slot kernel), the
scalar fallback, in-place update, and a full Wan-size residual stream gated
by a six-way producer output."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import dev_bf16, dev_f32, host_u16, misaligned_like

pytestmark = pytest.mark.gpu


def make(rows, dim, seed, bcast):
    res = inputs.normal_bf16((rows, dim), 1.0, seed, 1)
    gate = inputs.normal_bf16((dim,) if bcast else (rows, dim), 0.5, seed, 2)
    proj = inputs.normal_bf16((rows, dim), 2.0, seed, 3)
    return res, gate, proj


@pytest.mark.parametrize("bcast", [False, True])
@pytest.mark.parametrize("rows,dim", [(1, 8), (3, 3072), (5, 1536), (7, 1152), (130, 512),
                                      (2, 6), (3, 1030), (4, 12000), (1, 7), (2, 32768),
                                      (1, 40000), (3, 24), (9, 5376)])
def test_shapes(orc, bcast, rows, dim):
    print(f"gated residual bcast={bcast} rows={rows} dim={dim}", flush=True)
    res, gate, proj = make(rows, dim, rows + dim, bcast)
    out = alnp.gated_residual_bf16(dev_bf16(res), dev_bf16(gate), dev_bf16(proj))
    assert np.array_equal(host_u16(out), orc.gated_residual(res, gate, proj))


def test_in_place(orc):
    res, gate, proj = make(67, 3072, 51, False)
    r = dev_bf16(res)
    out = alnp.gated_residual_bf16(r, dev_bf16(gate), dev_bf16(proj), out=r)
    assert out.data_ptr() == r.data_ptr()
    assert np.array_equal(host_u16(r), orc.gated_residual(res, gate, proj))


def test_unaligned_fallback(orc):
    res, gate, proj = make(9, 3072, 52, False)
    r = misaligned_like((9, 3072), torch.bfloat16)
    r.copy_(dev_bf16(res))
    out = alnp.gated_residual_bf16(r, dev_bf16(gate), dev_bf16(proj))
    assert np.array_equal(host_u16(out), orc.gated_residual(res, gate, proj))


def test_full_size_with_six_way_gate(orc):
    """The MSA residual update of a DiT block at B1 S5070 D3072: the gate is
    chunk 2 of the six-way producer's output."""
    m = inputs.make("mod6", batch=1, seq=5070, dim=3072, seed=53)
    outs = alnp.adaln_modulation6_bf16(dev_f32(m["params"]), dev_f32(m["mod"]))
    gate = outs[2][0]
    res = inputs.normal_bf16((5070, 3072), 1.0, 53, 1)
    proj = inputs.normal_bf16((5070, 3072), 2.0, 53, 3)
    out = alnp.gated_residual_bf16(dev_bf16(res), gate, dev_bf16(proj))
    ref = orc.gated_residual(res, host_u16(gate), proj)
    assert np.array_equal(host_u16(out), ref)


def test_matches_torch_bf16_eager():
    res, gate, proj = make(300, 3072, 54, False)
    r, g, p = dev_bf16(res), dev_bf16(gate), dev_bf16(proj)
    out = alnp.gated_residual_bf16(r, g, p)
    ref = (r.float() + (g.float() * p.float()).to(torch.bfloat16).float()).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
