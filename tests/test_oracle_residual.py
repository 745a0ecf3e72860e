"""Pins for the oracle's residual-gate step (h3-blackwell-runtime compare
page, the residual-gate epilogue's numerical program): out = bf16(residual +
bf16(gate * proj)).  torch's bf16 eager arithmetic (each op in fp32, rounded
to bf16) is an independent library implementation of that program."""
import numpy as np
import torch

from dit_adaptive_layernorm_amd import inputs


def t16(u):
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_bf16_eager(orc):
    rows, dim = 37, 1536
    res = inputs.normal_bf16((rows, dim), 1.0, 41, 1)
    gate = inputs.normal_bf16((rows, dim), 0.5, 41, 2)
    proj = inputs.normal_bf16((rows, dim), 2.0, 41, 3)
    got = orc.gated_residual(res, gate, proj)
    ref = bits(t16(res) + t16(gate) * t16(proj))
    assert np.array_equal(got, ref)


def test_broadcast_gate(orc):
    rows, dim = 9, 512
    res = inputs.normal_bf16((rows, dim), 1.0, 42, 1)
    gate = inputs.normal_bf16((dim,), 0.5, 42, 2)
    proj = inputs.normal_bf16((rows, dim), 2.0, 42, 3)
    got = orc.gated_residual(res, gate, proj)
    ref = bits(t16(res) + t16(gate)[None, :] * t16(proj))
    assert np.array_equal(got, ref)
    rep = np.ascontiguousarray(np.broadcast_to(gate, (rows, dim)))
    assert np.array_equal(got, orc.gated_residual(res, rep, proj))


def test_special_gates(orc):
    rows, dim = 4, 64
    res = inputs.normal_bf16((rows, dim), 1.0, 43, 1)
    proj = inputs.normal_bf16((rows, dim), 1.0, 43, 3)
    zero = np.zeros((rows, dim), np.uint16)
    assert np.array_equal(orc.gated_residual(res, zero, proj), res)
    one = inputs.to_bf16_bits(np.ones((rows, dim), np.float32))
    assert np.array_equal(orc.gated_residual(res, one, proj), bits(t16(res) + t16(proj)))


def test_gate_product_is_rounded_before_the_add(orc):
    """gate * proj = (1 + 2^-7)(1 - 2^-8) = 1 + 2^-8 - 2^-15 rounds to 1.0 in
    bf16 before it meets the residual 2^-8; 1 + 2^-8 is then a tie and rounds
    to 1.0.  Without the product's bf16 boundary the sum 1 + 2^-7 - 2^-15
    would round to 1 + 2^-7."""
    res = inputs.to_bf16_bits(np.array([[2.0 ** -8]], np.float32))
    gate = inputs.to_bf16_bits(np.array([[1.0 + 2.0 ** -7]], np.float32))
    proj = inputs.to_bf16_bits(np.array([[1.0 - 2.0 ** -8]], np.float32))
    got = orc.gated_residual(res, gate, proj)
    assert got[0, 0] == inputs.to_bf16_bits(np.array([1.0], np.float32))[0]
