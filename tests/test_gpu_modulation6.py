"""Parity of the six-way modulation producer with the oracle, bit-exact,
through the C ABI: small and ragged shapes (vector and scalar kernels), the
full B1 S5070 D3072 workload on every token, and unaligned outputs."""
import numpy as np
import pytest
import torch

import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs
from parity import dev_f32, host_u16, misaligned_like

pytestmark = pytest.mark.gpu


def run_gpu(params, mod, out=None):
    outs = alnp.adaln_modulation6_bf16(dev_f32(params), dev_f32(mod), out=out)
    return np.stack([host_u16(o) for o in outs])


@pytest.mark.parametrize("B,S,D", [(1, 51, 1536), (2, 7, 3072), (1, 1, 8), (3, 5, 1152),
                                   (1, 4, 12), (2, 3, 7), (1, 2, 1), (1, 3, 5000)])
def test_small_shapes(orc, B, S, D):
    print(f"mod6 B={B} S={S} D={D}", flush=True)
    d = inputs.make("mod6", batch=B, seq=S, dim=D, seed=B * S + D)
    got = run_gpu(d["params"], d["mod"])
    assert np.array_equal(got, orc.modulation6(d["params"], d["mod"]))


def test_full_size_workload(orc):
    d = inputs.workload("modulation6_1x5070x3072")
    got = run_gpu(d["params"], d["mod"])
    assert np.array_equal(got, orc.modulation6(d["params"], d["mod"], threads=8))  # every token


def test_unaligned_outputs(orc):
    d = inputs.make("mod6", batch=1, seq=9, dim=3072, seed=2)
    out = [misaligned_like((1, 9, 3072), torch.bfloat16, elem_offset=k + 1) for k in range(6)]
    got = run_gpu(d["params"], d["mod"], out=out)
    assert np.array_equal(got, orc.modulation6(d["params"], d["mod"]))


def test_specials(orc):
    D = 16
    params = np.zeros((1, 2, 6, D), np.float32)
    params[0, 0, :, 0] = [1.0, 1.0, 3.0e38, -3.0e38, 1e-40, -0.0]
    mod = np.zeros((6, D), np.float32)
    mod[:, 0] = [2.0**-8, 3 * 2.0**-8, 3.0e38, -3.0e38, 1e-40, 0.0]
    got = run_gpu(params, mod)
    assert np.array_equal(got, orc.modulation6(params, mod))
