"""Pins for the oracle's six-way modulation producer: fp32 (B, S, 6, D)
params plus an fp32 (6, D) table, summed and rounded to six bf16 (B, S, D)
tensors ("adaptive-layernorm-producers" README, "Tensor Contract";
Benchmark Results, "Six-way modulation producer")."""
import numpy as np
import torch

from dit_adaptive_layernorm_amd import inputs


def test_chunk_to_plane_mapping(orc):
    B, S, D = 2, 3, 16
    params = np.zeros((B, S, 6, D), np.float32)
    for k in range(6):
        params[:, :, k, :] = 10 * (k + 1)
    params += np.arange(S, dtype=np.float32)[None, :, None, None]
    mod = np.tile(np.arange(6, dtype=np.float32)[:, None], (1, D))
    out = orc.modulation6(params, mod)
    assert out.shape == (6, B, S, D)
    vals = (out.astype(np.uint32) << 16).view(np.float32)
    for k in range(6):
        for s in range(S):
            assert np.all(vals[k, :, s, :] == 10 * (k + 1) + s + k)


def test_bf16_ties(orc):
    D = 8
    params = np.ones((1, 1, 6, D), np.float32)
    mod = np.zeros((6, D), np.float32)
    mod[0] = 2.0**-8          # 1 + 2^-8: tie -> 1.0
    mod[1] = 3 * 2.0**-8      # 1 + 3*2^-8: tie -> 1 + 2^-6
    mod[2] = -1.0             # exact zero
    mod[3] = np.inf
    mod[4] = 3.4e38           # overflow to inf in fp32, stays inf
    mod[5] = 2.0**-7
    out = orc.modulation6(params, mod)[:, 0, 0, 0]
    assert list(out) == [0x3F80, 0x3F82, 0x0000, 0x7F80, 0x7F80, 0x3F81]


def test_random_vs_library_rounding(orc):
    d = inputs.make("mod6", batch=2, seq=37, dim=384, seed=3)
    out = orc.modulation6(d["params"], d["mod"])
    s = d["params"] + d["mod"][None, None]          # numpy fp32 add (IEEE)
    ref = torch.from_numpy(np.ascontiguousarray(np.moveaxis(s, 2, 0))).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_threads_identical(orc):
    d = inputs.make("mod6", batch=1, seq=41, dim=256, seed=4)
    a = orc.modulation6(d["params"], d["mod"])
    b = orc.modulation6(d["params"], d["mod"], threads=5)
    assert np.array_equal(a, b)
