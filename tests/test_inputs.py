"""The seeded input generators: deterministic, right shapes and spreads."""
import numpy as np

from dit_adaptive_layernorm_amd import inputs


def f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_deterministic_and_stream_separated():
    a = inputs.make("ptok", rows=8, dim=64, seed=0)
    b = inputs.make("ptok", rows=8, dim=64, seed=0)
    c = inputs.make("ptok", rows=8, dim=64, seed=1)
    for k in ("x", "scale", "shift"):
        assert np.array_equal(a[k], b[k])
        assert not np.array_equal(a[k], c[k])
    assert not np.array_equal(a["scale"], a["shift"])


def test_workload_shapes():
    w = inputs.WORKLOADS
    assert w["ptok_fp8_2520x3072"]["rows"] == 2520
    d = inputs.make("table", rows=5, dim=32, chunks=6)
    assert d["temb"].shape == (5, 6, 32) and d["table"].shape == (6, 32)
    assert d["table"].dtype == np.float32 and d["temb"].dtype == np.uint16
    m = inputs.make("mod6", batch=1, seq=3, dim=16)
    assert m["params"].shape == (1, 3, 6, 16) and m["mod"].shape == (6, 16)


def test_spreads():
    d = inputs.make("ptok", rows=64, dim=1024, seed=2)
    assert abs(f32(d["x"]).std() - 1.0) < 0.02
    assert abs(f32(d["scale"]).std() - 0.1) < 0.002
    t = inputs.make("table", rows=64, dim=512, seed=2)
    assert abs(f32(t["temb"]).std() - 0.5) < 0.01


def test_outlier_fraction():
    x = f32(inputs.make("fp4", rows=256, dim=1024, seed=0)["x"])
    base = f32(inputs.normal_bf16((256, 1024), 1.0, 0, inputs.STREAM["x"]))
    frac = np.mean(x != base)
    assert 0.008 < frac < 0.012
    assert np.abs(x).max() > 40


def test_device_draws_deterministic_and_whole():
    """The device-side generator (used for calls past 2^32 elements), run on
    torch's CPU generator: the same seed and stream give the same tensor,
    another stream another one; a size that is not a multiple of the chunk
    is filled completely; spreads and dtypes as asked."""
    import torch
    kw = dict(device="cpu", chunk=1000)
    a = inputs.device_normal((37, 129), 0.5, 3, inputs.STREAM["x"], **kw)
    b = inputs.device_normal((37, 129), 0.5, 3, inputs.STREAM["x"], **kw)
    c = inputs.device_normal((37, 129), 0.5, 3, inputs.STREAM["scale"], **kw)
    assert a.dtype == torch.bfloat16 and a.shape == (37, 129)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    f = a.float()
    assert abs(f.std().item() - 0.5) < 0.03
    # The tail past the last whole chunk (37 * 129 = 4773 = 4 * 1000 + 773)
    # is drawn too: no zeros left from the allocation.
    assert torch.count_nonzero(f.view(-1)[4000:]).item() >= 770
    p = inputs.device_normal((2, 3, 6, 8), 1.0, 3, inputs.STREAM["params"], dtype=torch.float32, **kw)
    assert p.dtype == torch.float32 and p.shape == (2, 3, 6, 8)
