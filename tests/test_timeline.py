"""The measurement-only timeline build (libalnp_timeline.so): the FP8 row and
table kernels with per-wave clock records.  CPU: the library loads and
exports the product's entry points plus alnp_timeline_set; the benchmark's
summary of a record array gives the phases and the per-CU dispatch order it
is built from.  GPU: the timeline build writes the same output bytes as the
product library, and every wave leaves one complete record whose clock reads
follow the order of its work."""
import ctypes
import os

import numpy as np
import pytest
import torch

import bench
import dit_adaptive_layernorm_amd as alnp
from dit_adaptive_layernorm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "libalnp_timeline.so")


def test_timeline_library_exports_the_abi_and_its_setter():
    if not os.path.exists(PATH):
        pytest.fail("libalnp_timeline.so is not built (run the build)")
    L = bench.timeline_lib(alnp)
    assert L is not None
    for name in alnp.SIGNATURES:
        assert hasattr(L, name), name
    assert hasattr(L, "alnp_timeline_set")


def fake_records(rows, waves):
    """Records as the kernels write them: start, x issued, x landed, rstd,
    stores issued, stores done (100 MHz ticks), XCC_ID, HW_ID; two CUs."""
    rec = np.zeros((rows * 8, 8), np.int64)
    base = 10_000
    for r in range(rows):
        cu = r % 2
        start = base + 3 * (r // 2)
        for w in range(waves):
            t = [start + w, start + w + 5, base + 100 + 10 * (r // 2), 0, 0, 0]
            t[3] = t[2] + 40
            t[4] = t[3] + 30
            t[5] = t[4] + 7
            rec[r * waves + w, :6] = t
            rec[r * waves + w, 6] = 2                   # XCC 2
            rec[r * waves + w, 7] = (cu << 8) | (w << 4)  # CU id in bits 11:8
    return rec


def test_timeline_summary_of_known_records():
    rows, waves = 6, 2
    s = bench.timeline_summary(fake_records(rows, waves), rows)
    assert s["waves_per_row"] == waves and s["cus"] == 2
    # last rows: x landed at 10_000 + 100 + 20, stores done 77 ticks later
    assert s["end_us"] == pytest.approx((100 + 20 + 40 + 30 + 7) / 100.0)
    assert s["rstd_after_x"][2] == pytest.approx(0.40)
    assert s["output_pass"][2] == pytest.approx(0.30)
    # on each CU the rows in dispatch order landed at 100, 110, 120 ticks
    assert s["x_landed_by_order_on_cu"] == pytest.approx([1.0, 1.1, 1.2])
    # a missing wave record is reported, not summarized
    rec = fake_records(rows, waves)
    rec[3, :] = 0
    assert "error" in bench.timeline_summary(rec, rows)


@pytest.mark.gpu
@pytest.mark.parametrize("name,rows", [("ptok_fp8_2520x3072", 600), ("table_fp8_2520x3072", 600),
                                       ("ln_fp8_2520x3072", 257), ("awq_fp8_2520x3072", 600),
                                       ("bcast_fp8_16x2048", 16)])
def test_timeline_build_matches_the_product_and_records_every_wave(name, rows):
    print(f"timeline {name} rows={rows}", flush=True)
    L = bench.timeline_lib(alnp)
    assert L is not None
    kind = name.split("_")[0]
    dim = 2048 if name.startswith("bcast") else 3072
    d = inputs.make(kind, rows=rows, dim=dim)
    prod = bench.Producer(name, d, 1, torch, alnp)
    (fn, args), = prod.calls
    stream = torch.cuda.current_stream()
    outs = [t for t in prod.keep[0] if isinstance(t, torch.Tensor) and t.dtype == torch.uint8]
    assert fn(*args, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    buf = torch.zeros(rows * 8 * 8, dtype=torch.int64, device="cuda")
    assert L.alnp_timeline_set(buf.data_ptr()) == 0
    try:
        assert getattr(L, fn.__name__)(*args, stream.cuda_stream) == 0
        torch.cuda.synchronize()
    finally:
        L.alnp_timeline_set(None)
        torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)
    rec = buf.cpu().numpy().reshape(rows * 8, 8)
    waves = np.count_nonzero(rec[:, 0]) // rows
    assert waves == 2
    r = rec[: rows * waves]
    assert np.all(r[:, 0] > 0) and not np.any(rec[rows * waves:])
    assert np.all(np.diff(r[:, :6], axis=1) >= 0)
    assert "error" not in bench.timeline_summary(rec, rows)
