"""Benchmark of the adaptive-LayerNorm producers on one MI355X.

One step = one call of the per-token AdaLN -> FP8 producer (LayerNorm
statistics, per-token modulation, static-scale e4m3 quantization: the whole
FP8 hot path) at the Wan-video 2520 x 3072 shape the pages time, with inputs
resident in HBM.  Headline: achieved algorithmic HBM GB/s (and us/call),
timed COLD: consecutive steps rotate over enough input/output sets (>= 512 MB)
that the 256 MB Infinity Cache cannot serve a step's operands from a previous
step.  Launches are replayed from a HIP graph (the pages' graph method:
several launches per graph, time / launches).

The other producers (broadcast and table FP8, LN -> FP8, LN -> FP4,
six-way modulation, RMSNorm modulation, the MXFP8 / MXFP4 outputs, the
modfp8 and AWQ FP8 forms, AdaLN -> FP4 with row-major and with tiled modfp8
scales, and the residual gate) are timed the same way at their workload
sizes and reported under "rows", each beside its memory-only floor; the
headline JSON line is the per-token FP8 one.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only-headline] [--direct]

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
COLD_FOOTPRINT = 512 << 20     # 2x the Infinity Cache
# Plain copies used to scale the rocprofv3 byte counters: about the per-token
# workload's bytes, 256 MiB, and about the six-way workload's bytes.
COPY_SIZES = (54 << 20, 256 << 20, 560 << 20)
COUNTER_MAX_STEPS = 20
THOR_PTOK_US = 229.922         # pages: NVIDIA Thor, per-token M2520 D3072, raw op
REPEATS = 5                    # timed windows per measurement; the median is reported


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--repeats", type=int, default=REPEATS,
                   help="timed windows of --steps launches per measurement (median reported)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only-headline", action="store_true",
                   help="time only the per-token FP8 producer")
    p.add_argument("--only", default="",
                   help="comma-separated workload names to time (default: all)")
    p.add_argument("--modes", default="cold,warm",
                   help="cold (rotating >= 512 MB of buffer sets), warm (one set), or both")
    p.add_argument("--direct", action="store_true",
                   help="launch each step directly instead of replaying a HIP graph")
    p.add_argument("--no-overhead", action="store_true",
                   help="skip the small-shape launch-overhead table")
    p.add_argument("--no-floor", action="store_true",
                   help="skip timing the memory-only counterparts (libalnp_floor.so)")
    p.add_argument("--counters", action="store_true",
                   help="run under rocprofv3 counter collection (--pmc): warm mode only, at "
                        "most %d steps, one timed window, no floors, copies, overhead table "
                        "or CPU baseline" % COUNTER_MAX_STEPS)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain device copies of %s bytes (torch's copy and "
                        "alnp_floor_copy, four each; the reference for scaling rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE) and exit" % "/".join(map(str, COPY_SIZES)))
    p.add_argument("--floor-sweep", action="store_true",
                   help="only time the per-token producer and memory-only access patterns over "
                        "a range of row counts at dim 3072 and exit")
    p.add_argument("--timeline", action="store_true",
                   help="only record per-wave timelines of the FP8 row and table kernels "
                        "(libalnp_timeline.so, measurement only) for the FP8 workloads in "
                        "--only, cold, and exit")
    return p.parse_args()


def counter_guard(a, modes):
    """Counter collection (rocprofv3 --pmc) serializes every dispatch and
    samples counters around it.  One such run ended in a host segmentation
    fault (exit 139) while timing cold mode: thousands of buffer sets, each
    allocated and filled by its own device copies, then graphs of 1000
    launches.  Only the short warm form has been run under counters since.
    Returns an error message for anything else, or None."""
    collecting = os.environ.get("ROCPROF_COUNTER_COLLECTION", "").strip().lower() in (
        "1", "true", "yes", "on")
    if collecting and not a.counters:
        return "rocprofv3 counter collection is active: pass --counters"
    if not a.counters:
        return None
    if "cold" in modes:
        return "--counters takes --modes warm only (cold mode is not run under counters)"
    if a.steps > COUNTER_MAX_STEPS:
        return f"--counters takes at most {COUNTER_MAX_STEPS} steps"
    return None


# ---- workloads ----------------------------------------------------------------

def algorithmic_bytes(name, d):
    """Bytes a producer must move once: inputs read + outputs written."""
    if name.startswith("modulation6"):
        p = d["params"]
        return p.nbytes + d["mod"].nbytes + p.size // 6 * 6 * 2
    if name.startswith("residual"):
        return 4 * d["residual"].nbytes    # residual, gate, projection in; bf16 out
    x = d["x"]
    rows, dim = x.shape
    if name.startswith("adaln_fp4"):
        # x, e2m1 codes, e4m3 block scales (the tiled layout has no padding at
        # these sizes), and the (dim,) operands: bf16, or e4m3 plus two fp32 scalars
        ops = 2 * dim + 8 if "modfp8" in name else 2 * dim * 2
        return x.nbytes + rows * dim // 2 + rows * dim // 16 + ops
    if name.startswith("modfp8"):
        return x.nbytes + rows * dim + 4 + 2 * dim + 8   # e4m3 (dim,) operands, two scalars
    if name.startswith("awq"):
        return x.nbytes + rows * dim + 4 + 3 * dim * 2   # scale, shift, inv_s (dim,)
    if name.startswith("mxfp8_ptok"):
        return 3 * x.nbytes + rows * dim + rows * dim // 32   # x, scale, shift; e4m3 + E8M0
    if name.startswith("mxfp8_table"):
        return 3 * x.nbytes + 2 * dim * 4 + rows * dim + rows * dim // 32  # x, 2 temb chunks, 2 table rows
    if name.startswith("ln_mxfp4"):
        return x.nbytes + rows * dim // 2 + rows * dim // 32
    if name.startswith("rmsmod"):
        # x, bf16 out, the weight, the table rows the segments use, the indices
        used = len(np.unique(d["seg"]))
        return 2 * x.nbytes + dim * 2 + used * 2 * dim * 2 + rows * 4
    if name.startswith("ln_fp4"):
        return x.nbytes + rows * dim // 2 + rows * dim // 16
    b = x.nbytes + rows * dim + 4  # x, e4m3 out, act_scale
    if name.startswith("bcast") or name.startswith("ln_fp8"):
        b += 0 if name.startswith("ln_fp8") else 2 * dim * 2
    elif name.startswith("ptok"):
        b += 2 * rows * dim * 2
    elif name.startswith("table"):
        b += 2 * rows * dim * 2 + 2 * dim * 4   # two temb chunks + two table rows
    return b


def floor_lib():
    """libalnp_floor.so (memory-only counterparts of the producers, built with
    libalnp.so), or None if it was not built."""
    path = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "libalnp_floor.so")
    if not os.path.exists(path):
        return None
    F = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    F.alnp_floor_rows.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    F.alnp_floor_rows.restype = ctypes.c_int
    F.alnp_floor_modulation6.argtypes = [vp, i64, ctypes.c_int, ctypes.POINTER(vp), vp]
    F.alnp_floor_modulation6.restype = ctypes.c_int
    F.alnp_floor_rows_shape.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp,
                                        ctypes.c_int, ctypes.c_int, vp]
    F.alnp_floor_rows_shape.restype = ctypes.c_int
    F.alnp_floor_copy.argtypes = [vp, vp, i64, vp]
    F.alnp_floor_copy.restype = ctypes.c_int
    return F


# out_kind of alnp_floor_rows
FLOOR_FP8, FLOOR_NVFP4, FLOOR_BF16, FLOOR_MXFP8, FLOOR_MXFP4, FLOOR_NVFP4_TILED = 0, 1, 2, 3, 4, 5


def timeline_lib(alnp):
    """libalnp_timeline.so: the C ABI with the FP8 row and table kernels
    writing per-wave clock records (csrc/timeline.hpp), or None."""
    path = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "libalnp_timeline.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    for fn, (args, res) in alnp.SIGNATURES.items():
        f = getattr(L, fn)
        f.argtypes, f.restype = args, res
    L.alnp_timeline_set.argtypes = [ctypes.c_void_p]
    L.alnp_timeline_set.restype = ctypes.c_int
    return L


class Producer:
    """Device buffers for `sets` copies of one workload and a raw C-ABI
    launcher for set i (pointers precomputed: the step is the library call).
    With a floor library, `floor_calls` holds, per set, the memory-only
    counterpart of the call on the same buffers."""

    def __init__(self, name, d, sets, torch, alnp, floor=None):
        self.name, self.d, self.sets = name, d, sets
        self.torch, self.L = torch, alnp.lib()
        F = floor
        self.floor_calls = [] if F is not None else None

        def add_floor(fn_args):
            if F is not None:
                self.floor_calls.append(fn_args)
        dev = torch.device("cuda")
        bf = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(dev)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        self.keep = []
        self.calls = []
        kind = name.split("_")[0]
        if kind == "modulation6":
            p0, m0 = f32(d["params"]), f32(d["mod"])
            B, S, _, D = p0.shape
            for _ in range(sets):
                p, m = p0.clone(), m0.clone()
                outs = [torch.empty((B, S, D), dtype=torch.bfloat16, device=dev) for _ in range(6)]
                arr = (ctypes.c_void_p * 6)(*[o.data_ptr() for o in outs])
                self.keep += [p, m, outs, arr]
                self.calls.append((self.L.alnp_adaln_modulation6_bf16,
                                   (p.data_ptr(), m.data_ptr(), B, S, D, arr)))
                if F is not None:
                    add_floor((F.alnp_floor_modulation6, (p.data_ptr(), B * S, D, arr)))
            self.outs = lambda i: self.keep[4 * i + 2]
            return
        if kind == "residual":
            r0, g0, p0 = bf(d["residual"]), bf(d["gate"]), bf(d["proj"])
            rows, dim = r0.shape
            for _ in range(sets):
                r, g, pj = r0.clone(), g0.clone(), p0.clone()
                out = torch.empty_like(r)
                self.keep.append((r, g, pj, out))
                self.calls.append((self.L.alnp_gated_residual_bf16,
                                   (r.data_ptr(), g.data_ptr(), pj.data_ptr(), rows, dim, rows,
                                    out.data_ptr())))
                # the same bytes in the row floor's shape: three bf16 rows in, one out
                add_floor((F.alnp_floor_rows, (r.data_ptr(), g.data_ptr(), pj.data_ptr(), dim, rows,
                                               dim, FLOOR_BF16, out.data_ptr(), None))
                          if F is not None else None)
            return
        x0 = bf(d["x"])
        rows, dim = x0.shape
        u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev)
        if kind in ("modfp8", "adaln") and "scale_fp8" in d:
            # the floors read two shared bf16 (dim,) vectors in place of the
            # e4m3 operands (both stay in cache; a few KB either way)
            dummy = (bf(d["x"][0]), bf(d["x"][1]))
            self.keep.append(dummy)
        if name.startswith("adaln_fp4"):
            swz = "_swz" in name
            mod8 = "modfp8" in name
            sf_bytes = self.L.alnp_swizzled_sf_size(rows, dim) if swz else rows * dim // 16
            for _ in range(sets):
                x = x0.clone()
                packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=dev)
                sf = torch.empty(sf_bytes, dtype=torch.uint8, device=dev)
                if mod8:
                    sc8, sh8 = u8(d["scale_fp8"]), u8(d["shift_fp8"])
                    sdeq = torch.tensor([d["scale_deq"]], dtype=torch.float32, device=dev)
                    hdeq = torch.tensor([d["shift_deq"]], dtype=torch.float32, device=dev)
                    self.keep.append((x, sc8, sh8, sdeq, hdeq, packed, sf))
                    self.calls.append((self.L.alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16,
                                       (x.data_ptr(), sc8.data_ptr(), sh8.data_ptr(), sdeq.data_ptr(),
                                        hdeq.data_ptr(), d["eps"], rows, dim, packed.data_ptr(),
                                        sf.data_ptr(), None, None)))
                    a_ptr, b_ptr = dummy[0].data_ptr(), dummy[1].data_ptr()
                else:
                    sc, sh = bf(d["scale"]), bf(d["shift"])
                    self.keep.append((x, sc, sh, packed, sf))
                    fn = (self.L.alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16 if swz
                          else self.L.alnp_ada_layer_norm_quant_nvfp4_bf16)
                    self.calls.append((fn, (x.data_ptr(), sc.data_ptr(), sh.data_ptr(), d["eps"],
                                            rows, dim, packed.data_ptr(), sf.data_ptr(), None,
                                            None)))
                    a_ptr, b_ptr = sc.data_ptr(), sh.data_ptr()
                add_floor((F.alnp_floor_rows, (x.data_ptr(), a_ptr, b_ptr, 0, rows, dim,
                                               FLOOR_NVFP4_TILED if swz else FLOOR_NVFP4,
                                               packed.data_ptr(), sf.data_ptr()))
                          if F is not None else None)
            return
        if kind in ("modfp8", "awq"):
            act0 = torch.tensor([d["act_scale"]], dtype=torch.float32, device=dev)
            for _ in range(sets):
                x, act = x0.clone(), act0.clone()
                out = torch.empty((rows, dim), dtype=torch.uint8, device=dev)
                if kind == "modfp8":
                    sc8, sh8 = u8(d["scale_fp8"]), u8(d["shift_fp8"])
                    sdeq = torch.tensor([d["scale_deq"]], dtype=torch.float32, device=dev)
                    hdeq = torch.tensor([d["shift_deq"]], dtype=torch.float32, device=dev)
                    self.keep.append((x, act, sc8, sh8, sdeq, hdeq, out))
                    self.calls.append((self.L.alnp_ada_layer_norm_quant_fp8_modfp8_bf16,
                                       (x.data_ptr(), sc8.data_ptr(), sh8.data_ptr(),
                                        sdeq.data_ptr(), hdeq.data_ptr(), act.data_ptr(), d["eps"],
                                        rows, dim, out.data_ptr(), None, None)))
                    a_ptr, b_ptr = dummy[0].data_ptr(), dummy[1].data_ptr()
                else:
                    sc, sh, isv = bf(d["scale"]), bf(d["shift"]), bf(d["inv_s"])
                    self.keep.append((x, act, sc, sh, isv, out))
                    self.calls.append((self.L.alnp_awq_ada_layer_norm_quant_fp8_bf16,
                                       (x.data_ptr(), sc.data_ptr(), sh.data_ptr(), isv.data_ptr(),
                                        act.data_ptr(), d["eps"], rows, dim, out.data_ptr(), None,
                                        None)))
                    a_ptr, b_ptr = sc.data_ptr(), sh.data_ptr()
                add_floor((F.alnp_floor_rows, (x.data_ptr(), a_ptr, b_ptr, 0, rows, dim, FLOOR_FP8,
                                               out.data_ptr(), None))
                          if F is not None else None)
            return
        if name.startswith("mxfp8_table"):
            te0, tb0 = bf(d["temb"]), f32(d["table"])
            chunks = d["temb"].shape[1]
            for _ in range(sets):
                x, te = x0.clone(), te0.clone()
                out = torch.empty((rows, dim), dtype=torch.uint8, device=dev)
                sc_out = torch.empty((rows, dim // 32), dtype=torch.uint8, device=dev)
                self.keep.append((x, te, tb0, out, sc_out))
                self.calls.append((self.L.alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16,
                                   (x.data_ptr(), te.data_ptr(), tb0.data_ptr(), chunks,
                                    d["shift_idx"], d["scale_idx"], d["eps"], rows, dim,
                                    out.data_ptr(), sc_out.data_ptr(), None, None)))
                if F is not None:
                    add_floor((F.alnp_floor_rows,
                               (x.data_ptr(), te.data_ptr() + 2 * int(d["scale_idx"]) * dim,
                                te.data_ptr() + 2 * int(d["shift_idx"]) * dim, chunks * dim, rows,
                                dim, FLOOR_MXFP8, out.data_ptr(), sc_out.data_ptr())))
            return
        if name.startswith("mxfp8_ptok") or name.startswith("ln_mxfp4"):
            fp8 = name.startswith("mxfp8")
            sc0, sh0 = (bf(d["scale"]), bf(d["shift"])) if fp8 else (None, None)
            for _ in range(sets):
                x = x0.clone()
                out = torch.empty((rows, dim if fp8 else dim // 2), dtype=torch.uint8, device=dev)
                sc_out = torch.empty((rows, dim // 32), dtype=torch.uint8, device=dev)
                if fp8:
                    sc, sh = sc0.clone(), sh0.clone()
                    self.keep.append((x, sc, sh, out, sc_out))
                    self.calls.append((self.L.alnp_ada_layer_norm_quant_mxfp8_ptok_bf16,
                                       (x.data_ptr(), sc.data_ptr(), sh.data_ptr(), d["eps"], rows,
                                        dim, out.data_ptr(), sc_out.data_ptr(), None, None)))
                    if F is not None:
                        add_floor((F.alnp_floor_rows,
                                   (x.data_ptr(), sc.data_ptr(), sh.data_ptr(), dim, rows, dim,
                                    FLOOR_MXFP8, out.data_ptr(), sc_out.data_ptr())))
                else:
                    self.keep.append((x, out, sc_out))
                    self.calls.append((self.L.alnp_layer_norm_no_affine_quant_mxfp4_bf16,
                                       (x.data_ptr(), d["eps"], rows, dim, out.data_ptr(),
                                        sc_out.data_ptr(), None, None)))
                    if F is not None:
                        add_floor((F.alnp_floor_rows,
                                   (x.data_ptr(), None, None, 0, rows, dim, FLOOR_MXFP4,
                                    out.data_ptr(), sc_out.data_ptr())))
            return
        if kind == "rmsmod":
            w, sc, sh = bf(d["weight"]), bf(d["scale"]), bf(d["shift"])
            seg = torch.from_numpy(d["seg"]).to(dev)
            for _ in range(sets):
                x = x0.clone()
                out = torch.empty_like(x)
                self.keep.append((x, out, w, sc, sh, seg))
                self.calls.append((self.L.alnp_rms_norm_modulate_seg_bf16,
                                   (x.data_ptr(), w.data_ptr(), sc.data_ptr(), sh.data_ptr(),
                                    seg.data_ptr(), sc.shape[0], d["eps"], rows, dim,
                                    out.data_ptr(), None)))
                if F is not None:
                    add_floor((F.alnp_floor_rows, (x.data_ptr(), None, None, 0, rows, dim,
                                                   FLOOR_BF16, out.data_ptr(), None)))
            return
        act0 = torch.tensor([d.get("act_scale", 0.025)], dtype=torch.float32, device=dev)
        ops = {}
        if kind in ("bcast", "ptok"):
            ops = dict(scale=bf(d["scale"]), shift=bf(d["shift"]))
        elif kind == "table":
            ops = dict(temb=bf(d["temb"]), table=f32(d["table"]))
        for _ in range(sets):
            x, act = x0.clone(), act0.clone()
            o = {k: v.clone() for k, v in ops.items()}
            if kind == "fp4" or name.startswith("ln_fp4"):
                packed = torch.empty((rows, dim // 2), dtype=torch.uint8, device=dev)
                sf = torch.empty((rows, dim // 16), dtype=torch.uint8, device=dev)
                self.keep.append((x, packed, sf))
                self.calls.append((self.L.alnp_layer_norm_no_affine_quant_nvfp4_bf16,
                                   (x.data_ptr(), d["eps"], rows, dim, packed.data_ptr(),
                                    sf.data_ptr(), None, None)))
                if F is not None:
                    add_floor((F.alnp_floor_rows, (x.data_ptr(), None, None, 0, rows, dim,
                                                   FLOOR_NVFP4, packed.data_ptr(), sf.data_ptr())))
                continue
            out = torch.empty((rows, dim), dtype=torch.uint8, device=dev)
            self.keep.append((x, act, o, out))
            if F is not None:
                if kind == "ln":
                    a_ptr = b_ptr = None
                    stride = 0
                elif kind in ("bcast", "ptok"):
                    a_ptr, b_ptr = o["scale"].data_ptr(), o["shift"].data_ptr()
                    stride = dim if kind == "ptok" else 0
                else:
                    chunks = d["temb"].shape[1]
                    a_ptr = o["temb"].data_ptr() + 2 * int(d["scale_idx"]) * dim
                    b_ptr = o["temb"].data_ptr() + 2 * int(d["shift_idx"]) * dim
                    stride = chunks * dim
                add_floor((F.alnp_floor_rows, (x.data_ptr(), a_ptr, b_ptr, stride, rows, dim,
                                               FLOOR_FP8, out.data_ptr(), None)))
            if kind == "ln":
                self.calls.append((self.L.alnp_layer_norm_no_affine_quant_fp8_static_bf16,
                                   (x.data_ptr(), act.data_ptr(), d["eps"], rows, dim,
                                    out.data_ptr(), None, None)))
            elif kind == "bcast":
                self.calls.append((self.L.alnp_ada_layer_norm_quant_fp8_bf16,
                                   (x.data_ptr(), o["scale"].data_ptr(), o["shift"].data_ptr(),
                                    act.data_ptr(), d["eps"], rows, dim, out.data_ptr(),
                                    None, None)))
            elif kind == "ptok":
                self.calls.append((self.L.alnp_ada_layer_norm_quant_fp8_ptok_bf16,
                                   (x.data_ptr(), o["scale"].data_ptr(), o["shift"].data_ptr(),
                                    act.data_ptr(), d["eps"], rows, dim, out.data_ptr(),
                                    None, None)))
            else:
                chunks = d["temb"].shape[1]
                self.calls.append((self.L.alnp_ada_layer_norm_quant_fp8_ptok_table_bf16,
                                   (x.data_ptr(), o["temb"].data_ptr(), o["table"].data_ptr(),
                                    chunks, d["shift_idx"], d["scale_idx"], act.data_ptr(),
                                    d["eps"], rows, dim, out.data_ptr(), None, None)))

    def launch(self, i, stream):
        fn, args = self.calls[i % self.sets]
        st = fn(*args, stream)
        if st != 0:
            raise RuntimeError(f"{self.name}: status {st}")

    def launch_floor(self, i, stream):
        fn, args = self.floor_calls[i % self.sets]
        st = fn(*args, stream)
        if st != 0:
            raise RuntimeError(f"{self.name} floor: status {st}")


class HipEvents:
    """Timing events without the system-scope fence.  A HIP event recorded
    with default flags performs a system-scope release (L2 writeback and
    invalidation) when it completes; inside a short timed window that cost
    lands on the launches being timed.  Events created with
    hipEventDisableSystemFence record the timestamp without it, which HIP
    documents for events used only to measure time.  The events come from
    the HIP runtime the process already loaded (torch's), so they share
    its streams; the window's completion is waited for with a device
    synchronize before the elapsed times are read."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        with open("/proc/self/maps") as fh:
            paths = [l.split()[-1] for l in fh if "libamdhip64" in l and "/" in l]
        if not paths:
            raise RuntimeError("the HIP runtime is not loaded")
        H = ctypes.CDLL(paths[0])
        vp = ctypes.c_void_p
        H.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        H.hipEventRecord.argtypes = [vp, vp]
        H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        H.hipEventDestroy.argtypes = [vp]
        for f in (H.hipEventCreateWithFlags, H.hipEventRecord, H.hipEventElapsedTime,
                  H.hipEventDestroy):
            f.restype = ctypes.c_int
        self.H = H

    def new(self):
        e = ctypes.c_void_p()
        st = self.H.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {st}")
        return e

    def record(self, e, stream):
        st = self.H.hipEventRecord(e, stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord: {st}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        st = self.H.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime: {st}")
        return ms.value

    def free(self, *evs):
        for e in evs:
            self.H.hipEventDestroy(e)

    # -- graphs with event-record nodes --------------------------------------

    def _graph_api(self):
        H = self.H
        if getattr(self, "_graphs_ready", False):
            return H
        vp, pvp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)
        psz, sz = ctypes.POINTER(ctypes.c_size_t), ctypes.c_size_t
        sigs = {"hipStreamBeginCapture": [vp, ctypes.c_int],
                "hipStreamEndCapture": [vp, pvp],
                "hipGraphClone": [pvp, vp],
                "hipGraphGetNodes": [vp, pvp, psz],
                "hipGraphGetRootNodes": [vp, pvp, psz],
                "hipGraphNodeGetDependentNodes": [vp, pvp, psz],
                "hipGraphRemoveDependencies": [vp, pvp, pvp, sz],
                "hipGraphAddDependencies": [vp, pvp, pvp, sz],
                "hipGraphAddEventRecordNode": [pvp, vp, pvp, sz, vp],
                "hipGraphInstantiate": [pvp, vp, vp, vp, sz],
                "hipGraphLaunch": [vp, vp],
                "hipGraphExecDestroy": [vp],
                "hipGraphDestroy": [vp]}
        for name, args in sigs.items():
            fn = getattr(H, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        self._graphs_ready = True
        return H

    @staticmethod
    def _ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: HIP error {st}")

    def capture(self, stream, launch, idxs):
        """A graph of launch(i, stream) for i in idxs, captured on `stream`
        (a torch stream that nothing else uses meanwhile)."""
        H = self._graph_api()
        h = stream.cuda_stream
        self._ok(H.hipStreamBeginCapture(h, 1), "hipStreamBeginCapture")   # thread-local mode
        try:
            for i in idxs:
                launch(i, h)
        finally:
            g = ctypes.c_void_p()
            st = H.hipStreamEndCapture(h, ctypes.byref(g))
        self._ok(st, "hipStreamEndCapture")
        return g

    def _chain(self, g):
        """The nodes of a captured single-stream graph in launch order; it
        must be one chain (each node depends on the one before)."""
        H = self._graph_api()
        vp = ctypes.c_void_p
        n = ctypes.c_size_t(0)
        self._ok(H.hipGraphGetNodes(g, None, ctypes.byref(n)), "hipGraphGetNodes")
        total = n.value
        n = ctypes.c_size_t(0)
        self._ok(H.hipGraphGetRootNodes(g, None, ctypes.byref(n)), "hipGraphGetRootNodes")
        if n.value != 1:
            raise RuntimeError(f"captured graph has {n.value} root nodes, not one chain")
        root = (vp * 1)()
        self._ok(H.hipGraphGetRootNodes(g, root, ctypes.byref(n)), "hipGraphGetRootNodes")
        nodes = [root[0]]
        nxt = (vp * 1)()
        while True:
            n = ctypes.c_size_t(0)
            self._ok(H.hipGraphNodeGetDependentNodes(nodes[-1], None, ctypes.byref(n)),
                     "hipGraphNodeGetDependentNodes")
            if n.value == 0:
                break
            if n.value != 1:
                raise RuntimeError("captured graph is not one chain")
            self._ok(H.hipGraphNodeGetDependentNodes(nodes[-1], nxt, ctypes.byref(n)),
                     "hipGraphNodeGetDependentNodes")
            nodes.append(nxt[0])
        if len(nodes) != total:
            raise RuntimeError(f"captured graph is not one chain ({len(nodes)} of {total} nodes)")
        return nodes

    def _splice_event(self, g, a, b, ev):
        """Replace the edge a -> b of graph g by a -> record(ev) -> b."""
        H = self._graph_api()
        vp = ctypes.c_void_p
        fa, tb = (vp * 1)(a), (vp * 1)(b)
        self._ok(H.hipGraphRemoveDependencies(g, fa, tb, 1), "hipGraphRemoveDependencies")
        node = vp()
        self._ok(H.hipGraphAddEventRecordNode(ctypes.byref(node), g, fa, 1, ev),
                 "hipGraphAddEventRecordNode")
        self._ok(H.hipGraphAddDependencies(g, (vp * 1)(node), tb, 1), "hipGraphAddDependencies")

    def window_graph(self, seq, launches, nspace, steps, t0, t1):
        """One executable graph from `seq`, a captured chain of `launches`
        calls (spacer, then the timed calls, then a tail): a copy of it
        with an event-record node for t0 spliced in before the first timed
        call's kernels and one for t1 after the last timed call's.  One flat
        chain: nesting the three parts as child graphs instead cost about 4
        us per window on MI355X.  The graph launch's own start-up cost falls
        before the spacer, outside the window between the two event nodes."""
        H = self._graph_api()
        g = ctypes.c_void_p()
        self._ok(H.hipGraphClone(ctypes.byref(g), seq), "hipGraphClone")
        try:
            nodes = self._chain(g)
            per, rem = divmod(len(nodes), launches)
            if rem or per == 0:
                raise RuntimeError(f"{len(nodes)} graph nodes for {launches} calls")
            first, last = per * nspace, per * (nspace + steps) - 1
            self._splice_event(g, nodes[first - 1], nodes[first], t0)
            self._splice_event(g, nodes[last], nodes[last + 1], t1)
            ex = ctypes.c_void_p()
            self._ok(H.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0),
                     "hipGraphInstantiate")
        finally:
            H.hipGraphDestroy(g)
        return ex

    def free_captured(self, *graphs):
        for g in graphs:
            self._graph_api().hipGraphDestroy(g)

    def launch_graph(self, ex, stream):
        self._ok(self._graph_api().hipGraphLaunch(ex, stream.cuda_stream), "hipGraphLaunch")

    def free_graph(self, ex):
        self._graph_api().hipGraphExecDestroy(ex)


_EVENTS = None


def hip_events():
    global _EVENTS
    if _EVENTS is None:
        _EVENTS = HipEvents()
    return _EVENTS


def sets_for(nbytes, cold):
    return max(2, math.ceil(COLD_FOOTPRINT / nbytes)) if cold else 1


def _capture(torch, launch, idxs):
    """A HIP graph of launch(i) for i in idxs, captured on a side stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        hh = torch.cuda.current_stream().cuda_stream
        for i in idxs:
            launch(i, hh)
    return g


SPACER_MIN_LAUNCHES = 64
SPACER_MS = 20.0       # minimum GPU time of the spacer before each window
TAIL_LAUNCHES = 8      # launches after the closing event node of a timed window


def spacer_length(sets, steps, launch_us=None):
    """Launches of the untimed spacer before each timed window: whole
    rotations over the buffer sets (so that every set the timed window
    touches was last touched one full rotation earlier, with all the other
    sets' bytes in between); at least as many launches as the window and
    SPACER_MIN_LAUNCHES; and, given an estimate of one launch's time, at
    least SPACER_MS of work.  The last rule puts every window past the
    first ~10 ms of load, during which the per-launch time on these boxes
    first rises by up to 6% and then settles (clock and power management);
    a window then measures the settled rate whatever its length."""
    n = max(steps, SPACER_MIN_LAUNCHES)
    if launch_us:
        n = max(n, math.ceil(SPACER_MS * 1000.0 / launch_us))
    return sets * max(1, math.ceil(n / sets))


def time_launches(torch, stream, launch, sets, steps, warmup, use_graph, repeats=REPEATS):
    """Median, min and max microseconds per launch over `repeats` timed
    windows of exactly `steps` launches each (launch i uses buffer set
    i mod sets): time_interleaved with one variant."""
    return time_interleaved(torch, stream, [(launch, sets)], steps, warmup, use_graph, repeats)[0]


def time_interleaved(torch, stream, variants, steps, warmup, use_graph, repeats=REPEATS):
    """For each (launch, sets) in `variants`: median, min and max
    microseconds per launch over `repeats` timed windows of exactly `steps`
    launches each (launch i uses buffer set i mod sets), measured with HIP
    events on `stream`, the stream the launches run on (HipEvents: no
    system-scope fence).

    Each window is preceded by an untimed spacer of whole rotations over
    its variant's sets and at least SPACER_MS of work (spacer_length):
    every set the window touches has been evicted by the rotation through
    all the others, and the GPU has been under steady load for a while when
    the window opens.

    With a graph (the default), each window is one executable graph, a
    single captured chain: the spacer, an event-record node, the `steps`
    timed launches, a second event-record node and a short tail.  The cost of starting a graph
    launch (several microseconds on this runtime, paid once per launch
    however many kernels the graph holds) then falls before the spacer,
    outside the window, which holds exactly the timed launches.  All
    windows are launched back to back, between two device synchronizations,
    so the GPU does not idle between them, and the variants alternate
    window by window, in reverse order on odd repeats (A B C, C B A, ...):
    a slow drift of the clock or the memory system then moves every
    variant alike, and ratios between them (a producer against its
    memory-only floor) do not depend on which was timed first.  Without a
    graph the launches are enqueued directly, the events recorded on the
    stream, in the same order."""
    E = hip_events()
    h = stream.cuda_stream
    nv = len(variants)
    samples = [[] for _ in range(nv)]
    spacers = []
    order = [v for r in range(repeats) for v in (range(nv) if r % 2 == 0 else range(nv - 1, -1, -1))]
    with torch.cuda.stream(stream):
        for launch, sets in variants:
            for i in range(warmup):
                launch(i, h)
            torch.cuda.synchronize()
            # Rough per-launch time from a short untimed burst, to size the spacer.
            a, b = E.new(), E.new()
            E.record(a, stream)
            for i in range(16):
                launch(i, h)
            E.record(b, stream)
            torch.cuda.synchronize()
            spacers.append(spacer_length(sets, steps, E.elapsed_ms(a, b) * 1000.0 / 16))
            E.free(a, b)
        if use_graph:
            cap = torch.cuda.Stream()
            windows = []                          # per variant: [(exec, t0, t1)] * repeats
            for (launch, _), nspace in zip(variants, spacers):
                idx = (list(range(nspace)) + list(range(steps)) +
                       list(range(steps, steps + TAIL_LAUNCHES)))
                seq = E.capture(cap, lambda k, hh, launch=launch, idx=idx: launch(idx[k], hh),
                                range(len(idx)))
                ws = []
                for _ in range(repeats):
                    t0, t1 = E.new(), E.new()
                    ws.append((E.window_graph(seq, len(idx), nspace, steps, t0, t1), t0, t1))
                E.free_captured(seq)
                windows.append(ws)
            for ws in windows:                    # upload, untimed
                for ex, _, _ in ws:
                    E.launch_graph(ex, stream)
            torch.cuda.synchronize()
            nth = [0] * nv
            for v in order:                       # back to back: the GPU never idles
                E.launch_graph(windows[v][nth[v]][0], stream)
                nth[v] += 1
            torch.cuda.synchronize()
            for v, ws in enumerate(windows):
                for ex, t0, t1 in ws:
                    samples[v].append(E.elapsed_ms(t0, t1) * 1000.0 / steps)
                    E.free_graph(ex)
                    E.free(t0, t1)
        else:
            events = []
            for v in order:
                launch, _ = variants[v]
                t0, t1 = E.new(), E.new()
                for i in range(spacers[v]):
                    launch(i, h)
                E.record(t0, stream)
                for i in range(steps):
                    launch(i, h)
                E.record(t1, stream)
                events.append((v, t0, t1))
            torch.cuda.synchronize()
            for v, a, b in events:
                samples[v].append(E.elapsed_ms(a, b) * 1000.0 / steps)
                E.free(a, b)
    out = []
    for v in range(nv):
        us = sorted(samples[v])
        out.append({"us": float(np.median(us)), "min": us[0], "max": us[-1], "spacer": spacers[v],
                    "launches": warmup + 16 + (2 if use_graph else 1) * repeats *
                                (spacers[v] + steps + (TAIL_LAUNCHES if use_graph else 0))})
    return out


class CopyCeiling:
    """A plain copy (libalnp_floor.so's alnp_floor_copy) moving `nbytes` in
    total, half read and half written, over cold-rotated buffer sets: the
    practical ceiling for a stream of that size."""

    def __init__(self, nbytes, cold, torch, F):
        half = max(16, (nbytes // 2) // 16 * 16)
        self.nbytes = 2 * half
        self.sets = sets_for(self.nbytes, cold)
        self.bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
                      torch.empty(half, dtype=torch.uint8, device="cuda"))
                     for _ in range(self.sets)]
        self.F, self.half = F, half

    def launch(self, i, stream):
        src, dst = self.bufs[i % self.sets]
        st = self.F.alnp_floor_copy(src.data_ptr(), dst.data_ptr(), self.half, stream)
        if st != 0:
            raise RuntimeError(f"copy: status {st}")


# ---- launch overhead at small shapes ---------------------------------------------------

def launch_overhead(torch, alnp, inputs, stream, calls=400, graph_launches=32, replays=50,
                    repeats=REPEATS):
    """The pages' small-shape method (Benchmark Results, "Six-way modulation
    producer" and "NVIDIA Thor installed artifact"): per shape, the raw C ABI
    launched directly, the Python wrapper launched directly (A-B-B-A order),
    and a HIP graph of 32 launches replayed, time / 32.  Inputs stay the same
    buffers (warm): these shapes are latency-bound.  Every case is built and
    run once, untimed, before any is timed (first calls pay one-time costs),
    and each figure is the median of `repeats` rounds over all cases."""
    dev = torch.device("cuda")
    bf = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    L = alnp.lib()
    act = torch.tensor([0.025], dtype=torch.float32, device=dev)
    cases = {}
    for name, kind, rows, dim in (("ptok_fp8_51x1536", "ptok", 51, 1536),
                                  ("table_fp8_51x1536", "table", 51, 1536),
                                  ("ptok_fp8_105x1152", "ptok", 105, 1152),
                                  ("modulation6_1x51x1536", "mod6", 51, 1536)):
        if kind == "mod6":
            d = inputs.make("mod6", batch=1, seq=rows, dim=dim)
            p, m = f32(d["params"]), f32(d["mod"])
            outs = [torch.empty((1, rows, dim), dtype=torch.bfloat16, device=dev) for _ in range(6)]
            arr = (ctypes.c_void_p * 6)(*[o.data_ptr() for o in outs])
            raw = (lambda p, m, rows, dim, arr: lambda h: L.alnp_adaln_modulation6_bf16(
                p.data_ptr(), m.data_ptr(), 1, rows, dim, arr, h))(p, m, rows, dim, arr)
            wrap = (lambda p, m, outs: lambda h: alnp.adaln_modulation6_bf16(p, m, out=outs))(p, m, outs)
            keep = (p, m, outs, arr)
        elif kind == "ptok":
            d = inputs.make("ptok", rows=rows, dim=dim)
            x, sc, sh = bf(d["x"]), bf(d["scale"]), bf(d["shift"])
            out = torch.empty((rows, dim), dtype=torch.float8_e4m3fn, device=dev)
            raw = (lambda x, sc, sh, out, rows, dim: lambda h: L.alnp_ada_layer_norm_quant_fp8_ptok_bf16(
                x.data_ptr(), sc.data_ptr(), sh.data_ptr(), act.data_ptr(), 1e-5, rows, dim,
                out.data_ptr(), None, None, h))(x, sc, sh, out, rows, dim)
            wrap = (lambda x, sc, sh, out: lambda h: alnp.ada_layer_norm_quant_fp8_ptok_bf16(
                x, sc, sh, act, out=out))(x, sc, sh, out)
            keep = (x, sc, sh, out)
        else:
            d = inputs.make("table", rows=rows, dim=dim)
            x, te, tb = bf(d["x"]), bf(d["temb"]), f32(d["table"])
            out = torch.empty((rows, dim), dtype=torch.float8_e4m3fn, device=dev)
            raw = (lambda x, te, tb, out, rows, dim: lambda h: L.alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(
                x.data_ptr(), te.data_ptr(), tb.data_ptr(), 6, 0, 1, act.data_ptr(), 1e-5, rows,
                dim, out.data_ptr(), None, None, h))(x, te, tb, out, rows, dim)
            wrap = (lambda x, te, tb, out: lambda h: alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(
                x, te, tb, act, 0, 1, out=out))(x, te, tb, out)
            keep = (x, te, tb, out)
        cases[name] = {"raw": raw, "wrap": wrap, "keep": keep}

    E = hip_events()

    def elapsed(t0, t1):
        ms = E.elapsed_ms(t0, t1)
        E.free(t0, t1)
        return ms

    def direct(fn):
        with torch.cuda.stream(stream):
            h = stream.cuda_stream
            for _ in range(20):
                fn(h)
            t0, t1 = E.new(), E.new()
            torch.cuda.synchronize()
            E.record(t0, stream)
            for _ in range(calls):
                fn(h)
            E.record(t1, stream)
            torch.cuda.synchronize()
        return elapsed(t0, t1) * 1000.0 / calls

    def graphed(g):
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            t0, t1 = E.new(), E.new()
            E.record(t0, stream)
            for _ in range(replays):
                g.replay()
            E.record(t1, stream)
            torch.cuda.synchronize()
        return elapsed(t0, t1) * 1000.0 / (replays * graph_launches)

    # One untimed pass over every case, both call paths, then the graphs.
    with torch.cuda.stream(stream):
        for c in cases.values():
            for _ in range(50):
                c["raw"](stream.cuda_stream)
                c["wrap"](stream.cuda_stream)
        torch.cuda.synchronize()
    for c in cases.values():
        with torch.cuda.stream(stream):
            c["graph_raw"] = _capture(torch, lambda i, h, f=c["raw"]: f(h), range(graph_launches))
            c["graph_wrap"] = _capture(torch, lambda i, h, f=c["wrap"]: f(h), range(graph_launches))
    samples = {n: {"nat": [], "wr": [], "ga": [], "gb": []} for n in cases}
    for _ in range(repeats):
        for name, c in cases.items():
            a1, b1, b2, a2 = direct(c["raw"]), direct(c["wrap"]), direct(c["wrap"]), direct(c["raw"])
            samples[name]["nat"].append((a1 + a2) / 2)
            samples[name]["wr"].append((b1 + b2) / 2)
            samples[name]["ga"].append(graphed(c["graph_raw"]))
            samples[name]["gb"].append(graphed(c["graph_wrap"]))
    out = {}
    for name, sm in samples.items():
        med = {k: float(np.median(v)) for k, v in sm.items()}
        ratios = [w / n for w, n in zip(sm["wr"], sm["nat"])]
        out[name] = {"native_us": round(med["nat"], 3), "wrapper_us": round(med["wr"], 3),
                     "graph_native_us": round(med["ga"], 3), "graph_wrapper_us": round(med["gb"], 3),
                     "wrapper_over_native": round(float(np.median(ratios)), 3),
                     "wrapper_over_native_range": [round(min(ratios), 3), round(max(ratios), 3)]}
        print(f"# overhead {name}: native {med['nat']:.3f} us, wrapper {med['wr']:.3f} us, graph "
              f"native {med['ga']:.3f} us, graph wrapper {med['gb']:.3f} us (median of {repeats})",
              file=sys.stderr, flush=True)
    return out


# ---- counters from rocprofv3 (profiles/) --------------------------------------------

# Sources that build the FP8 row-producer kernels (the headline kernel).
PRODUCER_SOURCES = ("producers.hip", "rows.hpp", "device_common.hpp", "kernels.hpp")


def kernel_source_hash(files=PRODUCER_SOURCES):
    """Hash of the producer sources with comments and layout removed, so that
    an edit to comments alone does not mark the stored counters stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "csrc")
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(f.encode() + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


# ---- CPU baseline -------------------------------------------------------------------------

def cpu_baseline(d, nbytes):
    """The oracle on the host's cores: whole passes over the per-token
    workload, repeated until about 10 s of CPU time (threads x wall clock)
    has been spent (at most 10 passes); the median pass is reported."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    rows = d["x"].shape[0]
    oracle.adaln_fp8_ptok(d["x"][:8], d["scale"][:8], d["shift"][:8], 0.025)  # load
    passes = []
    while len(passes) < 10 and sum(passes) * threads < 10.0:
        t = time.perf_counter()
        oracle.adaln_fp8_ptok(d["x"], d["scale"], d["shift"], d["act_scale"], d["eps"],
                              threads=threads)
        passes.append(time.perf_counter() - t)
    dt = float(np.median(passes))
    # One thread on the first quarter of the rows (same per-row work).
    part = max(1, rows // 4)
    t = time.perf_counter()
    oracle.adaln_fp8_ptok(d["x"][:part], d["scale"][:part], d["shift"][:part], d["act_scale"],
                          d["eps"], threads=1)
    dt1 = time.perf_counter() - t
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_call": round(dt * 1e6, 1),
            "sample": f"the whole per-token 2520x3072 workload ({rows} rows), rows split "
                      f"over {threads} threads; median of {len(passes)} passes "
                      f"({sum(passes) * threads:.1f} s of CPU time), wall clock",
            "single_thread": {"value": round(nbytes * part / rows / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"rows 0..{part} of the same workload on one thread, "
                                        f"one pass ({dt1:.2f} s)"}}


# ---- main -------------------------------------------------------------------------------------

def rounded(t):
    """A time_launches record rounded for the JSON line."""
    return {"us_per_call": round(t["us"], 3), "us_min": round(t["min"], 3),
            "us_max": round(t["max"], 3)}


def calibrate_copy(torch, F):
    """Four plain copies of each size in COPY_SIZES, first torch's device copy,
    then alnp_floor_copy (distinct kernels and grid sizes in the counter
    output), for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    for nbytes in COPY_SIZES:
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        if F is not None:
            for _ in range(4):
                assert F.alnp_floor_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                         torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps({"calibrate_copy_bytes": list(COPY_SIZES), "copies_each": 4,
                      "kernels": ["torch copy_", "k_floor_copy"] if F is not None else
                      ["torch copy_"]}))


SWEEP_ROWS = (315, 630, 1260, 2520, 5040, 10080, 20160)
SWEEP_SHAPES = ((2, 3), (1, 6), (4, 2), (8, 1))


def floor_sweep(torch, alnp, inputs, F, stream, steps, warmup, use_graph, repeats):
    """The per-token producer beside its memory-only pattern and a plain copy
    of the same bytes, over row counts at dim 3072, cold, with a least-squares
    line time = intercept + bytes / slope for each; then, at 2520 rows, the
    memory-only pattern in each row shape that covers a 3072 row."""
    dim = 3072
    out = {"dim": dim, "sizes": [], "shapes": []}
    for rows in SWEEP_ROWS:
        d = inputs.make("ptok", rows=rows, dim=dim)
        nbytes = algorithmic_bytes("ptok", d)
        prod = Producer("ptok_sweep", d, sets_for(nbytes, True), torch, alnp, F)
        cp = CopyCeiling(nbytes, True, torch, F)
        k, f, c = time_interleaved(torch, stream, [(prod.launch, prod.sets),
                                                   (prod.launch_floor, prod.sets),
                                                   (cp.launch, cp.sets)],
                                   steps, warmup, use_graph, repeats)
        row = {"rows": rows, "bytes": nbytes, "kernel_us": round(k["us"], 3),
               "floor_us": round(f["us"], 3), "copy_us": round(c["us"], 3),
               "kernel_frac_of_peak": round(nbytes / k["us"] / 1e3 / HBM_PEAK_GBS, 4),
               "floor_frac_of_peak": round(nbytes / f["us"] / 1e3 / HBM_PEAK_GBS, 4),
               "copy_frac_of_peak": round(cp.nbytes / c["us"] / 1e3 / HBM_PEAK_GBS, 4)}
        out["sizes"].append(row)
        print(f"# sweep {rows}x{dim}: kernel {row['kernel_us']} us, floor {row['floor_us']} us, "
              f"copy {row['copy_us']} us", file=sys.stderr, flush=True)
        if rows == 2520:
            def shape_launch(waves, vpt):
                def launch(i, h):
                    fn, args = prod.floor_calls[i % prod.sets]
                    st = F.alnp_floor_rows_shape(*args, waves, vpt, h)
                    if st != 0:
                        raise RuntimeError(f"floor shape {waves}x{vpt}: status {st}")
                return launch
            ts = time_interleaved(torch, stream, [(shape_launch(w, v), prod.sets)
                                                  for w, v in SWEEP_SHAPES],
                                  steps, warmup, use_graph, repeats)
            for (waves, vpt), t in zip(SWEEP_SHAPES, ts):
                out["shapes"].append({"waves": waves, "vpt": vpt, "us": round(t["us"], 3),
                                      "frac_of_peak": round(nbytes / t["us"] / 1e3 / HBM_PEAK_GBS, 4)})
                print(f"# shape {waves}x{vpt}: {t['us']:.3f} us", file=sys.stderr, flush=True)
        del prod, cp
        torch.cuda.empty_cache()
    b = np.array([r["bytes"] for r in out["sizes"]], np.float64)
    for key in ("kernel_us", "floor_us", "copy_us"):
        t = np.array([r[key] for r in out["sizes"]], np.float64)
        slope, icpt = np.polyfit(b, t, 1)
        out[key.replace("_us", "_fit")] = {"intercept_us": round(float(icpt), 3),
                                           "slope_gbs": round(float(1e-3 / slope), 1)}
    print(json.dumps({"floor_sweep": out, "steps": steps, "repeats": repeats}), flush=True)


TIMELINE_WORKLOADS = ("ptok_fp8_2520x3072", "table_fp8_2520x3072", "ln_fp8_2520x3072",
                      "modfp8_fp8_2520x3072", "awq_fp8_2520x3072")
TIMELINE_REPEATS = 5


def timeline_summary(rec, rows):
    """Summary of one launch's per-wave records (rows x waves, 8 words each;
    timeline.hpp): phase times in us from the first wave's start, as
    percentiles (0, 10, 50, 90, 99, 100) over waves, and the median time x
    landed by a row's dispatch order on its CU."""
    waves = int(np.count_nonzero(rec[:, 0])) // rows
    r = rec[: rows * waves].astype(np.float64)
    if waves == 0 or np.count_nonzero(r[:, 0]) != rows * waves:
        return {"error": "incomplete records", "waves_per_row": waves}
    t0 = r[:, 0].min()
    u = (r[:, :6] - t0) / 100.0                      # 100 MHz clock -> us
    pct = lambda v: [round(float(np.percentile(v, q)), 2) for q in (0, 10, 50, 90, 99, 100)]
    out = {"waves_per_row": waves, "end_us": round(float(u[:, 5].max()), 2),
           "start": pct(u[:, 0]), "x_issued_after_start": pct(u[:, 1] - u[:, 0]),
           "x_landed": pct(u[:, 2]), "rstd_after_x": pct(u[:, 3] - u[:, 2]),
           "output_pass": pct(u[:, 4] - u[:, 3]), "stores_done": pct(u[:, 5])}
    # Rows on each CU (XCC, SE, SH, CU from the XCC_ID and HW_ID registers),
    # in the order their first wave started.
    hw = rec[: rows * waves, 7].astype(np.int64).reshape(rows, waves)[:, 0]
    xcc = rec[: rows * waves, 6].astype(np.int64).reshape(rows, waves)[:, 0] & 0xF
    cu = (xcc << 8) | (((hw >> 13) & 7) << 5) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 0xF)
    start = u[:, 0].reshape(rows, waves).min(1)
    landed = u[:, 2].reshape(rows, waves).max(1)
    order = np.zeros(rows, np.int64)
    for c in np.unique(cu):
        idx = np.nonzero(cu == c)[0]
        order[idx[np.argsort(start[idx], kind="stable")]] = np.arange(idx.size)
    out["cus"] = int(np.unique(cu).size)
    out["x_landed_by_order_on_cu"] = [round(float(np.median(landed[order == k])), 2)
                                      for k in range(int(order.max()) + 1)]
    return out


def timeline(torch, alnp, inputs, stream, names):
    """Per-wave timelines: for each workload, TIMELINE_REPEATS launches, each
    the last of a back-to-back run over the cold rotation of buffer sets, on
    the timeline build of the library.  Prints one JSON line."""
    L = timeline_lib(alnp)
    if L is None:
        print(json.dumps({"error": "--timeline needs libalnp_timeline.so"}))
        sys.exit(2)
    res = {}
    for name in names:
        if name not in TIMELINE_WORKLOADS:
            print(json.dumps({"error": f"--timeline covers {', '.join(TIMELINE_WORKLOADS)}"}))
            sys.exit(2)
        d = inputs.make("ln", rows=2520, dim=3072) if name.startswith("ln_") else inputs.workload(name)
        rows = d["x"].shape[0]
        sets = sets_for(algorithmic_bytes(name, d), True)
        prod = Producer(name, d, sets, torch, alnp)
        calls = [(getattr(L, fn.__name__), args) for fn, args in prod.calls]
        buf = torch.zeros(rows * 8 * 8, dtype=torch.int64, device="cuda")
        if L.alnp_timeline_set(buf.data_ptr()) != 0:
            raise RuntimeError("alnp_timeline_set failed")
        reps = []
        for rep in range(TIMELINE_REPEATS):
            buf.zero_()
            with torch.cuda.stream(stream):
                for i in range(sets):
                    fn, args = calls[(rep + 1 + i) % sets]
                    st = fn(*args, stream.cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"{name}: status {st}")
            torch.cuda.synchronize()
            reps.append(timeline_summary(buf.cpu().numpy().reshape(rows * 8, 8), rows))
            print(f"# timeline {name} launch {rep}: end {reps[-1].get('end_us')} us",
                  file=sys.stderr, flush=True)
        L.alnp_timeline_set(None)
        torch.cuda.synchronize()
        res[name] = reps
        del prod, buf
        torch.cuda.empty_cache()
    print(json.dumps({"timeline": res, "clock": "s_memrealtime, 100 MHz", "launches": TIMELINE_REPEATS}))


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; the producers are "
                          "row-independent and would shard rows across GPUs with no "
                          "exchange, but no multi-GPU path exists", "n_gpus": a.gpus}))
        sys.exit(2)
    modes = [m for m in a.modes.split(",") if m in ("cold", "warm")]
    err = counter_guard(a, modes)
    if err:
        print(json.dumps({"error": err, "modes": modes, "steps": a.steps}))
        sys.exit(2)
    import torch

    import dit_adaptive_layernorm_amd as alnp
    from dit_adaptive_layernorm_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    use_graph = not a.direct
    repeats = 1 if a.counters else max(1, a.repeats)
    F = None if (a.no_floor or a.counters) else floor_lib()
    if a.calibrate_copy:
        calibrate_copy(torch, floor_lib())
        return
    stream = torch.cuda.Stream()
    if a.timeline:
        timeline(torch, alnp, inputs, stream,
                 [n for n in a.only.split(",") if n] or list(TIMELINE_WORKLOADS))
        return
    if a.floor_sweep:
        if F is None:
            print(json.dumps({"error": "--floor-sweep needs libalnp_floor.so"}))
            sys.exit(2)
        floor_sweep(torch, alnp, inputs, F, stream, a.steps, a.warmup, use_graph, repeats)
        return

    head = "ptok_fp8_2520x3072"
    names = [head] if a.only_headline else [
        head, "table_fp8_2520x3072", "bcast_fp8_16x2048", "ln_fp8_2520x3072",
        "ln_fp4_4096x3072", "modulation6_1x5070x3072", "rmsmod_bf16_37810x5376",
        "mxfp8_ptok_2520x3072", "mxfp8_table_2520x3072", "ln_mxfp4_4096x3072",
        "modfp8_fp8_2520x3072", "awq_fp8_2520x3072", "adaln_fp4_4096x3072",
        "adaln_fp4_swz_modfp8_4096x3072", "residual_bf16_5070x3072"]
    if a.only:
        names = [n for n in a.only.split(",") if n]
    results = {}
    head_inputs = None
    if F is None and not (a.no_floor or a.counters):
        print("# libalnp_floor.so not built: no practical floors", file=sys.stderr, flush=True)
    for name in names:
        if name == "ln_fp8_2520x3072":
            d = inputs.make("ln", rows=2520, dim=3072)
        elif name == "mxfp8_ptok_2520x3072":
            d = inputs.workload("ptok_fp8_2520x3072")
        elif name == "mxfp8_table_2520x3072":
            d = inputs.workload("table_fp8_2520x3072")
        elif name == "ln_mxfp4_4096x3072":
            d = inputs.workload("ln_fp4_4096x3072")
        else:
            d = inputs.workload(name)
        if name == head:
            head_inputs = d
        nbytes = algorithmic_bytes(name, d)
        r = {"bytes": nbytes}
        for mode in modes:
            cold = mode == "cold"
            sets = sets_for(nbytes, cold)
            print(f"# timing {name} {mode}: {sets} buffer sets, {a.steps} steps x {repeats}",
                  file=sys.stderr, flush=True)
            prod = Producer(name, d, sets, torch, alnp, F if cold else None)
            # The producer, its memory-only floor and a plain copy of the same
            # bytes, their windows interleaved (time_interleaved).
            variants = [(prod.launch, sets)]
            if prod.floor_calls:
                variants.append((prod.launch_floor, sets))
            cp = CopyCeiling(nbytes, True, torch, F) if cold and F is not None else None
            if cp is not None:
                variants.append((cp.launch, cp.sets))
            res = time_interleaved(torch, stream, variants, a.steps, a.warmup, use_graph, repeats)
            t = res[0]
            f = res[1] if prod.floor_calls else None
            c = res[-1] if cp is not None else None
            print(f"# launches {name} {mode} producer: warmup {a.warmup}, burst 16, spacer "
                  f"{t['spacer']}, steps {a.steps}, tail {TAIL_LAUNCHES if use_graph else 0}, "
                  f"repeats {repeats}, graph {int(use_graph)}, total {t['launches']}, "
                  f"interleaved with {len(variants) - 1} other series",
                  file=sys.stderr, flush=True)
            rec = rounded(t)
            rec["spacer_launches"] = t["spacer"]
            rec.update({"gbs": round(nbytes / t["us"] / 1e3, 1), "sets": sets,
                        "footprint_mb": round(sets * nbytes / 2**20, 1)})
            if f is not None:
                rec["floor_us"] = round(f["us"], 3)
                rec["floor_us_range"] = [round(f["min"], 3), round(f["max"], 3)]
                rec["floor_frac_of_peak"] = round(nbytes / f["us"] / 1e3 / HBM_PEAK_GBS, 4)
                rec["frac_of_floor"] = round(f["us"] / t["us"], 4)
            if c is not None:
                rec["copy_us"] = round(c["us"], 3)
                rec["copy_frac_of_peak"] = round(cp.nbytes / c["us"] / 1e3 / HBM_PEAK_GBS, 4)
            del prod, cp
            r[mode] = rec
            torch.cuda.empty_cache()
        note = ""
        if "cold" in r and "floor_us" in r["cold"]:
            c = r["cold"]
            note = (f"; memory-only floor {c['floor_us']} us "
                    f"({100 * c['floor_frac_of_peak']:.1f}% of peak), "
                    f"kernel at {100 * c['frac_of_floor']:.1f}% of it")
        if "cold" in r and "copy_us" in r["cold"]:
            note += f"; copy of the same bytes {r['cold']['copy_us']} us"
        print(f"# {name}: " + ", ".join(
            f"{m} {r[m]['us_per_call']} us [{r[m]['us_min']}, {r[m]['us_max']}] "
            f"({r[m]['gbs']} GB/s)" for m in modes) + note, file=sys.stderr, flush=True)
        results[name] = r

    if head not in results or "cold" not in results[head] or "warm" not in results[head]:
        print(json.dumps({"partial": True, "steps": a.steps, "repeats": repeats,
                          "rows": results}), flush=True)
        return
    h = results[head]
    us = h["cold"]["us_per_call"]
    gbs = h["cold"]["gbs"]
    traffic = measured_traffic(head)
    line = {
        "metric": "us/call and achieved HBM GB/s (% of peak) for AdaLN->FP8 at 2520x3072",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(THOR_PTOK_US / us, 3),
        "vs_baseline_ref": "pages' NVIDIA Thor SM110a per-token M2520 D3072 raw op, 229.922 us "
                           "(another machine; context only)",
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.1) per-token scale/shift, bf16)",
        "config": {"workload": head, "rows": 2520, "dim": 3072, "act_scale": 0.025,
                   "eps": 1e-5, "io": "bf16 in, e4m3 out, fp32 arithmetic",
                   "timing": "cold", "buffer_sets": h["cold"]["sets"],
                   "footprint_mb": h["cold"]["footprint_mb"],
                   "launch": "hipgraph" if use_graph else "direct",
                   "repeats": repeats,
                   "statistic": f"median of {repeats} timed windows of exactly {a.steps} "
                                "launches, each between two event-record nodes of one graph "
                                "that first rotates through every buffer set untimed"},
        "us_per_call": us,
        "us_range": [h["cold"]["us_min"], h["cold"]["us_max"]],
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "warm_us_per_call": h["warm"]["us_per_call"],
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_adaln_fp8_rows<3 vectors/thread, 2 waves, per-token>",
                     "algorithmic_bytes_per_launch": h["bytes"]},
        "rows": {k: v for k, v in results.items() if k != head},
    }
    c = h["cold"]
    if "floor_us" in c:
        line["roofline"]["practical_floor"] = {
            "us": c["floor_us"], "achieved": round(h["bytes"] / c["floor_us"] / 1e3, 1),
            "frac_of_peak": c["floor_frac_of_peak"], "kernel_frac_of_floor": c["frac_of_floor"],
            "what": "memory-only counterpart (libalnp_floor.so): the same loads and stores in "
                    "the producer's row shape, no arithmetic, timed the same way"}
    if "copy_us" in c:
        line["roofline"]["copy_ceiling"] = {
            "us": c["copy_us"], "frac_of_peak": c["copy_frac_of_peak"],
            "what": "plain device copy (alnp_floor_copy) of the same number of bytes, half read "
                    "and half written, timed the same way"}
    if not (a.no_overhead or a.only_headline or a.only or a.counters):
        line["launch_overhead"] = launch_overhead(torch, alnp, inputs, stream, repeats=repeats)
    if not (a.no_cpu_baseline or a.counters):
        line["cpu_baseline"] = cpu_baseline(head_inputs, h["bytes"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
