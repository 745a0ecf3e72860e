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
six-way modulation, RMSNorm modulation, and the MXFP8 / MXFP4 outputs) are
timed the same way at their workload sizes and reported under "rows", each
beside its memory-only floor; the headline JSON line is the per-token FP8
one.

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
COPY_BYTES = 256 << 20         # plain copy used to scale the rocprofv3 byte counters
THOR_PTOK_US = 229.922         # pages: NVIDIA Thor, per-token M2520 D3072, raw op


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
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
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run four plain device copies of 256 MiB (reference for "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE scaling) and exit")
    return p.parse_args()


# ---- workloads ----------------------------------------------------------------

def algorithmic_bytes(name, d):
    """Bytes a producer must move once: inputs read + outputs written."""
    if name.startswith("modulation6"):
        p = d["params"]
        return p.nbytes + d["mod"].nbytes + p.size // 6 * 6 * 2
    x = d["x"]
    rows, dim = x.shape
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
    return F


# out_kind of alnp_floor_rows
FLOOR_FP8, FLOOR_NVFP4, FLOOR_BF16, FLOOR_MXFP8, FLOOR_MXFP4 = 0, 1, 2, 3, 4


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
        x0 = bf(d["x"])
        rows, dim = x0.shape
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


def sets_for(nbytes, cold):
    return max(2, math.ceil(COLD_FOOTPRINT / nbytes)) if cold else 1


def time_producer(prod, steps, warmup, use_graph, torch, stream, floor=False):
    """Average us per step over exactly `steps` launches on `stream` (a
    dedicated stream, as a pipeline would use), measured with HIP events
    recorded on that stream.  With a graph, the `steps` launches are captured
    once and the graph is replayed once untimed (upload) before the timed
    replay.  floor=True times the memory-only counterparts instead."""
    h = stream.cuda_stream
    launch = prod.launch_floor if floor else prod.launch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i, h)
        torch.cuda.synchronize()
        g = None
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                hh = torch.cuda.current_stream().cuda_stream
                for i in range(steps):
                    launch(i, hh)
            g.replay()
            torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        if use_graph:
            g.replay()
        else:
            for i in range(steps):
                launch(i, h)
        t1.record(stream)
        torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) * 1000.0 / steps


# ---- launch overhead at small shapes ---------------------------------------------------

def launch_overhead(torch, alnp, inputs, stream, calls=400, graph_launches=32, replays=50):
    """The pages' small-shape method (Benchmark Results, "Six-way modulation
    producer" and "NVIDIA Thor installed artifact"): per shape, the raw C ABI
    launched directly, the Python wrapper launched directly (A-B-B-A order),
    and a HIP graph of 32 launches replayed, time / 32.  Inputs stay the same
    buffers (warm): these shapes are latency-bound."""
    dev = torch.device("cuda")
    bf = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    L = alnp.lib()
    cases = {}
    act = torch.tensor([0.025], dtype=torch.float32, device=dev)
    for name, kind, rows, dim in (("ptok_fp8_51x1536", "ptok", 51, 1536),
                                  ("table_fp8_51x1536", "table", 51, 1536),
                                  ("ptok_fp8_105x1152", "ptok", 105, 1152),
                                  ("modulation6_1x51x1536", "mod6", 51, 1536)):
        if kind == "mod6":
            d = inputs.make("mod6", batch=1, seq=rows, dim=dim)
            p, m = f32(d["params"]), f32(d["mod"])
            outs = [torch.empty((1, rows, dim), dtype=torch.bfloat16, device=dev) for _ in range(6)]
            arr = (ctypes.c_void_p * 6)(*[o.data_ptr() for o in outs])
            raw = lambda h: L.alnp_adaln_modulation6_bf16(p.data_ptr(), m.data_ptr(), 1, rows, dim, arr, h)
            wrap = lambda h: alnp.adaln_modulation6_bf16(p, m, out=outs)
        elif kind == "ptok":
            d = inputs.make("ptok", rows=rows, dim=dim)
            x, sc, sh = bf(d["x"]), bf(d["scale"]), bf(d["shift"])
            out = torch.empty((rows, dim), dtype=torch.float8_e4m3fn, device=dev)
            raw = lambda h: L.alnp_ada_layer_norm_quant_fp8_ptok_bf16(
                x.data_ptr(), sc.data_ptr(), sh.data_ptr(), act.data_ptr(), 1e-5, rows, dim,
                out.data_ptr(), None, None, h)
            wrap = lambda h: alnp.ada_layer_norm_quant_fp8_ptok_bf16(x, sc, sh, act, out=out)
        else:
            d = inputs.make("table", rows=rows, dim=dim)
            x, te, tb = bf(d["x"]), bf(d["temb"]), f32(d["table"])
            out = torch.empty((rows, dim), dtype=torch.float8_e4m3fn, device=dev)
            raw = lambda h: L.alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(
                x.data_ptr(), te.data_ptr(), tb.data_ptr(), 6, 0, 1, act.data_ptr(), 1e-5, rows,
                dim, out.data_ptr(), None, None, h)
            wrap = lambda h: alnp.ada_layer_norm_quant_fp8_ptok_table_bf16(x, te, tb, act, 0, 1, out=out)

        def direct(fn):
            with torch.cuda.stream(stream):
                h = stream.cuda_stream
                for _ in range(20):
                    fn(h)
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                t0.record(stream)
                for _ in range(calls):
                    fn(h)
                t1.record(stream)
                torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1000.0 / calls

        def graphed(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                    hh = torch.cuda.current_stream().cuda_stream
                    for _ in range(graph_launches):
                        fn(hh)
                g.replay()
                torch.cuda.synchronize()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                t0.record(stream)
                for _ in range(replays):
                    g.replay()
                t1.record(stream)
                torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1000.0 / (replays * graph_launches)

        a1, b1, b2, a2 = direct(raw), direct(wrap), direct(wrap), direct(raw)
        ga, gb = graphed(raw), graphed(wrap)
        nat, wr = (a1 + a2) / 2, (b1 + b2) / 2
        cases[name] = {"native_us": round(nat, 3), "wrapper_us": round(wr, 3),
                       "graph_native_us": round(ga, 3), "graph_wrapper_us": round(gb, 3),
                       "wrapper_over_native": round(wr / nat, 3)}
        print(f"# overhead {name}: native {nat:.3f} us, wrapper {wr:.3f} us, graph native "
              f"{ga:.3f} us, graph wrapper {gb:.3f} us", file=sys.stderr, flush=True)
    return cases


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

def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the producers are "
                          "row-independent and would shard rows across GPUs with no "
                          "exchange, but no multi-GPU path is built", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    import dit_adaptive_layernorm_amd as alnp
    from dit_adaptive_layernorm_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    use_graph = not a.direct
    if a.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "copies": 4}))
        return

    head = "ptok_fp8_2520x3072"
    names = [head] if a.only_headline else [
        head, "table_fp8_2520x3072", "bcast_fp8_16x2048", "ln_fp8_2520x3072",
        "ln_fp4_4096x3072", "modulation6_1x5070x3072", "rmsmod_bf16_37810x5376",
        "mxfp8_ptok_2520x3072", "mxfp8_table_2520x3072", "ln_mxfp4_4096x3072"]
    if a.only:
        names = [n for n in a.only.split(",") if n]
    modes = [m for m in a.modes.split(",") if m in ("cold", "warm")]
    results = {}
    head_inputs = None
    stream = torch.cuda.Stream()
    F = None if a.no_floor else floor_lib()
    if F is None and not a.no_floor:
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
            sets = sets_for(nbytes, mode == "cold")
            prod = Producer(name, d, sets, torch, alnp, F if mode == "cold" else None)
            us = time_producer(prod, a.steps, a.warmup, use_graph, torch, stream)
            r[mode] = {"us_per_call": round(us, 3), "gbs": round(nbytes / us / 1e3, 1),
                       "sets": sets, "footprint_mb": round(sets * nbytes / 2**20, 1)}
            if prod.floor_calls:
                fus = time_producer(prod, a.steps, a.warmup, use_graph, torch, stream, floor=True)
                r[mode]["floor_us"] = round(fus, 3)
                r[mode]["floor_frac_of_peak"] = round(nbytes / fus / 1e3 / HBM_PEAK_GBS, 4)
                r[mode]["frac_of_floor"] = round(fus / us, 4)
            del prod
            torch.cuda.empty_cache()
        floor_note = ""
        if "cold" in r and "floor_us" in r["cold"]:
            c = r["cold"]
            floor_note = (f"; memory-only floor {c['floor_us']} us "
                          f"({100 * c['floor_frac_of_peak']:.1f}% of peak), "
                          f"kernel at {100 * c['frac_of_floor']:.1f}% of it")
        print(f"# {name}: " + ", ".join(f"{m} {r[m]['us_per_call']} us ({r[m]['gbs']} GB/s)"
                                        for m in modes) + floor_note, file=sys.stderr, flush=True)
        results[name] = r

    if head not in results or "cold" not in results[head] or "warm" not in results[head]:
        print(json.dumps({"partial": True, "rows": results}), flush=True)
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
                   "eps": 1e-5, "timing": "cold", "buffer_sets": h["cold"]["sets"],
                   "footprint_mb": h["cold"]["footprint_mb"],
                   "launch": "hipgraph" if use_graph else "direct"},
        "us_per_call": us,
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "warm_us_per_call": h["warm"]["us_per_call"],
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_adaln_fp8_rows<3 vectors/thread, 2 waves, per-token>",
                     "algorithmic_bytes_per_launch": h["bytes"]},
        "rows": {k: v for k, v in results.items() if k != head},
    }
    if "floor_us" in h["cold"]:
        c = h["cold"]
        line["roofline"]["practical_floor"] = {
            "us": c["floor_us"], "achieved": round(h["bytes"] / c["floor_us"] / 1e3, 1),
            "frac_of_peak": c["floor_frac_of_peak"], "kernel_frac_of_floor": c["frac_of_floor"],
            "what": "memory-only counterpart (libalnp_floor.so): the same loads and stores in "
                    "the producer's row shape, no arithmetic, timed the same way"}
    if not a.no_overhead and not a.only_headline and not a.only:
        line["launch_overhead"] = launch_overhead(torch, alnp, inputs, stream)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head_inputs, h["bytes"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
