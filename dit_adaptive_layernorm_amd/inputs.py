"""Seeded synthetic inputs for the adaptive-LayerNorm producers.

This module only draws random numbers and lays them out; it holds none of the
producers' arithmetic.  It serves the parity tests (both the HIP path and the
CPU oracle get the same arrays) and the benchmark.

Recipe: numpy PCG64 seeded with SeedSequence([seed, stream_id]), one stream id
per tensor; standard normal draws in float64, scaled by sigma, rounded to
float32; bf16 tensors are then rounded to bf16 by torch's CPU conversion
(round to nearest even).  bf16 tensors are returned as uint16 bit patterns.
Tensors too large to draw on the host (calls past 2^32 elements) are drawn on
the GPU instead (device_normal).

The workloads follow the shapes the pages measure (Wan-video 2520 x 3072 and
4096 x 3072 rows, the decode-action 16 x 2048 row block, the six-way
modulation producer at B1 S5070 D3072) with value distributions chosen per
workload: activations N(0, 1), modulation operands N(0, 0.1), timestep
embedding chunks N(0, 0.5), and for the FP4 producer a 1% Bernoulli mask of
x20 outliers applied before the bf16 rounding.

The RMSNorm-modulation producer runs at the h3 page's canonical hidden shape,
37810 tokens x 5376, with its request layout of three segments (tokens
[0, 100) use modulation row 1, [100, 514) row 2, the rest row 0): RMSNorm
weight 1 + N(0, 0.1), scale/shift tables (3, dim) N(0, 0.1).  Small parity
cases draw each row's segment uniformly instead.
"""
from __future__ import annotations

import numpy as np
import torch

# One stream id per tensor role, so that adding a tensor never shifts another.
STREAM = {"x": 1, "scale": 2, "shift": 3, "temb": 4, "table": 5, "params": 6,
          "mod": 7, "outlier": 8, "weight": 9, "seg": 10, "scale_fp8": 11,
          "shift_fp8": 12, "inv_s": 13, "gate": 14, "proj": 15}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with torch (library RTNE); uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_f32(shape, sigma: float, seed: int, stream: int) -> np.ndarray:
    return (rng(seed, stream).standard_normal(shape) * sigma).astype(np.float32)


def normal_bf16(shape, sigma: float, seed: int, stream: int) -> np.ndarray:
    return to_bf16_bits(normal_f32(shape, sigma, seed, stream))


def to_e4m3_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 to e4m3 (OCP float8_e4m3fn) with torch's conversion; uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def outlier_bf16(shape, seed: int, stream: int, outlier_stream: int,
                 p: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """N(0,1) with each element independently (probability p) scaled by factor."""
    f = normal_f32(shape, 1.0, seed, stream)
    mask = rng(seed, outlier_stream).random(shape) < p
    f = np.where(mask, f * np.float32(factor), f).astype(np.float32)
    return to_bf16_bits(f)


# ---- device-side draws, for calls too large to draw on the host -------------

def device_normal(shape, sigma: float, seed: int, stream: int, dtype=torch.bfloat16,
                  device: str = "cuda", chunk: int = 1 << 28) -> torch.Tensor:
    """N(0, sigma) drawn on the GPU: torch's generator for `device`, seeded
    with (seed << 8) + stream, float32 draws of `chunk` elements at a time,
    scaled by sigma and rounded to `dtype` by torch (round to nearest even).
    Deterministic for a given seed, stream, shape and chunk.  Callers copy
    the rows they check to the host."""
    g = torch.Generator(device=device).manual_seed((seed << 8) + stream)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for a in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - a)
        flat[a:a + n] = (torch.randn(n, generator=g, device=device) * sigma).to(dtype)
    return out


# ---- the five workloads ----------------------------------------------------

ACT_SCALE = 0.025
EPS = 1e-5

WORKLOADS = {
    "bcast_fp8_16x2048": dict(kind="bcast", rows=16, dim=2048),
    "ptok_fp8_2520x3072": dict(kind="ptok", rows=2520, dim=3072),
    "table_fp8_2520x3072": dict(kind="table", rows=2520, dim=3072, chunks=6,
                                shift_idx=0, scale_idx=1),
    "modulation6_1x5070x3072": dict(kind="mod6", batch=1, seq=5070, dim=3072),
    "ln_fp4_4096x3072": dict(kind="fp4", rows=4096, dim=3072),
    "rmsmod_bf16_37810x5376": dict(kind="rmsmod", rows=37810, dim=5376, segments=3,
                                   layout="h3"),
    # the README's further entries, at the shapes above: e4m3 modulation
    # operands and AWQ smoothing at the per-token size, AdaLN -> FP4 at the FP4
    # size, and the residual gate at the six-way size (a per-token gate)
    "modfp8_fp8_2520x3072": dict(kind="modfp8", rows=2520, dim=3072),
    "awq_fp8_2520x3072": dict(kind="awq", rows=2520, dim=3072),
    "adaln_fp4_4096x3072": dict(kind="adaln_fp4", rows=4096, dim=3072),
    "adaln_fp4_swz_modfp8_4096x3072": dict(kind="adaln_fp4_modfp8", rows=4096, dim=3072),
    "residual_bf16_5070x3072": dict(kind="residual", rows=5070, dim=3072),
}

# The h3 page's request layout: (first token, end token, modulation row).
H3_SEGMENTS = ((0, 100, 1), (100, 514, 2), (514, None, 0))


def segment_ids(rows: int, segments: int, layout: str, seed: int) -> np.ndarray:
    """Per-row modulation row index (int32): the h3 layout, or uniform draws."""
    if layout == "h3":
        seg = np.zeros(rows, np.int32)
        for a, b, k in H3_SEGMENTS:
            seg[a:rows if b is None else min(b, rows)] = k
        return seg
    return rng(seed, STREAM["seg"]).integers(0, segments, rows).astype(np.int32)


def make(kind: str, seed: int = 0, rows: int = 0, dim: int = 0, chunks: int = 6,
         shift_idx: int = 0, scale_idx: int = 1, batch: int = 1, seq: int = 0,
         outliers: bool = True, segments: int = 3, layout: str = "random") -> dict:
    """Inputs for one producer at any shape, same distributions as above.

    kind: "ln" | "bcast" | "ptok" | "table" | "fp4" | "mod6" | "rmsmod", or the
    variants "modfp8" | "awq" | "adaln_fp4" | "adaln_fp4_modfp8" | "residual".
    """
    s = STREAM
    if kind == "residual":
        # residual stream N(0, 1), per-token gate N(0, 0.5), projection N(0, 2)
        return dict(residual=normal_bf16((rows, dim), 1.0, seed, s["x"]),
                    gate=normal_bf16((rows, dim), 0.5, seed, s["gate"]),
                    proj=normal_bf16((rows, dim), 2.0, seed, s["proj"]))
    if kind in ("adaln_fp4", "adaln_fp4_modfp8"):
        d = make("fp4", seed=seed, rows=rows, dim=dim, outliers=outliers)
        if kind == "adaln_fp4":
            d["scale"] = normal_bf16((dim,), 0.1, seed, s["scale"])
            d["shift"] = normal_bf16((dim,), 0.1, seed, s["shift"])
        else:
            d.update(modfp8_operands(dim, seed))
        return d
    if kind == "rmsmod":
        w = (normal_f32((dim,), 0.1, seed, s["weight"]) + np.float32(1.0)).astype(np.float32)
        return dict(x=normal_bf16((rows, dim), 1.0, seed, s["x"]), weight=to_bf16_bits(w),
                    scale=normal_bf16((segments, dim), 0.1, seed, s["scale"]),
                    shift=normal_bf16((segments, dim), 0.1, seed, s["shift"]),
                    seg=segment_ids(rows, segments, layout, seed), eps=EPS)
    if kind == "mod6":
        return dict(params=normal_f32((batch, seq, 6, dim), 1.0, seed, s["params"]),
                    mod=normal_f32((6, dim), 0.1, seed, s["mod"]))
    if kind == "fp4":
        x = (outlier_bf16((rows, dim), seed, s["x"], s["outlier"]) if outliers
             else normal_bf16((rows, dim), 1.0, seed, s["x"]))
        return dict(x=x, eps=EPS)
    d = dict(x=normal_bf16((rows, dim), 1.0, seed, s["x"]), act_scale=ACT_SCALE, eps=EPS)
    if kind == "bcast":
        d["scale"] = normal_bf16((dim,), 0.1, seed, s["scale"])
        d["shift"] = normal_bf16((dim,), 0.1, seed, s["shift"])
    elif kind == "ptok":
        d["scale"] = normal_bf16((rows, dim), 0.1, seed, s["scale"])
        d["shift"] = normal_bf16((rows, dim), 0.1, seed, s["shift"])
    elif kind == "table":
        d["temb"] = normal_bf16((rows, chunks, dim), 0.5, seed, s["temb"])
        d["table"] = normal_f32((chunks, dim), 0.1, seed, s["table"])
        d["shift_idx"] = shift_idx
        d["scale_idx"] = scale_idx
    elif kind == "modfp8":
        d.update(modfp8_operands(dim, seed))
    elif kind == "awq":
        d["scale"] = normal_bf16((dim,), 0.1, seed, s["scale"])
        d["shift"] = normal_bf16((dim,), 0.1, seed, s["shift"])
        # per-channel smoothing factors in [0.5, ~2.5)
        d["inv_s"] = to_bf16_bits(np.abs(normal_f32((dim,), 0.5, seed, s["inv_s"])) + np.float32(0.5))
    elif kind != "ln":
        raise ValueError(kind)
    return d


# fp32 dequantization scalars of the e4m3 modulation operands
MODFP8_DEQ = (0.5, 0.25)


def modfp8_operands(dim: int, seed: int) -> dict:
    """e4m3 (dim,) scale / shift codes of N(0, 0.3) draws and their fp32
    dequantization scalars (MODFP8_DEQ), so the operands are N(0, 0.15) and
    N(0, 0.075) in value."""
    return dict(scale_fp8=to_e4m3_bits(normal_f32((dim,), 0.3, seed, STREAM["scale_fp8"])),
                shift_fp8=to_e4m3_bits(normal_f32((dim,), 0.3, seed, STREAM["shift_fp8"])),
                scale_deq=MODFP8_DEQ[0], shift_deq=MODFP8_DEQ[1])


def workload(name: str, seed: int = 0) -> dict:
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    d = make(kind, seed=seed, **w)
    d["kind"] = kind
    return d
