"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device
and comparing the HIP path's codes and statistics with the oracle's.

Tolerances (the pages' validation policy, "adaptive-layernorm-producers"
README, "Validation": exact small shapes, only adjacent FP8-code boundary
differences on long shapes):
  - FP8 / FP4 codes: at least 99.9% equal to the oracle's, every other code
    within one step on the signed-ordinal scale (+-magnitude index, +-0 -> 0),
    so no sign flips except through zero.  FP4 block-scale bytes likewise.
  - Row statistics: |dmean| <= 1e-5 * max(|mean|, sigma_row) (a purely relative
    bound is ill-posed for mean ~ 0), |drstd| <= 1e-5 * rstd.
  - bf16 (six-way): bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

MIN_EQUAL = 0.999


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def act(v: float = 0.025) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def misaligned_like(shape, dtype, elem_offset=1):
    """A contiguous tensor whose data pointer is elem_offset elements past a
    256-byte aligned allocation (so not 16-byte aligned)."""
    n = int(np.prod(shape))
    base = torch.empty(n + elem_offset + 16, dtype=dtype, device="cuda")
    return base[elem_offset:elem_offset + n].view(shape)


def e4m3_ordinal(c):
    c = np.asarray(c, np.uint8)
    m = (c & 0x7F).astype(np.int32)
    return np.where(c & 0x80, -m, m)


def e2m1_ordinal(c):
    c = np.asarray(c, np.uint8)
    m = (c & 0x7).astype(np.int32)
    return np.where(c & 0x8, -m, m)


def unpack_e2m1(packed):
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def assert_codes_close(got, ref, ordinal, what="codes", min_equal=MIN_EQUAL):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return
    eq = got == ref
    # +0 and -0 are the same value; count them as equal too.
    d = np.abs(ordinal(got) - ordinal(ref))
    frac = np.mean(eq | (d == 0))
    assert frac >= min_equal, f"{what}: only {frac:.6f} equal"
    worst = int(d.max())
    assert worst <= 1, f"{what}: a code is {worst} steps away (at {np.unravel_index(d.argmax(), d.shape)})"


def assert_stats_close(mean, rstd, ref_mean, ref_rstd, rel=1e-5):
    mean, rstd = np.asarray(mean, np.float64), np.asarray(rstd, np.float64)
    rm, rr = np.asarray(ref_mean, np.float64), np.asarray(ref_rstd, np.float64)
    sigma = 1.0 / rr
    assert np.all(np.abs(mean - rm) <= rel * np.maximum(np.abs(rm), sigma)), "row mean"
    assert np.all(np.abs(rstd - rr) <= rel * rr), "row rstd"


def sample_rows(rows: int, n: int, seed: int = 0) -> np.ndarray:
    """Sorted sample of row indices, always including the first and last."""
    r = np.random.default_rng(seed)
    pick = r.choice(rows, size=min(n, rows), replace=False)
    return np.unique(np.concatenate([pick, [0, rows - 1]]))
