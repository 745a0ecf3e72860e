"""The memory-only counterparts of the producers (libalnp_floor.so), which the
benchmark times beside them as a practical floor.  CPU: the library loads,
exports its two launchers and rejects what the row kernels do not take
before touching the GPU.  GPU: every floor kernel stores exactly the bytes its
producer stores (all output and scale bytes, nothing else), checked against a
numpy model of its XOR pattern."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "dit_adaptive_layernorm_amd", "libalnp_floor.so")
FP8, NVFP4, BF16, MXFP8, MXFP4, NVFP4_TILED = 0, 1, 2, 3, 4, 5


def floor_lib():
    if not os.path.exists(PATH):
        pytest.fail("libalnp_floor.so is not built (run the build)")
    F = ctypes.CDLL(PATH)
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


def test_floor_library_exports_and_rejects_bad_arguments():
    F = floor_lib()
    A, B = 1 << 12, 1 << 13  # aligned stand-in addresses: never dereferenced here
    assert F.alnp_floor_rows(A, None, None, 0, 0, 64, FP8, B, None, None) == 0   # no rows: no-op
    assert F.alnp_floor_rows(None, None, None, 0, 4, 64, FP8, B, None, None) == -1
    assert F.alnp_floor_rows(A, None, None, 0, 4, 48, FP8, B, None, None) == -1  # dim % 32
    assert F.alnp_floor_rows(A + 4, None, None, 0, 4, 64, FP8, B, None, None) == -1
    assert F.alnp_floor_rows(A, None, A, 0, 4, 64, FP8, B, None, None) == -1     # b without a
    assert F.alnp_floor_rows(A, None, None, -1, 4, 64, FP8, B, None, None) == -1
    for kind in (NVFP4, MXFP8, MXFP4, NVFP4_TILED):
        assert F.alnp_floor_rows(A, None, None, 0, 4, 64, kind, B, None, None) == -1
    assert F.alnp_floor_rows(A, None, None, 0, 4, 96, NVFP4_TILED, B, B, None) == -1  # dim % 64
    assert F.alnp_floor_rows(A, None, None, 0, 4, 64, 9, B, None, None) == -2
    assert F.alnp_floor_rows(A, None, None, 0, 4, 1 << 21, FP8, B, None, None) == -1
    outs = (ctypes.c_void_p * 6)(*([B] * 6))
    assert F.alnp_floor_modulation6(A, 0, 64, outs, None) == 0
    assert F.alnp_floor_modulation6(A, 4, 60, outs, None) == -1
    outs[3] = None
    assert F.alnp_floor_modulation6(A, 4, 64, outs, None) == -1
    # Explicit row shapes: the shape must cover the row (dim 3072 = 384
    # vectors), with only the last vector slot past its end.
    shape = lambda w, v, dim=3072: F.alnp_floor_rows_shape(A, None, None, 0, 0, dim, FP8, B, None,
                                                           w, v, None)
    for w, v in ((1, 6), (2, 3), (4, 2), (8, 1)):
        assert shape(w, v) == 0
    for w, v in ((3, 2), (1, 5), (2, 2), (4, 3), (8, 2), (2, 0), (2, 9)):
        assert shape(w, v) == -1, (w, v)
    # Copies: 16-byte multiples of 16-byte aligned pointers.
    assert F.alnp_floor_copy(A, B, 0, None) == 0
    assert F.alnp_floor_copy(A, B, 24, None) == -1
    assert F.alnp_floor_copy(A + 8, B, 32, None) == -1
    assert F.alnp_floor_copy(None, B, 32, None) == -1
    assert F.alnp_floor_copy(A, B, -16, None) == -1


def xor_words(x, a=None, b=None):
    """(rows, dim) uint16 streams -> (rows, dim/8, 4) uint32 words x ^ a ^ b."""
    w = np.ascontiguousarray(x).view(np.uint32).reshape(x.shape[0], -1, 4).copy()
    for s in (a, b):
        if s is not None:
            w ^= np.broadcast_to(np.ascontiguousarray(s), x.shape).copy().view(np.uint32).reshape(w.shape)
    return w


def expected_rows(kind, x, a=None, b=None):
    rows, dim = x.shape
    w = xor_words(x, a, b)
    if kind == BF16:
        return w.reshape(rows, -1).view(np.uint16).reshape(rows, dim), None
    if kind in (FP8, MXFP8):
        out = np.stack([w[..., 0] ^ w[..., 1], w[..., 2] ^ w[..., 3]], -1).reshape(rows, -1)
        out = out.view(np.uint8).reshape(rows, dim)
    else:
        out = (w[..., 0] ^ w[..., 1] ^ w[..., 2] ^ w[..., 3]).view(np.uint8).reshape(rows, dim // 2)
    lo = (w[..., 0] & 0xFF).astype(np.uint8)
    if kind == NVFP4:
        return out, lo[:, 0::2]
    if kind in (MXFP8, MXFP4):
        return out, lo[:, 0::4]
    return out, None


@pytest.mark.gpu
@pytest.mark.parametrize("kind,nin,stride_kind,rows,dim", [
    (FP8, 3, "ptok", 5, 3072), (FP8, 3, "bcast", 3, 2048), (FP8, 1, "none", 4, 3072),
    (FP8, 3, "table", 3, 3072), (NVFP4, 1, "none", 4, 3072), (BF16, 1, "none", 3, 5376),
    (MXFP8, 3, "ptok", 3, 3072), (MXFP8, 3, "table", 2, 3072), (MXFP4, 1, "none", 3, 3072),
    (FP8, 3, "ptok", 3, 96), (NVFP4, 1, "none", 2, 96), (BF16, 1, "none", 2, 160),
])
def test_floor_rows_store_the_producers_bytes(kind, nin, stride_kind, rows, dim):
    import torch
    F = floor_lib()
    print(f"floor rows kind={kind} nin={nin} {stride_kind} {rows}x{dim}", flush=True)
    r = np.random.default_rng(kind * 100 + rows + dim)
    u16 = lambda shape: r.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    dev = lambda h: torch.from_numpy(h.view(np.int16)).cuda()
    x = u16((rows, dim))
    chunks, si, hi = 6, 1, 4
    if stride_kind == "table":
        temb = u16((rows, chunks, dim))
        a_h, b_h = temb[:, si, :], temb[:, hi, :]
        t_d = dev(temb)
        a_ptr = t_d.data_ptr() + 2 * si * dim
        b_ptr = t_d.data_ptr() + 2 * hi * dim
        stride = chunks * dim
    elif stride_kind in ("ptok", "bcast"):
        shape = (rows, dim) if stride_kind == "ptok" else (dim,)
        a_h, b_h = u16(shape), u16(shape)
        a_d, b_d = dev(a_h), dev(b_h)
        a_ptr, b_ptr = a_d.data_ptr(), b_d.data_ptr()
        stride = dim if stride_kind == "ptok" else 0
    else:
        a_h = b_h = None
        a_ptr = b_ptr = None
        stride = 0
    want, want_s = expected_rows(kind, x, a_h, b_h)
    out = torch.full((want.size * want.itemsize,), 0xA5, dtype=torch.uint8, device="cuda")
    scales = None
    if want_s is not None:
        scales = torch.full((want_s.size,), 0x5A, dtype=torch.uint8, device="cuda")
    x_d = dev(x)
    st = F.alnp_floor_rows(x_d.data_ptr(), a_ptr, b_ptr, stride, rows, dim, kind, out.data_ptr(),
                           scales.data_ptr() if scales is not None else None,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, np.ascontiguousarray(want).view(np.uint8).reshape(-1))
    if want_s is not None:
        assert np.array_equal(scales.cpu().numpy(), want_s.reshape(-1))


def tiled_offset(r, c, cols):
    """The 128x4 tiled scale layout: 512-byte tiles of 128 rows x 4 columns,
    tile-row-major; (r mod 32) picks a 16-byte unit, (r div 32) mod 4 the
    4-byte group in it, c mod 4 the byte."""
    tile = (r // 128) * ((cols + 3) // 4) + c // 4
    return tile * 512 + (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4


@pytest.mark.gpu
@pytest.mark.parametrize("rows,dim", [(5, 3072), (256, 3072), (512, 128)])
def test_floor_rows_tiled_scales(rows, dim):
    """The tiled-scale floor stores the NVFP4 floor's codes, and its scale
    bytes at their tiled positions (rows a multiple of 256 take the XCD-grouped
    order, which must not change which bytes land where)."""
    import torch
    F = floor_lib()
    print(f"floor rows tiled {rows}x{dim}", flush=True)
    r = np.random.default_rng(rows + dim)
    x = r.integers(0, 1 << 16, size=(rows, dim), dtype=np.uint16)
    want, want_rm = expected_rows(NVFP4, x)
    cols = dim // 16
    size = -(-rows // 128) * 128 * (-(-cols // 4) * 4)
    want_s = np.full(size, 0x5A, np.uint8)
    for rr in range(rows):
        for c in range(cols):
            want_s[tiled_offset(rr, c, cols)] = want_rm[rr, c]
    out = torch.full((want.size,), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((size,), 0x5A, dtype=torch.uint8, device="cuda")
    x_d = torch.from_numpy(x.view(np.int16)).cuda()
    st = F.alnp_floor_rows(x_d.data_ptr(), None, None, 0, rows, dim, NVFP4_TILED, out.data_ptr(),
                           scales.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.ascontiguousarray(want).view(np.uint8).reshape(-1))
    assert np.array_equal(scales.cpu().numpy(), want_s)


@pytest.mark.gpu
@pytest.mark.parametrize("tokens,dim", [(9, 256), (12, 3072)])
def test_floor_modulation6_stores_the_six_outputs(tokens, dim):
    import torch
    F = floor_lib()
    print(f"floor modulation6 {tokens}x{dim}", flush=True)
    r = np.random.default_rng(tokens + dim)
    p = r.integers(0, 1 << 32, size=(tokens, 6, dim), dtype=np.uint32)
    p_d = torch.from_numpy(p.view(np.int32)).cuda()
    outs = [torch.full((tokens, dim), 0x1234, dtype=torch.int16, device="cuda") for _ in range(6)]
    arr = (ctypes.c_void_p * 6)(*[o.data_ptr() for o in outs])
    st = F.alnp_floor_modulation6(p_d.data_ptr(), tokens, dim, arr,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for k in range(6):
        want = (p[:, k, :] >> 16).astype(np.uint16)
        assert np.array_equal(outs[k].cpu().numpy().view(np.uint16), want), k


@pytest.mark.gpu
@pytest.mark.parametrize("waves,vpt", [(1, 6), (2, 3), (4, 2), (8, 1)])
def test_floor_rows_shape_stores_the_same_bytes(waves, vpt):
    """Every row shape of the per-token pattern stores the same bytes."""
    import torch
    F = floor_lib()
    rows, dim = 5, 3072
    print(f"floor rows shape {waves}x{vpt} {rows}x{dim}", flush=True)
    r = np.random.default_rng(waves * 10 + vpt)
    u16 = lambda shape: r.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    dev = lambda h: torch.from_numpy(h.view(np.int16)).cuda()
    x, a, b = u16((rows, dim)), u16((rows, dim)), u16((rows, dim))
    want, _ = expected_rows(FP8, x, a, b)
    out = torch.full((rows * dim,), 0xA5, dtype=torch.uint8, device="cuda")
    xd, ad, bd = dev(x), dev(a), dev(b)
    st = F.alnp_floor_rows_shape(xd.data_ptr(), ad.data_ptr(), bd.data_ptr(), dim, rows, dim, FP8,
                                 out.data_ptr(), None, waves, vpt,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.ascontiguousarray(want).view(np.uint8).reshape(-1))


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 16 * 1023, 16 * 1024 * 5 + 48, 27095040])
def test_floor_copy_copies(nbytes):
    import torch
    F = floor_lib()
    print(f"floor copy {nbytes} bytes", flush=True)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    st = F.alnp_floor_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0x5A).all())
