// floor.hip -- memory-only counterparts of the producers, for measurement.
//
// Each kernel here makes the same global loads and stores as a producer, in
// the producer's row shape (its waves per row and vectors per thread, one
// workgroup per row; the six-way token-group mapping), and replaces the
// method's arithmetic by a few XORs that keep every loaded byte live.  The
// table and RMSNorm producers put two rows in a workgroup on large calls;
// their floors keep one row per workgroup, the plain streaming layout.  Timed
// beside a producer on the same buffers, such a kernel gives the time this
// access pattern takes on the chip with no arithmetic at all: a practical
// floor for the producer, tighter than bytes / vendor peak, which no kernel
// reaches once launch cost and latency are counted.  Built into its own
// library (libalnp_floor.so); nothing here is part of the producers' API.
#include "rows.hpp"

namespace alnp {
namespace {

// Output layouts of the row floor.
enum FloorOut : int {
    kOutFp8 = 0,    // 1 byte per element
    kOutNvfp4 = 1,  // dim/2 bytes of codes + dim/16 scale bytes per row
    kOutBf16 = 2,   // 2 bytes per element
    kOutMxfp8 = 3,  // 1 byte per element + dim/32 scale bytes per row
    kOutMxfp4 = 4,  // dim/2 bytes of codes + dim/32 scale bytes per row
    kOutNvfp4Tiled = 5,  // as kOutNvfp4, scales in the 128x4 tiled layout, rows in
                         // the tiled FP4 producers' XCD-grouped order
};

// Byte offset of scale (r, c) in the 128x4 tiled layout (the producers'
// layout, restated here so that this library stays self-contained).
__device__ __forceinline__ int64_t tiled_offset(int64_t r, int c, int cols)
{
    const int64_t tile = (r >> 7) * ((cols + 3) >> 2) + (c >> 2);
    const int rr = (int)(r & 127);
    return tile * 512 + (rr & 31) * 16 + (rr >> 5) * 4 + (c & 3);
}

struct FloorRowArgs {
    const uint16_t* x;
    const uint16_t* a;      // optional second stream (nullptr: none)
    const uint16_t* b;      // optional third stream
    int64_t ab_stride;      // elements between rows of a and b (0: one shared vector)
    int64_t rows;
    int dim;
    uint8_t* out;
    uint8_t* scales;
};

template <int VPT, int WAVES, int OUT, int NIN>
__global__ __launch_bounds__(WAVES * 64) void k_floor_rows(FloorRowArgs f)
{
    constexpr int T = WAVES * 64;
    const int t = threadIdx.x;
    int64_t row = grid_row();
    if (row >= f.rows)
        return;
    if (OUT == kOutNvfp4Tiled && (f.rows & 255) == 0) {
        const int64_t x = row & 7, k = row >> 3;
        const int64_t g = x + 8 * (k >> 5), m = k & 31;
        row = (g >> 2) * 128 + 32 * (m >> 3) + 8 * (g & 3) + (m & 7);
    }
    const int dim = f.dim;
    const int nvec = dim >> 3;
    const bool stream_ab = f.ab_stride != 0;
    const uint16_t* xr = f.x + row * dim;
    const uint16_t* ar = NIN > 1 ? f.a + row * f.ab_stride : nullptr;
    const uint16_t* br = NIN > 2 ? f.b + row * f.ab_stride : nullptr;
    uint4 xv[VPT], av[VPT], bv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(xr, v * T + t, nvec, v == VPT - 1);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        if (NIN > 1)
            av[v] = stream_ab ? ld_row<true>(ar, v * T + t, nvec, v == VPT - 1)
                              : ld_row<false>(ar, v * T + t, nvec, v == VPT - 1);
        if (NIN > 2)
            bv[v] = stream_ab ? ld_row<true>(br, v * T + t, nvec, v == VPT - 1)
                              : ld_row<false>(br, v * T + t, nvec, v == VPT - 1);
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (v == VPT - 1 && i >= nvec)
            continue;
        uint4 w = xv[v];
        if (NIN > 1) {
            w.x ^= av[v].x; w.y ^= av[v].y; w.z ^= av[v].z; w.w ^= av[v].w;
        }
        if (NIN > 2) {
            w.x ^= bv[v].x; w.y ^= bv[v].y; w.z ^= bv[v].z; w.w ^= bv[v].w;
        }
        if (OUT == kOutBf16) {
            st_stream(reinterpret_cast<uint16_t*>(f.out) + row * dim + (int64_t)i * 8, w);
        } else if (OUT == kOutFp8 || OUT == kOutMxfp8) {
            st_stream(f.out + row * dim + (int64_t)i * 8, make_uint2(w.x ^ w.y, w.z ^ w.w));
            if (OUT == kOutMxfp8 && (i & 3) == 0)
                f.scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)w.x;
        } else {
            st_stream(f.out + row * (dim >> 1) + (int64_t)i * 4, w.x ^ w.y ^ w.z ^ w.w);
            if (OUT == kOutNvfp4 && (i & 1) == 0)
                f.scales[row * (dim >> 4) + (i >> 1)] = (uint8_t)w.x;
            if (OUT == kOutNvfp4Tiled && (i & 1) == 0)
                f.scales[tiled_offset(row, i >> 1, dim >> 4)] = (uint8_t)w.x;
            if (OUT == kOutMxfp4 && (i & 3) == 0)
                f.scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)w.x;
        }
    }
}

template <int OUT, int NIN>
hipError_t launch_floor_rows(const FloorRowArgs& f, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(f.rows);
#define ALNP_LAUNCH(V, W) hipLaunchKernelGGL((k_floor_rows<V, W, OUT, NIN>), grid, dim3(W * 64), 0, s, f)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_floor_nin(const FloorRowArgs& f, int nin, RowShape rs, hipStream_t s)
{
    switch (nin) {
    case 1: return launch_floor_rows<OUT, 1>(f, rs, s);
    case 2: return launch_floor_rows<OUT, 2>(f, rs, s);
    default: return launch_floor_rows<OUT, 3>(f, rs, s);
    }
}

constexpr int kTokensPerThread = 4;

struct FloorMod6Args {
    const float* params;  // (tokens, 6, dim)
    int64_t tokens;
    int dim;
    uint16_t* out[6];
};

// The six-way producer's mapping (a wave per 512 consecutive floats of a
// token's span, two contiguous 1 KiB loads per token, 4 tokens, every load
// issued before the first store, lane pairs storing 16 bytes each after one
// DPP swap); the output is the upper half of each fp32 (truncation) instead
// of the rounded sum.
__global__ __launch_bounds__(256) void k_floor_mod6(FloorMod6Args a)
{
    const int span = 6 * a.dim;
    const int blk = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 512;
    if (blk >= span)
        return;  // whole wave
    const int lane = threadIdx.x & 63;
    int e[2], k[2];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int eh = blk + 256 * h + 4 * lane;
        ok[h] = eh < span;
        e[h] = ok[h] ? eh : 0;
        k[h] = (e[h] >= a.dim) + (e[h] >= 2 * a.dim) + (e[h] >= 3 * a.dim) + (e[h] >= 4 * a.dim) +
               (e[h] >= 5 * a.dim);
    }
    const int64_t t0 = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * kTokensPerThread;
    uint4 p[kTokensPerThread][2];
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
        const int64_t t = t0 + u < a.tokens ? t0 + u : a.tokens - 1;
        const float* pt = a.params + t * span;
        p[u][0] = ld_stream(pt + e[0]);
        p[u][1] = ld_stream(pt + e[1]);
    }
    const bool odd = lane & 1;
    const int hs = odd ? 1 : 0;
    uint16_t* out = a.out[0];
#pragma unroll
    for (int c = 1; c < 6; ++c)
        out = k[hs] == c ? a.out[c] : out;
    const int js = (odd ? e[1] - 4 : e[0]) - k[hs] * a.dim;
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
        const int64_t t = t0 + u;
        if (t >= a.tokens)
            break;
        uint2 o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            o[h].x = (p[u][h].x >> 16) | (p[u][h].y & 0xFFFF0000u);
            o[h].y = (p[u][h].z >> 16) | (p[u][h].w & 0xFFFF0000u);
        }
        const uint2 snd = odd ? o[0] : o[1];
        const uint32_t r0 = __builtin_amdgcn_mov_dpp(snd.x, 0xB1, 0xF, 0xF, false);
        const uint32_t r1 = __builtin_amdgcn_mov_dpp(snd.y, 0xB1, 0xF, 0xF, false);
        if (ok[hs])
            st_stream(out + t * a.dim + js, odd ? make_uint4(r0, r1, o[1].x, o[1].y)
                                                : make_uint4(o[0].x, o[0].y, r0, r1));
    }
}

// Plain device-to-device copy, the practical ceiling for a stream of
// a given size: each thread moves kCopyVecs 16-byte vectors, 256 threads
// apart (every load instruction of a wave covers 1 KiB), with the same
// non-temporal loads and stores as the producers.
constexpr int kCopyVecs = 4;

__global__ __launch_bounds__(256) void k_floor_copy(const uint4* src, uint4* dst, int64_t nvec)
{
    const int64_t base = (int64_t)blockIdx.x * (256 * kCopyVecs) + threadIdx.x;
    uint4 v[kCopyVecs];
#pragma unroll
    for (int k = 0; k < kCopyVecs; ++k) {
        const int64_t i = base + k * 256;
        v[k] = i < nvec ? ld_stream(src + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kCopyVecs; ++k) {
        const int64_t i = base + k * 256;
        if (i < nvec)
            st_stream(dst + i, v[k]);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace alnp

using namespace alnp;

// Memory-only row kernel in a row producer's launch shape.
//   x: (rows, dim) bf16, streamed.  a, b: optional bf16 operand rows (nullptr
//   for none; b only with a); row r of a starts at a + r * ab_stride elements
//   (ab_stride 0: one (dim,) vector shared by every row, read through cache).
//   out_kind: 0 = 1 B/element; 1 = NVFP4 (dim/2 code bytes per row, scales
//   (rows, dim/16)); 2 = bf16 (rows, dim); 3 = MXFP8 (1 B/element, scales
//   (rows, dim/32)); 4 = MXFP4 (dim/2 code bytes, scales (rows, dim/32));
//   5 = NVFP4 with scales in the 128x4 tiled layout (dim a multiple of 64),
//   rows in the tiled FP4 producers' order.
// Returns 0, or -1 for a shape or pointer the row kernels do not take (dim
// not a multiple of 32, rows longer than the register-resident row shapes,
// unaligned pointers), -2 for an unknown out_kind, -6 for a launch failure.
static int floor_rows(const uint16_t* x, const uint16_t* a, const uint16_t* b, int64_t ab_stride,
                      int64_t rows, int dim, int out_kind, void* out, uint8_t* scales,
                      RowShape rs, hipStream_t stream);

extern "C" int alnp_floor_rows(const uint16_t* x, const uint16_t* a, const uint16_t* b,
                               int64_t ab_stride, int64_t rows, int dim, int out_kind, void* out,
                               uint8_t* scales, hipStream_t stream)
{
    return floor_rows(x, a, b, ab_stride, rows, dim, out_kind, out, scales,
                      dim > 0 ? row_shape(dim) : RowShape{0, 0}, stream);
}

// The same memory-only row kernel in a row shape given by the caller (waves
// per row: 1, 2, 4 or 8; 16-byte vectors per thread: 1..8), for comparing
// access patterns at one size.  The shape must cover the row, with only each
// thread's last vector slot allowed past its end: waves * 64 * vpt >= dim / 8
// and (vpt - 1) * waves * 64 <= dim / 8.  Same arguments and returns as
// alnp_floor_rows; -1 also for a shape that breaks these rules.
extern "C" int alnp_floor_rows_shape(const uint16_t* x, const uint16_t* a, const uint16_t* b,
                                     int64_t ab_stride, int64_t rows, int dim, int out_kind,
                                     void* out, uint8_t* scales, int waves, int vpt,
                                     hipStream_t stream)
{
    if (waves != 1 && waves != 2 && waves != 4 && waves != 8)
        return -1;
    if (vpt < 1 || vpt > 8 || dim <= 0 || dim % 32 != 0)
        return -1;
    const int nvec = dim / 8;
    if (waves * 64 * vpt < nvec || (vpt - 1) * waves * 64 > nvec)
        return -1;
    return floor_rows(x, a, b, ab_stride, rows, dim, out_kind, out, scales,
                      RowShape{waves * 64, vpt}, stream);
}

static int floor_rows(const uint16_t* x, const uint16_t* a, const uint16_t* b, int64_t ab_stride,
                      int64_t rows, int dim, int out_kind, void* out, uint8_t* scales,
                      RowShape rs, hipStream_t stream)
{
    if (rows <= 0)
        return 0;
    if (!x || !out || dim <= 0 || dim % 32 != 0 || (b && !a) || ab_stride < 0)
        return -1;
    if (!aligned16(x) || !aligned16(out) || (a && !aligned16(a)) || (b && !aligned16(b)))
        return -1;
    const bool want_scales = out_kind == kOutNvfp4 || out_kind == kOutMxfp8 ||
                             out_kind == kOutMxfp4 || out_kind == kOutNvfp4Tiled;
    if (want_scales && !scales)
        return -1;
    if (rs.vpt == 0)
        return -1;
    FloorRowArgs f{x, a, b, ab_stride, rows, dim, static_cast<uint8_t*>(out), scales};
    const int nin = b ? 3 : a ? 2 : 1;
    hipError_t e;
    switch (out_kind) {
    case kOutFp8: e = launch_floor_nin<kOutFp8>(f, nin, rs, stream); break;
    case kOutNvfp4: e = launch_floor_nin<kOutNvfp4>(f, nin, rs, stream); break;
    case kOutBf16: e = launch_floor_nin<kOutBf16>(f, nin, rs, stream); break;
    case kOutMxfp8: e = launch_floor_nin<kOutMxfp8>(f, nin, rs, stream); break;
    case kOutMxfp4: e = launch_floor_nin<kOutMxfp4>(f, nin, rs, stream); break;
    case kOutNvfp4Tiled:
        if (dim % 64 != 0)
            return -1;  // whole tiles of scale columns only
        e = launch_floor_nin<kOutNvfp4Tiled>(f, nin, rs, stream);
        break;
    default: return -2;
    }
    return e == hipSuccess ? 0 : -6;
}

// Memory-only six-way kernel: params (tokens, 6, dim) fp32 -> six (tokens,
// dim) bf16 outputs, the six-way producer's grid.  dim a multiple of 8,
// 16-byte aligned pointers.  Returns 0, -1 (shape, pointer) or -6.
extern "C" int alnp_floor_modulation6(const float* params, int64_t tokens, int dim,
                                      uint16_t* const* out, hipStream_t stream)
{
    if (tokens <= 0)
        return 0;
    if (!params || !out || dim <= 0 || dim % 8 != 0 || !aligned16(params))
        return -1;
    FloorMod6Args a{params, tokens, dim, {}};
    for (int k = 0; k < 6; ++k) {
        if (!out[k] || !aligned16(out[k]))
            return -1;
        a.out[k] = out[k];
    }
    const int64_t waves = (6 * (int64_t)dim + 511) / 512;
    const int64_t groups = (tokens + kTokensPerThread - 1) / kTokensPerThread;
    const int64_t gy = groups < 65535 ? groups : 65535;
    const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)gy, (unsigned)((groups + gy - 1) / gy));
    hipLaunchKernelGGL(k_floor_mod6, grid, dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Plain copy of nbytes from src to dst (device pointers, 16-byte aligned,
// nbytes a multiple of 16 and at most 2^40).  Returns 0, -1 (shape,
// pointer) or -6.
extern "C" int alnp_floor_copy(const void* src, void* dst, int64_t nbytes, hipStream_t stream)
{
    if (nbytes == 0)
        return 0;
    if (!src || !dst || nbytes < 0 || nbytes % 16 != 0 || nbytes > (int64_t(1) << 40) ||
        !aligned16(src) || !aligned16(dst))
        return -1;
    const int64_t nvec = nbytes / 16;
    const int64_t per_block = 256 * kCopyVecs;
    const dim3 grid((unsigned)((nvec + per_block - 1) / per_block));
    hipLaunchKernelGGL(k_floor_copy, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), nvec);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
