// rows.hpp -- pieces shared by the row producers (producers.hip, fp4.hip,
// rmsmod.hip): vector loads with a tail check, row statistics, the
// workgroup-per-row fallback's reductions, launch geometry and the macros that
// dispatch a row shape to its kernel instantiation.
//
// Kernel design (MI355X): the problem is a pure stream (3-7 bytes moved per
// element, ~15 flops), so the kernels are built for HBM, not MFMA.
//  - Fast path: one workgroup per row, 1, 2, 4 or 8 waves (a template
//    parameter, so launch bounds and indexing are compile-time), each thread
//    holding VPT 16-byte vectors of the row (vector i = v * threads + t), so every load
//    instruction of a wave covers 1 KiB of contiguous memory.  For dim 3072:
//    two waves, three vectors per thread.  The row stays in registers: x is
//    requested up front, operands shared by every row with it, and streamed
//    per-row operands once the row statistics are known (their bytes then
//    arrive while the statistics run); mean and variance are two passes
//    over registers with DPP wave reductions and one LDS exchange between
//    the waves.  Spreading a row over
//    several waves keeps the serial arithmetic each wave does after its data
//    arrives short, which is what bounds the end of the kernel.  Streamed
//    operands use non-temporal loads and the outputs non-temporal stores.
//  - Fallback (dim not a multiple of 8, rows longer than 32768, or operands
//    not 16-byte aligned): one 256-thread workgroup per row, element loops.
//    Same arithmetic.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace alnp {

// ---- fast path: one workgroup per row, row held in registers ---------------

// Vector i of a row (eight elements), or zeros past the row end.  The row
// shapes put every vector slot but a thread's last inside the row, so only
// the last (`tail`, a constant once the slot loop is unrolled) is checked.
template <bool STREAM>
__device__ __forceinline__ uint4 ld_row(const uint16_t* row, int i, int nvec, bool tail)
{
    if (tail && i >= nvec)
        return make_uint4(0, 0, 0, 0);
    return STREAM ? ld_stream(row + 8 * i) : ld_keep(row + 8 * i);
}

// Row statistics from a thread's VPT register vectors (vector v of thread t is
// row vector v * nthreads + t; only the last slot can lie past the row end,
// where it holds zeros and `tail_ok` is false).  Two passes over registers:
// the sum (v_dot2_f32_bf16 against (1, 1)), then the squared deviations from
// the mean.  mean = sum * (1/dim), var = sum_sq * (1/dim), rstd = 1/sqrt(var
// + eps), all fp32.  The deviations x - mean are returned in d for the
// caller's pass over the row.  `reduce` sums a value over the row's waves
// and takes the slot index (0 or 1) of its LDS partials.  row_mean and
// row_rstd are the two passes on their own, for callers that issue loads
// between them; row_stats runs both.  thread_sum and thread_sumsq are a
// thread's share of each pass before the reduction, for callers that also
// work between a share and its reduction.
template <int VPT>
__device__ __forceinline__ float thread_sum(const uint4 (&xv)[VPT])
{
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        s = sum_bf16x8(xv[v], s);
    return s;
}

template <int VPT>
__device__ __forceinline__ float thread_sumsq(const uint4 (&xv)[VPT], bool tail_ok, float mean,
                                              float (&d)[VPT][8])
{
    float q = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        float f[8];
        unpack8(xv[v], f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            d[v][e] = f[e] - mean;
        if (v < VPT - 1 || tail_ok) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                q = __builtin_fmaf(d[v][e], d[v][e], q);
        }
    }
    return q;
}

template <int VPT, typename Reduce>
__device__ __forceinline__ float row_mean(const uint4 (&xv)[VPT], float inv_dim, Reduce reduce)
{
    return reduce(thread_sum<VPT>(xv), 0) * inv_dim;
}

template <int VPT, typename Reduce>
__device__ __forceinline__ float row_rstd(const uint4 (&xv)[VPT], bool tail_ok, float mean,
                                          float inv_dim, float eps, Reduce reduce,
                                          float (&d)[VPT][8])
{
    const float var = reduce(thread_sumsq<VPT>(xv, tail_ok, mean, d), 1) * inv_dim;
    return rsqrt_refined(var + eps);
}

template <int VPT, typename Reduce>
__device__ __forceinline__ void row_stats(const uint4 (&xv)[VPT], bool tail_ok, float inv_dim,
                                          float eps, Reduce reduce, float (&d)[VPT][8],
                                          float& mean, float& rstd)
{
    mean = row_mean<VPT>(xv, inv_dim, reduce);
    rstd = row_rstd<VPT>(xv, tail_ok, mean, inv_dim, eps, reduce, d);
}

// Row index of a workgroup in the 2-D grid (x fastest); the grid can hold
// more workgroups than rows.
__device__ __forceinline__ int64_t grid_row() { return (int64_t)blockIdx.y * gridDim.x + blockIdx.x; }

// Eight e4m3 operand codes of vector i of a (dim,) byte vector, or zeros.
__device__ __forceinline__ uint2 ld_fp8x8(const uint8_t* p, int i, int nvec, bool tail)
{
    if (tail && i >= nvec)
        return make_uint2(0, 0);
    return *reinterpret_cast<const uint2*>(p + 8 * i);
}

// ---- fallback: one workgroup per row ----------------------------------------

// Sum over the 256 threads of a workgroup, same bits in every thread.
__device__ __forceinline__ float block_sum(float v, float* lds4)
{
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0)
        lds4[threadIdx.x >> 6] = v;
    __syncthreads();
    const float r = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float ldbf(const uint16_t* p, int64_t i)
{
    return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ void block_row_stats(const uint16_t* xr, int dim, float inv_dim,
                                                float eps, float* lds4, float& mean,
                                                float& rstd)
{
    float s = 0.f;
    for (int j = threadIdx.x; j < dim; j += 256)
        s += ldbf(xr, j);
    mean = block_sum(s, lds4) * inv_dim;
    float q = 0.f;
    for (int j = threadIdx.x; j < dim; j += 256) {
        const float d = ldbf(xr, j) - mean;
        q = __builtin_fmaf(d, d, q);
    }
    const float var = block_sum(q, lds4) * inv_dim;
    rstd = rsqrt_refined(var + eps);
}

// ---- launch geometry -------------------------------------------------------

// Grid cap for the workgroup-per-row fallback, whose rows loop.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

// One workgroup per row on a 2-D grid: x up to 65535 rows, y the rest.
inline dim3 row_grid(int64_t rows)
{
    const int64_t gx = std::min<int64_t>(rows, 65535);
    return dim3((unsigned)gx, (unsigned)((rows + gx - 1) / gx));
}

#define ALNP_VPT_CASES(WAVES, LAUNCH)                                               \
    switch (rs.vpt) {                                                               \
    case 1: LAUNCH(1, WAVES); break;                                                \
    case 2: LAUNCH(2, WAVES); break;                                                \
    case 3: LAUNCH(3, WAVES); break;                                                \
    case 4: LAUNCH(4, WAVES); break;                                                \
    case 5: LAUNCH(5, WAVES); break;                                                \
    case 6: LAUNCH(6, WAVES); break;                                                \
    case 7: LAUNCH(7, WAVES); break;                                                \
    case 8: LAUNCH(8, WAVES); break;                                                \
    default: return hipErrorInvalidValue;                                           \
    }

#define ALNP_SHAPE_CASES(LAUNCH)                                                    \
    switch (rs.threads) {                                                           \
    case 64: ALNP_VPT_CASES(1, LAUNCH) break;                                       \
    case 128: ALNP_VPT_CASES(2, LAUNCH) break;                                      \
    case 256: ALNP_VPT_CASES(4, LAUNCH) break;                                      \
    case 512: ALNP_VPT_CASES(8, LAUNCH) break;                                      \
    default: return hipErrorInvalidValue;                                           \
    }

}  // namespace alnp
