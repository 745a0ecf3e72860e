// rmsmod.hip -- RMSNorm with segment-selected modulation -> bf16, for gfx950.
//
// RMSNorm with an optional weight, then (n * (scale[seg] + 1)) + shift[seg]
// with every step a bf16 operation (RL-Kernel norm_modulate page; h3 page,
// "Implementation Phases" and "NVFP4 Modulation Producer Fusion",
// "Exactness Contract").
#include "rows.hpp"

namespace alnp {

// One modulated pair: the RMSNorm values of two elements before their bf16
// rounding, their operands, and the bf16 results packed.  Each step is an
// fp32 operation rounded to bf16: n = bf16(n), t = bf16(scale + 1),
// u = bf16(n * t), y = bf16(u + shift).  The intermediate roundings keep
// each value as a float (bf16_round); only y is packed.  The first form
// takes t already computed (bf16 values held exactly in fp32).
__device__ __forceinline__ uint32_t modulate_t_bf16x2(float n0, float n1, float t0, float t1,
                                                      float sh0, float sh1)
{
    const float u0 = bf16_round(bf16_round(n0) * t0);
    const float u1 = bf16_round(bf16_round(n1) * t1);
    return pack_bf16x2(u0 + sh0, u1 + sh1);
}

__device__ __forceinline__ uint32_t modulate_bf16x2(float n0, float n1, float sc0, float sc1,
                                                    float sh0, float sh1)
{
    return modulate_t_bf16x2(n0, n1, bf16_round(sc0 + 1.0f), bf16_round(sc1 + 1.0f), sh0, sh1);
}

// One workgroup per row, the row in registers (same shapes as the FP8
// kernels).  The row's table index is one uniform load; an index outside
// [0, segments) reads table row 0 (in bounds) and writes NaN.  The sum of
// squares is a single reduction: v_dot2_f32_bf16 of each bf16 pair with
// itself, DPP wave sums, one LDS exchange.
template <int VPT, int WAVES, bool W>
__global__ __launch_bounds__(WAVES * 64) void k_rms_mod_rows(RmsArgs a)
{
    __shared__ float red[16];
    constexpr int T = WAVES * 64;
    constexpr int NW = W ? VPT : 1;
    const int t = threadIdx.x;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const int64_t row = grid_row();
    if (row >= a.rows)
        return;  // whole workgroup
    const int32_t sidx = a.seg[row];
    const bool in_range = sidx >= 0 && sidx < a.segments;
    const int64_t srow = in_range ? sidx : 0;

    uint4 xv[VPT], wv[NW], scv[VPT], shv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(a.x + row * dim, v * T + t, nvec, v == VPT - 1);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        if (W)
            wv[v] = ld_row<false>(a.weight, v * T + t, nvec, v == VPT - 1);
        scv[v] = ld_row<false>(a.scale + srow * dim, v * T + t, nvec, v == VPT - 1);
        shv[v] = ld_row<false>(a.shift + srow * dim, v * T + t, nvec, v == VPT - 1);
    }
    float q = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        q = sumsq_bf16x8(xv[v], q);
    const float rstd = rsqrt_refined(group_sum(q, red, WAVES) * a.inv_dim + a.eps);

    const bool tail_ok = (VPT - 1) * T + t < nvec;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (v == VPT - 1 && !tail_ok)
            continue;
        float f[8], w8[8], sc[8], sh[8];
        unpack8(xv[v], f);
        if (W)
            unpack8(wv[v], w8);
        unpack8(scv[v], sc);
        unpack8(shv[v], sh);
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float n0 = f[2 * k] * rstd, n1 = f[2 * k + 1] * rstd;
            if (W) {
                n0 = n0 * w8[2 * k];
                n1 = n1 * w8[2 * k + 1];
            }
            o[k] = modulate_bf16x2(n0, n1, sc[2 * k], sc[2 * k + 1], sh[2 * k], sh[2 * k + 1]);
            o[k] = in_range ? o[k] : 0x7FC07FC0u;
        }
        st_stream(a.out + row * dim + (int64_t)i * 8, make_uint4(o[0], o[1], o[2], o[3]));
    }
    if (t == 0 && a.row_rstd)
        a.row_rstd[row] = rstd;
}

// Rows [g * SPAN, g * SPAN + SPAN) of workgroup g, one after another, each
// as in k_rms_mod_rows (same arithmetic and reduction order, so the same
// bits).  Consecutive rows mostly share their segment, so the weight and the
// segment's modulation rows are read once per span into registers and read
// again only when the segment changes; re-reading them from L2 for every row
// is what separates the one-row kernel from a plain copy of the activations.
// With the segment's scale row the kernel keeps t = bf16(scale + 1) as fp32
// (exact), computed once per segment instead of once per row.  The rows' x
// is requested into the two halves of a register pair (the second row's with
// the first, further rows' before the current row is reduced); the loop is
// unrolled, so nothing is copied between rows.  The span's table indices come in with one vector load (SPAN <= 64),
// and the two reduction slots alternate so that one row's partials are not
// overwritten before every wave has read them.
template <int VPT, int WAVES, bool W, int SPAN>
__global__ __launch_bounds__(WAVES * 64) void k_rms_mod_span(RmsArgs a)
{
    __shared__ float red[2][16];
    constexpr int T = WAVES * 64;
    constexpr int NW = W ? VPT : 1;
    const int t = threadIdx.x;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const int64_t r0 = grid_row() * SPAN;
    if (r0 >= a.rows)
        return;  // whole workgroup
    const int n = (int)min<int64_t>(SPAN, a.rows - r0);
    const bool tail_ok = (VPT - 1) * T + t < nvec;
    const int lane = t & (kWave - 1);
    const int32_t segv = lane < n ? a.seg[r0 + lane] : 0;

    uint4 xv[2][VPT], wv[NW], shv[VPT];
    float tv[VPT][8];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[0][v] = ld_row<true>(a.x + r0 * dim, v * T + t, nvec, v == VPT - 1);
    // The second row's x too, before anything else: a CU's loads queue
    // behind each other, and loads issued ahead of x hold up the x of its
    // later rows.  37810 x 5376: 140.4 -> 138.5 us (A-B, bit-identical).
    if (SPAN > 1 && n > 1) {
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            xv[1][v] = ld_row<true>(a.x + (r0 + 1) * dim, v * T + t, nvec, v == VPT - 1);
    }
    int64_t cur = -1;  // segment whose rows tv / shv hold
#pragma unroll
    for (int k = 0; k < SPAN; ++k) {
        if (k >= n)
            break;  // whole workgroup
        const int64_t row = r0 + k;
        const int32_t sidx = __builtin_amdgcn_readlane(segv, k);
        const bool in_range = sidx >= 0 && sidx < a.segments;
        const int64_t srow = in_range ? sidx : 0;
        const uint4(&x)[VPT] = xv[k & 1];
        if (k + 1 < n && k + 1 >= 2) {
#pragma unroll
            for (int v = 0; v < VPT; ++v)
                xv[(k + 1) & 1][v] = ld_row<true>(a.x + (row + 1) * dim, v * T + t, nvec, v == VPT - 1);
        }
        float q = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            q = sumsq_bf16x8(x[v], q);
        // The weight and the segment's rows (L2 hits) are requested once
        // this row's x has landed (its sum of squares is formed), not with
        // x: loads a CU issues ahead of its later rows' x hold those up in
        // its load queue, and these arrive while the sum is exchanged.
        // 37810 x 5376: 138.3 -> 134.3 us (A-B, bit-identical).
        const bool fresh = srow != cur;
        uint4 scv[VPT];
        if (k == 0 || fresh) {
            asm volatile("" ::"v"(q));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (W && k == 0) {
#pragma unroll
            for (int v = 0; v < VPT; ++v)
                wv[v] = ld_row<false>(a.weight, v * T + t, nvec, v == VPT - 1);
        }
        if (fresh) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                scv[v] = ld_row<false>(a.scale + srow * dim, v * T + t, nvec, v == VPT - 1);
                shv[v] = ld_row<false>(a.shift + srow * dim, v * T + t, nvec, v == VPT - 1);
            }
        }
        const float rstd = rsqrt_refined(group_sum(q, red[k & 1], WAVES) * a.inv_dim + a.eps);
        if (fresh) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                float sc[8];
                unpack8(scv[v], sc);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    tv[v][e] = bf16_round(sc[e] + 1.0f);
            }
            cur = srow;
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = v * T + t;
            if (v == VPT - 1 && !tail_ok)
                continue;
            float f[8], w8[8], sh[8];
            unpack8(x[v], f);
            if (W)
                unpack8(wv[v], w8);
            unpack8(shv[v], sh);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float n0 = f[2 * e] * rstd, n1 = f[2 * e + 1] * rstd;
                if (W) {
                    n0 = n0 * w8[2 * e];
                    n1 = n1 * w8[2 * e + 1];
                }
                o[e] = modulate_t_bf16x2(n0, n1, tv[v][2 * e], tv[v][2 * e + 1], sh[2 * e],
                                         sh[2 * e + 1]);
                o[e] = in_range ? o[e] : 0x7FC07FC0u;
            }
            st_stream(a.out + row * dim + (int64_t)i * 8, make_uint4(o[0], o[1], o[2], o[3]));
        }
        if (t == 0 && a.row_rstd)
            a.row_rstd[row] = rstd;
    }
}

__global__ __launch_bounds__(256) void k_rms_mod_block(RmsArgs a)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    const int32_t sidx = a.seg[row];
    const bool in_range = sidx >= 0 && sidx < a.segments;
    const int64_t srow = in_range ? sidx : 0;
    float q = 0.f;
    for (int j = threadIdx.x; j < dim; j += 256) {
        const float v = ldbf(xr, j);
        q = __builtin_fmaf(v, v, q);
    }
    const float rstd = rsqrt_refined(block_sum(q, lds4) * a.inv_dim + a.eps);
    for (int j = threadIdx.x; j < dim; j += 256) {
        float n = ldbf(xr, j) * rstd;
        if (a.weight)
            n = n * ldbf(a.weight, j);
        const uint32_t y = modulate_bf16x2(n, 0.f, ldbf(a.scale, srow * dim + j), 0.f,
                                           ldbf(a.shift, srow * dim + j), 0.f);
        a.out[row * dim + j] = in_range ? (uint16_t)(y & 0xFFFFu) : (uint16_t)0x7FC0;
    }
    if (threadIdx.x == 0 && a.row_rstd)
        a.row_rstd[row] = rstd;
    }
}

// ---- launchers ----------------------------------------------------------------

// Rows per workgroup of k_rms_mod_span, and the row count from which it is
// used: with fewer rows, one row per workgroup keeps more rows in flight (the
// span kernel's registers allow about half the waves per SIMD).  Two rows per
// workgroup was the fastest span on the 37810-row Wan workload (longer spans
// leave too few rows in flight).
constexpr int kRmsSpan = 2;
constexpr int64_t kRmsSpanMinRows = 4096;

template <bool W>
static hipError_t launch_rms_rows(const RmsArgs& a, RowShape rs, hipStream_t s)
{
    if (a.rows >= kRmsSpanMinRows) {
        const dim3 grid = row_grid((a.rows + kRmsSpan - 1) / kRmsSpan);
#define ALNP_LAUNCH(V, WV) \
    hipLaunchKernelGGL((k_rms_mod_span<V, WV, W, kRmsSpan>), grid, dim3(WV * 64), 0, s, a)
        ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        return hipGetLastError();
    }
    const dim3 grid = row_grid(a.rows);
#define ALNP_LAUNCH(V, WV) hipLaunchKernelGGL((k_rms_mod_rows<V, WV, W>), grid, dim3(WV * 64), 0, s, a)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_rms_modulate(const RmsArgs& args, bool fast, hipStream_t s)
{
    RmsArgs a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (rs.vpt > 0)
        return a.weight ? launch_rms_rows<true>(a, rs, s) : launch_rms_rows<false>(a, rs, s);
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_rms_mod_block, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace alnp
