// producers.hip -- LayerNorm / adaptive-LayerNorm producers for gfx950.
//
// What is computed (per row of a bf16 (rows, dim) activation) follows the
// "adaptive-layernorm-producers" README ("Available Functions", "Tensor
// Contract"): LayerNorm without affine weights, DiT modulation
// (xhat * (1 + scale)) + shift (operation order from the h3-blackwell-runtime
// page, "NVFP4 Modulation Producer Fusion", "Exactness Contract"), then
// static-scale e4m3 or block-16 e2m1 quantization.  The same row kernels
// also write the MX block formats (E8M0 scale per 32 elements, OCP MX v1.0),
// and a sibling kernel computes RMSNorm with segment-selected modulation in
// bf16 operations (RL-Kernel norm_modulate page; h3 page, "Implementation
// Phases").
//
// Kernel design (MI355X): the problem is a pure stream (3-7 bytes moved per
// element, ~15 flops), so the kernels are built for HBM, not MFMA.
//  - Fast path: one workgroup per row, 1, 2, 4 or 8 waves (a template
//    parameter, so launch bounds and indexing are compile-time), each thread
//    holding VPT
//    16-byte vectors of the row (vector i = v * threads + t), so every load
//    instruction of a wave covers 1 KiB of contiguous memory.  For dim 3072:
//    two waves, three vectors per thread.  The row stays in registers: x,
//    then the per-token operands, are requested up front so their latency
//    overlaps; mean and variance are two passes over registers with DPP wave
//    reductions and one LDS exchange between the waves.  Spreading a row over
//    several waves keeps the serial arithmetic each wave does after its data
//    arrives short, which is what bounds the end of the kernel.  Streamed
//    operands use non-temporal loads and the outputs non-temporal stores.
//  - Fallback (dim not a multiple of 8, rows longer than 32768, or operands
//    not 16-byte aligned): one 256-thread workgroup per row, element loops.
//    Same arithmetic.
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
// and takes the slot index (0 or 1) of its LDS partials.
template <int VPT, typename Reduce>
__device__ __forceinline__ void row_stats(const uint4 (&xv)[VPT], bool tail_ok, float inv_dim,
                                          float eps, Reduce reduce, float (&d)[VPT][8],
                                          float& mean, float& rstd)
{
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        s = sum_bf16x8(xv[v], s);
    mean = reduce(s, 0) * inv_dim;
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
    const float var = reduce(q, 1) * inv_dim;
    rstd = rsqrt_refined(var + eps);
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

// MX: MXFP8 output, one E8M0 scale per 32 elements (the four vectors of a
// lane quad) in place of the static act_scale.
template <int VPT, int WAVES, int FORM, bool MX = false>
__global__ __launch_bounds__(WAVES * 64) void k_adaln_fp8_rows(Fp8Args a)
{
    __shared__ float red[32];  // two sets of per-wave partials
    constexpr int T = WAVES * 64;
    // Register arrays per operand kind (size 1 where the form has none).
    constexpr bool kBf16Ops = FORM == kBcast || FORM == kPtok || FORM == kTable || FORM == kAwq;
    constexpr int NB = kBf16Ops ? VPT : 1;
    // Table rows are held from the start for up to 4 vectors per thread; with
    // more, holding them (16 floats per vector) would spill, so each vector's
    // table values are read in the output pass instead.
    constexpr bool kTableEarly = FORM == kTable && VPT <= 4;
    constexpr int NT = kTableEarly ? 2 * VPT : 1;
    constexpr int N8 = FORM == kModFp8 ? VPT : 1;
    constexpr int NI = FORM == kAwq ? VPT : 1;
    const int t = threadIdx.x;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const float inv = MX ? 0.f : 1.0f / *a.act_scale;
    const int64_t row = grid_row();
    if (row >= a.rows)
        return;  // whole workgroup
    {
        uint4 xv[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v)
            xv[v] = ld_row<true>(a.x + row * dim, v * T + t, nvec, v == VPT - 1);

        // Modulation operands, requested before the reductions.  Per-token
        // rows and temb chunks are streamed; (dim,) vectors are shared by
        // every row and kept in cache.
        uint4 scv[NB], shv[NB];
        uint2 sc8[N8], sh8[N8];
        uint4 isv[NI];
        // Table rows (fp32, shared by every row, L2-resident): also requested
        // before the reductions so their latency is not added at the end.
        float4 tsv[NT], thv[NT];
        if (kTableEarly) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                const int i = v * T + t;
                const int j = i < nvec ? 8 * i : 0;
                const float4* ts = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim + j);
                const float4* th = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim + j);
                tsv[2 * v] = ts[0];
                tsv[2 * v + 1] = ts[1];
                thv[2 * v] = th[0];
                thv[2 * v + 1] = th[1];
            }
        }
        if (FORM == kBcast || FORM == kAwq) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                scv[v] = ld_row<false>(a.scale, v * T + t, nvec, v == VPT - 1);
                shv[v] = ld_row<false>(a.shift, v * T + t, nvec, v == VPT - 1);
                if (FORM == kAwq)
                    isv[v] = ld_row<false>(a.inv_s, v * T + t, nvec, v == VPT - 1);
            }
        } else if (FORM == kPtok || FORM == kTable) {
            const uint16_t* scr = FORM == kPtok ? a.scale + row * dim
                                                : a.temb + (row * a.chunks + a.scale_idx) * dim;
            const uint16_t* shr = FORM == kPtok ? a.shift + row * dim
                                                : a.temb + (row * a.chunks + a.shift_idx) * dim;
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                scv[v] = ld_row<true>(scr, v * T + t, nvec, v == VPT - 1);
                shv[v] = ld_row<true>(shr, v * T + t, nvec, v == VPT - 1);
            }
        } else if (FORM == kModFp8) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                sc8[v] = ld_fp8x8(a.scale_fp8, v * T + t, nvec, v == VPT - 1);
                sh8[v] = ld_fp8x8(a.shift_fp8, v * T + t, nvec, v == VPT - 1);
            }
        }
        const float sdeq = FORM == kModFp8 ? *a.scale_deq : 0.f;
        const float hdeq = FORM == kModFp8 ? *a.shift_deq : 0.f;

        const bool tail_ok = (VPT - 1) * T + t < nvec;
        float mean, rstd, d[VPT][8];
        row_stats<VPT>(xv, tail_ok, a.inv_dim, a.eps,
                       [&](float v, int k) { return group_sum(v, red + 16 * k, WAVES); }, d, mean,
                       rstd);

#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = v * T + t;
            if (v == VPT - 1 && !tail_ok)
                continue;
            float sc[8], sh[8];
            if (FORM == kNone) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = 0.f;
                    sh[e] = 0.f;
                }
            } else if (FORM == kModFp8) {
                // Dequantize: e4m3 value times its fp32 scalar, one rounding.
                unpack_e4m3x8(sc8[v], sc);
                unpack_e4m3x8(sh8[v], sh);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = sc[e] * sdeq;
                    sh[e] = sh[e] * hdeq;
                }
            } else {
                unpack8(scv[v], sc);
                unpack8(shv[v], sh);
                if (FORM == kTable) {
                    float4 t0, t1, h0, h1;
                    if (kTableEarly) {
                        t0 = tsv[2 * v];
                        t1 = tsv[2 * v + 1];
                        h0 = thv[2 * v];
                        h1 = thv[2 * v + 1];
                    } else {
                        const float4* ts = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim + 8 * i);
                        const float4* th = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim + 8 * i);
                        t0 = ts[0];
                        t1 = ts[1];
                        h0 = th[0];
                        h1 = th[1];
                    }
                    const float ts[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
                    const float th[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sc[e] = sc[e] + ts[e];
                        sh[e] = sh[e] + th[e];
                    }
                }
            }
            float is[8];
            if (FORM == kAwq)
                unpack8(isv[v], is);
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xhat = d[v][e] * rstd;
                float y = (xhat * (1.0f + sc[e])) + sh[e];
                if (FORM == kAwq)
                    y = y * is[e];  // per-channel smoothing before the static scale
                q[e] = MX ? y : y * inv;
            }
            if (!MX)
                sat448x8(q);
            if (MX) {
                // Block scale 2^E from the quad's maximum; elements y * 2^-E
                // (exact), saturated at 448.  The quad's lanes store the same
                // scale byte.
                const int E = mx_scale_exp(quad_max(absmax8(q)), 8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    q[e] = sat448(__builtin_amdgcn_ldexpf(q[e], -E));
                a.mx_scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
            }
            st_stream(a.out + row * dim + (int64_t)i * 8,
                      make_uint2(pack_e4m3x4(q[0], q[1], q[2], q[3]),
                                 pack_e4m3x4(q[4], q[5], q[6], q[7])));
        }
        if (t == 0) {
            if (a.row_mean) a.row_mean[row] = mean;
            if (a.row_rstd) a.row_rstd[row] = rstd;
        }
    }
}

// Table form with the two selected fp32 table rows staged in LDS and shared by
// the two rows of a workgroup.  Holding the table in registers costs ~50
// VGPRs per thread, which leaves room for only 2048 of the 2520 rows of the
// Wan workload on the chip at once; from LDS the kernel keeps the per-token
// kernel's register budget and reads each table element from L2 once per
// two rows instead of once per row.  The table loads (L2 hits) are issued
// before the row loads so that the LDS fill does not wait behind them.
constexpr int kTableRows = 2;     // rows per workgroup
constexpr int kTableMaxDim = 8192; // 2 table rows * 8192 * 4 B = 64 KiB of LDS

template <int VPT, int WAVES, int R = kTableRows, bool MX = false>
__global__ __launch_bounds__(R * WAVES * 64) void k_adaln_fp8_table_lds(Fp8Args a)
{
    extern __shared__ float4 tab[];   // [0, dim/4): scale row, [dim/4, dim/2): shift row
    __shared__ float red[2][R * WAVES];
    constexpr int T = WAVES * 64;      // threads per row
    constexpr int NT = R * T;          // threads per workgroup
    const int tid = threadIdx.x;
    const int rr = tid / T, t = tid % T;
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const int n4 = dim >> 2;
    const float inv = MX ? 0.f : 1.0f / *a.act_scale;
    const int64_t row = grid_row() * R + rr;
    const bool valid = row < a.rows;

    // Table rows first: up to 8 float4 per thread in flight, the rest (only
    // for dims above 4 * 2 * NT ... 8192) loaded after the row operands.
    const float4* tsrc = reinterpret_cast<const float4*>(a.table + (int64_t)a.scale_idx * dim);
    const float4* thsrc = reinterpret_cast<const float4*>(a.table + (int64_t)a.shift_idx * dim);
    constexpr int kFirst = 8;
    float4 tv[kFirst];
#pragma unroll
    for (int k = 0; k < kFirst; ++k) {
        const int idx = tid + k * NT;  // over the 2 * n4 table vectors
        tv[k] = idx < n4 ? tsrc[idx] : idx < 2 * n4 ? thsrc[idx - n4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t lrow = valid ? row : 0;
    const uint16_t* xr = a.x + lrow * dim;
    const uint16_t* scr = a.temb + (lrow * a.chunks + a.scale_idx) * dim;
    const uint16_t* shr = a.temb + (lrow * a.chunks + a.shift_idx) * dim;
    // A workgroup's second row past the end (odd row counts) computes on row 0
    // and stores nothing.
    uint4 xv[VPT], scv[VPT], shv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(xr, v * T + t, nvec, v == VPT - 1);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        scv[v] = ld_row<true>(scr, v * T + t, nvec, v == VPT - 1);
        shv[v] = ld_row<true>(shr, v * T + t, nvec, v == VPT - 1);
    }

#pragma unroll
    for (int k = 0; k < kFirst; ++k) {
        const int idx = tid + k * NT;
        if (idx < 2 * n4)
            tab[idx] = tv[k];
    }
    for (int idx = tid + kFirst * NT; idx < 2 * n4; idx += NT)
        tab[idx] = idx < n4 ? tsrc[idx] : thsrc[idx - n4];

    // Row statistics over the row's WAVES waves (the barriers also publish
    // the LDS table).
    const bool tail_ok = (VPT - 1) * T + t < nvec;
    float mean, rstd, d[VPT][8];
    row_stats<VPT>(xv, tail_ok, a.inv_dim, a.eps,
                   [&](float v, int k) { return subgroup_sum(v, red[k], rr * WAVES, WAVES); }, d,
                   mean, rstd);
    if (!valid)
        return;

#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (v == VPT - 1 && !tail_ok)
            continue;
        float sc[8], sh[8];
        unpack8(scv[v], sc);
        unpack8(shv[v], sh);
        const float4 s0 = tab[2 * i], s1 = tab[2 * i + 1];
        const float4 h0 = tab[n4 + 2 * i], h1 = tab[n4 + 2 * i + 1];
        const float ts[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float th[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        float q8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float scale = sc[e] + ts[e];
            const float shift = sh[e] + th[e];
            const float xhat = d[v][e] * rstd;
            const float y = (xhat * (1.0f + scale)) + shift;
            q8[e] = MX ? y : y * inv;
        }
        if (!MX)
            sat448x8(q8);
        if (MX) {
            // MXFP8: as in k_adaln_fp8_rows (a quad of lanes holds one block).
            const int E = mx_scale_exp(quad_max(absmax8(q8)), 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                q8[e] = sat448(__builtin_amdgcn_ldexpf(q8[e], -E));
            a.mx_scales[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
        }
        st_stream(a.out + row * dim + (int64_t)i * 8,
                  make_uint2(pack_e4m3x4(q8[0], q8[1], q8[2], q8[3]),
                             pack_e4m3x4(q8[4], q8[5], q8[6], q8[7])));
    }
    if (t == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
}

// Byte offset of block scale (r, c) in the 128x4 tiled layout for `cols`
// scales per row: tiles of 128 rows x 4 scales, 512 bytes each, laid out
// tile-row-major; inside a tile, (r mod 32) selects a 16-byte unit, (r div 32)
// mod 4 the 4-byte group in it, c mod 4 the byte.
__device__ __forceinline__ int64_t sf_swizzled_offset(int64_t r, int c, int cols)
{
    const int col_tiles = (cols + 3) >> 2;
    const int64_t tile = (r >> 7) * col_tiles + (c >> 2);
    const int rr = (int)(r & 127);
    return tile * 512 + (rr & 31) * 16 + (rr >> 5) * 4 + (c & 3);
}

// Store the block scale of (row, c); in the tiled layout the writer of a
// row's last scale also zeroes the row's padding columns.
template <bool SWZ>
__device__ __forceinline__ void store_scale(uint8_t* sf, int64_t row, int c, int cols, uint8_t code)
{
    if (!SWZ) {
        sf[row * cols + c] = code;
        return;
    }
    sf[sf_swizzled_offset(row, c, cols)] = code;
    if (c == cols - 1)
        for (int p = cols; p < ((cols + 3) & ~3); ++p)
            sf[sf_swizzled_offset(row, p, cols)] = 0;
}

// 1 / s for every e4m3 code s below 0x7F (0 for code 0), rounded to nearest
// even by the compiler's constant evaluation (IEEE binary32 division).
struct E4m3Recip {
    float v[128];
    constexpr E4m3Recip() : v()
    {
        for (int c = 1; c < 127; ++c) {
            const int e = (c >> 3) & 15, m = c & 7;
            float p = 1.0f;  // 2^e
            for (int k = 0; k < e; ++k)
                p *= 2.0f;
            const float s = e == 0 ? (float)m / 512.0f : (float)(8 + m) * p / 1024.0f;
            v[c] = 1.0f / s;
        }
    }
};
__device__ const E4m3Recip kE4m3Recip{};

// LayerNorm (FORM kNone), broadcast AdaLN (kBcast) or AdaLN with e4m3
// operands and fp32 dequantization scalars (kModFp8) -> FP4: NVFP4 (e4m3
// scale per 16 elements) or, with MX, MXFP4 (E8M0 scale per 32 elements,
// row-major).
template <int VPT, int WAVES, int FORM, bool SWZ, bool MX = false>
__global__ __launch_bounds__(WAVES * 64) void k_fp4_rows(Fp4Args a)
{
    __shared__ float red[32];     // two sets of per-wave partials
    __shared__ float inv_s[128];  // 1 / s for every e4m3 scale code s
    constexpr int T = WAVES * 64;
    constexpr int NM = FORM == kBcast ? VPT : 1;
    constexpr int N8 = FORM == kModFp8 ? VPT : 1;
    const int t = threadIdx.x;
    const int dim = a.dim;
    const int nvec = dim >> 3;  // even, since dim % 16 == 0
    const int cols = dim >> 4;
    const int64_t row = grid_row();
    if (row >= a.rows)
        return;  // whole workgroup
    // The encode factors 1 / s, staged from the compile-time table into LDS
    // (requested here, written once the row loads are in flight).
    const float recip0 = !MX && t < 128 ? kE4m3Recip.v[t] : 0.f;
    const float recip1 = !MX && T == 64 ? kE4m3Recip.v[t + 64] : 0.f;

    uint4 xv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(a.x + row * dim, v * T + t, nvec, v == VPT - 1);
    uint4 scv[NM], shv[NM];
    uint2 sc8[N8], sh8[N8];
    if (FORM == kBcast) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            scv[v] = ld_row<false>(a.scale, v * T + t, nvec, v == VPT - 1);
            shv[v] = ld_row<false>(a.shift, v * T + t, nvec, v == VPT - 1);
        }
    } else if (FORM == kModFp8) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            sc8[v] = ld_fp8x8(a.scale_fp8, v * T + t, nvec, v == VPT - 1);
            sh8[v] = ld_fp8x8(a.shift_fp8, v * T + t, nvec, v == VPT - 1);
        }
    }
    const float sdeq = FORM == kModFp8 ? *a.scale_deq : 0.f;
    const float hdeq = FORM == kModFp8 ? *a.shift_deq : 0.f;
    if (!MX && t < 128)
        inv_s[t] = recip0;
    if (!MX && T == 64)
        inv_s[t + 64] = recip1;

    const bool tail_ok = (VPT - 1) * T + t < nvec;
    float mean, rstd, d[VPT][8];
    row_stats<VPT>(xv, tail_ok, a.inv_dim, a.eps,
                   [&](float v, int k) { return group_sum(v, red + 16 * k, WAVES); }, d, mean,
                   rstd);
    if (WAVES == 1 && !MX)
        __syncthreads();  // inv_s visible (row_stats has no barrier for one wave)

    // Block scale s = e4m3(amax / 6): amax is a bf16 value, and for every
    // finite bf16 amax the product amax * RN(1/6) rounds to the same e4m3
    // code as the correctly rounded quotient (checked exhaustively on the
    // host), so the kernel multiplies.
    const float kSixth = 1.0f / 6.0f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        // The two halves of a 16-element block sit in lanes t and t ^ 1
        // (T is a multiple of 64 and nvec is even, so both lanes of a pair
        // take the same branch).
        const int i = v * T + t;
        if (v == VPT - 1 && !tail_ok)
            continue;
        float b[8], y[8];
        if (FORM != kNone) {
            float sc[8], sh[8];
            if (FORM == kModFp8) {
                // Dequantize: e4m3 value times its fp32 scalar, one rounding.
                unpack_e4m3x8(sc8[v], sc);
                unpack_e4m3x8(sh8[v], sh);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = sc[e] * sdeq;
                    sh[e] = sh[e] * hdeq;
                }
            } else {
                unpack8(scv[v], sc);
                unpack8(shv[v], sh);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xhat = d[v][e] * rstd;
                y[e] = (xhat * (1.0f + sc[e])) + sh[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                y[e] = d[v][e] * rstd;
        }
        if constexpr (MX) {
            // Stage through bf16; the block maximum of the staged values is
            // bf16(max |y|) (rounding is monotone).  gfx950's scaled convert
            // divides the bf16 pairs by the power-of-two scale exactly and
            // rounds to nearest even onto E2M1 (checked for every bf16 value
            // and every exponent).
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
            const float m = bf16_lo(pack_bf16x2(absmax8(y), 0.f));
            const int E = mx_scale_exp(quad_max(m), 2);
            const float xs = __uint_as_float((uint32_t)(E + 127) << 23);
            uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w[0]), xs, 0);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[1]), xs, 1);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[2]), xs, 2);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[3]), xs, 3);
            st_stream(a.packed + row * (dim / 2) + (int64_t)i * 4, word);
            a.sf[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
            continue;
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            // Stage through bf16 (round to nearest even).
            const uint32_t w = pack_bf16x2(y[e], y[e + 1]);
            b[e] = bf16_lo(w);
            b[e + 1] = bf16_hi(w);
        }
        const float amax = pair_max(absmax8(b));
        const uint32_t scode = pack_e4m3x4(fminf(amax * kSixth, 448.0f), 0.f, 0.f, 0.f) & 0xFFu;
        // A zero scale gives zero codes (a select, not a branch: inv_s[0] is
        // 0 and would leave the signs of negative values).
        const float enc = inv_s[scode];
        const uint32_t word = pack_e2m1x8(b[0] * enc, b[1] * enc, b[2] * enc, b[3] * enc,
                                          b[4] * enc, b[5] * enc, b[6] * enc, b[7] * enc);
        st_stream(a.packed + row * (dim / 2) + (int64_t)i * 4, scode != 0 ? word : 0u);
        // Both lanes of the pair hold the block's scale and store the same
        // byte (no lane condition).
        store_scale<SWZ>(a.sf, row, i >> 1, cols, (uint8_t)scode);
    }
    if (t == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
}

// ---- RMSNorm with segment-selected modulation -> bf16 ----------------------

// One modulated pair: the bf16 RMSNorm outputs n of two elements (already
// rounded, packed), their operands, and the bf16 results packed.  Each step
// is an fp32 operation rounded to bf16: t = bf16(scale + 1), u = bf16(n * t),
// y = bf16(u + shift).
__device__ __forceinline__ uint32_t modulate_bf16x2(uint32_t n, float sc0, float sc1, float sh0,
                                                    float sh1)
{
    const uint32_t t = pack_bf16x2(sc0 + 1.0f, sc1 + 1.0f);
    const uint32_t u = pack_bf16x2(bf16_lo(n) * bf16_lo(t), bf16_hi(n) * bf16_hi(t));
    return pack_bf16x2(bf16_lo(u) + sh0, bf16_hi(u) + sh1);
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
            o[k] = modulate_bf16x2(pack_bf16x2(n0, n1), sc[2 * k], sc[2 * k + 1], sh[2 * k],
                                   sh[2 * k + 1]);
            o[k] = in_range ? o[k] : 0x7FC07FC0u;
        }
        st_stream(a.out + row * dim + (int64_t)i * 8, make_uint4(o[0], o[1], o[2], o[3]));
    }
    if (t == 0 && a.row_rstd)
        a.row_rstd[row] = rstd;
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

__global__ __launch_bounds__(256) void k_adaln_fp8_block(Fp8Args a, int form)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    const float inv = 1.0f / *a.act_scale;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int j = threadIdx.x; j < dim; j += 256) {
        float sc = 0.f, sh = 0.f;
        if (form == kBcast) {
            sc = ldbf(a.scale, j);
            sh = ldbf(a.shift, j);
        } else if (form == kPtok) {
            sc = ldbf(a.scale, row * dim + j);
            sh = ldbf(a.shift, row * dim + j);
        } else if (form == kTable) {
            sc = ldbf(a.temb, (row * a.chunks + a.scale_idx) * dim + j) +
                 a.table[(int64_t)a.scale_idx * dim + j];
            sh = ldbf(a.temb, (row * a.chunks + a.shift_idx) * dim + j) +
                 a.table[(int64_t)a.shift_idx * dim + j];
        } else if (form == kModFp8) {
            sc = __builtin_amdgcn_cvt_f32_fp8((int)a.scale_fp8[j], 0) * *a.scale_deq;
            sh = __builtin_amdgcn_cvt_f32_fp8((int)a.shift_fp8[j], 0) * *a.shift_deq;
        } else if (form == kAwq) {
            sc = ldbf(a.scale, j);
            sh = ldbf(a.shift, j);
        }
        const float xhat = (ldbf(xr, j) - mean) * rstd;
        float y = (xhat * (1.0f + sc)) + sh;
        if (form == kAwq)
            y = y * ldbf(a.inv_s, j);
        a.out[row * dim + j] = (uint8_t)(pack_e4m3x4(sat448(y * inv), 0.f, 0.f, 0.f) & 0xFFu);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    }
}

// One thread per 16-element block; modulation by a.form.
__device__ __forceinline__ float fp4_block_y(const Fp4Args& a, const uint16_t* xr, int j,
                                             float mean, float rstd)
{
    const float xhat = (ldbf(xr, j) - mean) * rstd;
    if (a.form == kBcast)
        return (xhat * (1.0f + ldbf(a.scale, j))) + ldbf(a.shift, j);
    if (a.form == kModFp8) {
        const float sc = __builtin_amdgcn_cvt_f32_fp8((int)a.scale_fp8[j], 0) * *a.scale_deq;
        const float sh = __builtin_amdgcn_cvt_f32_fp8((int)a.shift_fp8[j], 0) * *a.shift_deq;
        return (xhat * (1.0f + sc)) + sh;
    }
    return xhat;
}

__global__ __launch_bounds__(256) void k_fp4_block(Fp4Args a)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int k = threadIdx.x; k < dim / 16; k += 256) {
        float b[16];
        float amax = 0.f;
        for (int e = 0; e < 16; e += 2) {
            const int j = 16 * k + e;
            const uint32_t w = pack_bf16x2(fp4_block_y(a, xr, j, mean, rstd),
                                           fp4_block_y(a, xr, j + 1, mean, rstd));
            b[e] = bf16_lo(w);
            b[e + 1] = bf16_hi(w);
            amax = fmaxf(amax, fmaxf(fabsf(b[e]), fabsf(b[e + 1])));
        }
        const float target = fminf(amax / 6.0f, 448.0f);
        const uint32_t scode = pack_e4m3x4(target, 0.f, 0.f, 0.f) & 0xFFu;
        const float s = e4m3_value(scode);
        const float enc = s != 0.f ? 1.0f / s : 0.f;
        for (int e = 0; e < 16; e += 2) {
            uint32_t byte = 0;
            if (s != 0.f)
                byte = e2m1_code(b[e] * enc) | (e2m1_code(b[e + 1] * enc) << 4);
            a.packed[row * (dim / 2) + 8 * k + e / 2] = (uint8_t)byte;
        }
        if (a.sf_layout == kSfSwizzled)
            store_scale<true>(a.sf, row, k, dim / 16, (uint8_t)scode);
        else
            store_scale<false>(a.sf, row, k, dim / 16, (uint8_t)scode);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
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
        const uint32_t y = modulate_bf16x2(pack_bf16x2(n, 0.f), ldbf(a.scale, srow * dim + j), 0.f,
                                           ldbf(a.shift, srow * dim + j), 0.f);
        a.out[row * dim + j] = in_range ? (uint16_t)(y & 0xFFFFu) : (uint16_t)0x7FC0;
    }
    if (threadIdx.x == 0 && a.row_rstd)
        a.row_rstd[row] = rstd;
    }
}

// MX fallbacks: one workgroup per row, one thread per 32-element block.
__global__ __launch_bounds__(256) void k_mxfp8_block(Fp8Args a, int form)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int k = threadIdx.x; k < dim / 32; k += 256) {
        float y[32];
        float amax = 0.f;
        for (int e = 0; e < 32; ++e) {
            const int j = 32 * k + e;
            float sc = 0.f, sh = 0.f;
            if (form == kBcast) {
                sc = ldbf(a.scale, j);
                sh = ldbf(a.shift, j);
            } else if (form == kPtok) {
                sc = ldbf(a.scale, row * dim + j);
                sh = ldbf(a.shift, row * dim + j);
            } else if (form == kTable) {
                sc = ldbf(a.temb, (row * a.chunks + a.scale_idx) * dim + j) +
                     a.table[(int64_t)a.scale_idx * dim + j];
                sh = ldbf(a.temb, (row * a.chunks + a.shift_idx) * dim + j) +
                     a.table[(int64_t)a.shift_idx * dim + j];
            }
            const float xhat = (ldbf(xr, j) - mean) * rstd;
            y[e] = (xhat * (1.0f + sc)) + sh;
            amax = fmaxf(amax, fabsf(y[e]));
        }
        const int E = mx_scale_exp(amax, 8);
        for (int e = 0; e < 32; ++e)
            a.out[row * dim + 32 * k + e] =
                (uint8_t)(pack_e4m3x4(sat448(__builtin_amdgcn_ldexpf(y[e], -E)), 0.f, 0.f, 0.f) & 0xFFu);
        a.mx_scales[row * (dim / 32) + k] = (uint8_t)(E + 127);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    }
}

__global__ __launch_bounds__(256) void k_mxfp4_block(Fp4Args a)
{
    __shared__ float lds4[4];
    const int dim = a.dim;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.inv_dim, a.eps, lds4, mean, rstd);
    for (int k = threadIdx.x; k < dim / 32; k += 256) {
        uint32_t w[16];
        float amax = 0.f;
        for (int e = 0; e < 32; e += 2) {
            const int j = 32 * k + e;
            w[e / 2] = pack_bf16x2(fp4_block_y(a, xr, j, mean, rstd), fp4_block_y(a, xr, j + 1, mean, rstd));
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e / 2])), fabsf(bf16_hi(w[e / 2]))));
        }
        const int E = mx_scale_exp(amax, 2);
        const float xs = __uint_as_float((uint32_t)(E + 127) << 23);
        for (int e = 0; e < 32; e += 8) {
            uint32_t word = 0;
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[e / 2]), xs, 0);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[e / 2 + 1]), xs, 1);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[e / 2 + 2]), xs, 2);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[e / 2 + 3]), xs, 3);
            for (int q = 0; q < 4; ++q)
                a.packed[row * (dim / 2) + 16 * k + e / 2 + q] = (uint8_t)(word >> (8 * q));
        }
        a.sf[row * (dim / 32) + k] = (uint8_t)(E + 127);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
    }
}

// ---- standalone quantizer ---------------------------------------------------

__global__ __launch_bounds__(256) void k_quant_fp8(const float* v, const float* act, int64_t n,
                                                   uint8_t* out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float inv = 1.0f / *act;
    out[i] = (uint8_t)(pack_e4m3x4(sat448(v[i] * inv), 0.f, 0.f, 0.f) & 0xFFu);
}

// ---- launchers ----------------------------------------------------------------

// Grid cap for the workgroup-per-row fallback, whose rows loop.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

RowShape row_shape(int dim)
{
    // Waves per row (1, 2, 4 or 8) and 16-byte vectors per thread (1..8) for
    // a row of dim/8 vectors: the least padding, with 2-4 vectors per thread
    // preferred (fewer waves and barriers than 1, shorter per-wave tails than
    // 5-8), then 3.
    const int nvec = dim / 8;
    RowShape best{0, 0};
    double best_score = 1e30;
    for (int vpt = 1; vpt <= 8; ++vpt) {
        int waves = 1;
        while (waves * 64 * vpt < nvec && waves < 8)
            waves *= 2;
        if (waves * 64 * vpt < nvec || (vpt - 1) * waves * 64 > nvec)
            continue;  // too short, or more than the last slot past the end
        const double waste = double(waves * 64 * vpt - nvec) / nvec;
        const double score = waste + (vpt == 1 ? 0.1 : vpt > 4 ? 0.02 * (vpt - 4) : 0.0) +
                             (vpt == 3 ? -1e-3 : 0.0);
        if (score < best_score) {
            best_score = score;
            best = RowShape{waves * 64, vpt};
        }
    }
    return best;
}

// One workgroup per row on a 2-D grid: x up to 65535 rows, y the rest.
static dim3 row_grid(int64_t rows)
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

template <int FORM>
static hipError_t launch_fp8_rows(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(a.rows);
#define ALNP_LAUNCH(V, W) \
    hipLaunchKernelGGL((k_adaln_fp8_rows<V, W, FORM>), grid, dim3(W * 64), 0, s, a)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

// The LDS table kernel runs rows of at most 4 waves (its caller checks), so
// the 8-wave shapes are not instantiated.
template <int V, int W>
static void launch_table_lds_shape(const Fp8Args& a, dim3 grid, size_t lds, hipStream_t s)
{
    if constexpr (W <= 4)
        hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W>), grid, dim3(kTableRows * W * 64), lds, s, a);
}

static hipError_t launch_fp8_table_lds(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid((a.rows + kTableRows - 1) / kTableRows);
    const size_t lds = 2 * (size_t)a.dim * sizeof(float);
#define ALNP_LAUNCH(V, W) launch_table_lds_shape<V, W>(a, grid, lds, s)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_adaln_fp8(const Fp8Args& args, int form, bool fast, hipStream_t s)
{
    Fp8Args a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (rs.vpt > 0 && form == kTable && a.dim <= kTableMaxDim && rs.threads <= 256)
        return launch_fp8_table_lds(a, rs, s);
    if (rs.vpt > 0) {
        switch (form) {
        case kNone: return launch_fp8_rows<kNone>(a, rs, s);
        case kBcast: return launch_fp8_rows<kBcast>(a, rs, s);
        case kPtok: return launch_fp8_rows<kPtok>(a, rs, s);
        case kTable: return launch_fp8_rows<kTable>(a, rs, s);
        case kModFp8: return launch_fp8_rows<kModFp8>(a, rs, s);
        case kAwq: return launch_fp8_rows<kAwq>(a, rs, s);
        default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_adaln_fp8_block, grid, dim3(256), 0, s, a, form);
    return hipGetLastError();
}

template <int FORM>
static hipError_t launch_mxfp8_rows(const Fp8Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(a.rows);
#define ALNP_LAUNCH(V, W) \
    hipLaunchKernelGGL((k_adaln_fp8_rows<V, W, FORM, true>), grid, dim3(W * 64), 0, s, a)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

template <int V, int W>
static void launch_table_lds_mx_shape(const Fp8Args& a, dim3 grid, size_t lds, hipStream_t s)
{
    if constexpr (W <= 4)
        hipLaunchKernelGGL((k_adaln_fp8_table_lds<V, W, kTableRows, true>), grid,
                           dim3(kTableRows * W * 64), lds, s, a);
}

hipError_t launch_mxfp8(const Fp8Args& args, int form, bool fast, hipStream_t s)
{
    Fp8Args a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (rs.vpt > 0 && form == kTable && a.dim <= kTableMaxDim && rs.threads <= 256) {
        const dim3 grid = row_grid((a.rows + kTableRows - 1) / kTableRows);
        const size_t lds = 2 * (size_t)a.dim * sizeof(float);
#define ALNP_LAUNCH(V, W) launch_table_lds_mx_shape<V, W>(a, grid, lds, s)
        ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        return hipGetLastError();
    }
    if (rs.vpt > 0) {
        switch (form) {
        case kNone: return launch_mxfp8_rows<kNone>(a, rs, s);
        case kBcast: return launch_mxfp8_rows<kBcast>(a, rs, s);
        case kPtok: return launch_mxfp8_rows<kPtok>(a, rs, s);
        case kTable: return launch_mxfp8_rows<kTable>(a, rs, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (form != kNone && form != kBcast && form != kPtok && form != kTable)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_mxfp8_block, grid, dim3(256), 0, s, a, form);
    return hipGetLastError();
}

template <int FORM, bool SWZ, bool MX = false>
static hipError_t launch_fp4_rows(const Fp4Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(a.rows);
#define ALNP_LAUNCH(V, W) hipLaunchKernelGGL((k_fp4_rows<V, W, FORM, SWZ, MX>), grid, dim3(W * 64), 0, s, a)
    ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_fp4(const Fp4Args& args, bool fast, hipStream_t s)
{
    Fp4Args a = args;
    a.inv_dim = 1.0f / (float)a.dim;
    const RowShape rs = fast ? row_shape(a.dim) : RowShape{0, 0};
    if (a.mx) {
        if (a.sf_layout != kSfRowMajor || (a.form != kNone && a.form != kBcast))
            return hipErrorInvalidValue;  // MXFP4: LN or broadcast AdaLN, row-major scales
        if (rs.vpt > 0)
            return a.form == kBcast ? launch_fp4_rows<kBcast, false, true>(a, rs, s)
                                    : launch_fp4_rows<kNone, false, true>(a, rs, s);
        const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
        hipLaunchKernelGGL(k_mxfp4_block, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if (rs.vpt > 0) {
        const bool swz = a.sf_layout == kSfSwizzled;
        switch (a.form) {
        case kNone:
            return swz ? launch_fp4_rows<kNone, true>(a, rs, s) : launch_fp4_rows<kNone, false>(a, rs, s);
        case kBcast:
            return swz ? launch_fp4_rows<kBcast, true>(a, rs, s) : launch_fp4_rows<kBcast, false>(a, rs, s);
        case kModFp8:
            if (!swz)
                return hipErrorInvalidValue;  // offered with tiled scales only
            return launch_fp4_rows<kModFp8, true>(a, rs, s);
        default:
            return hipErrorInvalidValue;
        }
    }
    const dim3 grid((unsigned)std::min<int64_t>(a.rows, kMaxGrid));
    hipLaunchKernelGGL(k_fp4_block, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const float* v, const float* act, int64_t n, uint8_t* out,
                            hipStream_t s)
{
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_quant_fp8, dim3((unsigned)blocks), dim3(256), 0, s, v, act, n, out);
    return hipGetLastError();
}

template <bool W>
static hipError_t launch_rms_rows(const RmsArgs& a, RowShape rs, hipStream_t s)
{
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
