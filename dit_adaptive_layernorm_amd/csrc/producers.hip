// producers.hip -- LayerNorm / adaptive-LayerNorm producers for gfx950.
//
// What is computed (per row of a bf16 (rows, dim) activation) follows the
// "adaptive-layernorm-producers" README ("Available Functions", "Tensor
// Contract"): LayerNorm without affine weights, DiT modulation
// (xhat * (1 + scale)) + shift (operation order from the h3-blackwell-runtime
// page, "NVFP4 Modulation Producer Fusion", "Exactness Contract"), then
// static-scale e4m3 or block-16 e2m1 quantization.
//
// Kernel design (MI355X): the problem is a pure stream (3-7 bytes moved per
// element, ~15 flops), so the kernels are built for HBM, not MFMA.
//  - Fast path: one wave64 per row, four rows per 256-thread workgroup.  A
//    lane owns NV 16-byte vectors of the row (vector i = v*64 + lane), so
//    every load instruction of a wave covers 1 KiB of contiguous memory.
//    The whole row stays in registers: x, then the per-token operands, are
//    requested up front so their latency overlaps; mean and variance are two
//    passes over registers with DPP wave reductions (no LDS, no barrier).
//  - Fallback (dim not a multiple of 8, rows longer than 8192, or operands
//    not 16-byte aligned): one 256-thread workgroup per row, element loops,
//    LDS for the cross-wave sums.  Same arithmetic.
#include "device_common.hpp"
#include "kernels.hpp"

namespace alnp {

// ---- operand forms --------------------------------------------------------

enum Form { kNone = 0, kBcast = 1, kPtok = 2, kTable = 3 };

// Eight consecutive fp32 of `p` starting at element e (16-byte aligned).
__device__ __forceinline__ void load_f32x8(const float* p, float f[8])
{
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// ---- fast path: one wave per row --------------------------------------------

// Loads vector i of a bf16 row, or zeros past the end of the row.
__device__ __forceinline__ uint4 ld16(const uint16_t* row, int i, int nvec)
{
    return i < nvec ? reinterpret_cast<const uint4*>(row)[i] : make_uint4(0, 0, 0, 0);
}

// Row statistics from the NV register vectors of a lane.  Zero-filled
// vectors past the row end add nothing to the sum and are skipped in the
// squared deviations.
template <int NV>
__device__ __forceinline__ void row_stats(const uint4 (&xv)[NV], int lane, int nvec, int dim,
                                          float eps, float& mean, float& rstd)
{
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float f[8];
        unpack8(xv[v], f);
        s += ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
    }
    mean = wave_sum(s) / (float)dim;
    float q = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        if (v * kWave + lane < nvec) {
            float f[8];
            unpack8(xv[v], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = f[e] - mean;
                q = __builtin_fmaf(d, d, q);
            }
        }
    }
    const float var = wave_sum(q) / (float)dim;
    rstd = (float)(1.0 / sqrt((double)var + (double)eps));
}

template <int NV, int FORM>
__global__ __launch_bounds__(256) void k_adaln_fp8_wave(Fp8Args a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows)
        return;  // the whole wave leaves together
    const int dim = a.dim;
    const int nvec = dim >> 3;
    const uint16_t* xr = a.x + row * dim;

    uint4 xv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
        xv[v] = ld16(xr, v * kWave + lane, nvec);

    // Modulation operands, requested before the reductions.
    const uint16_t* scr = nullptr;
    const uint16_t* shr = nullptr;
    if (FORM == kBcast) {
        scr = a.scale;
        shr = a.shift;
    } else if (FORM == kPtok) {
        scr = a.scale + row * dim;
        shr = a.shift + row * dim;
    } else if (FORM == kTable) {
        scr = a.temb + (row * a.chunks + a.scale_idx) * dim;
        shr = a.temb + (row * a.chunks + a.shift_idx) * dim;
    }
    uint4 scv[FORM == kNone ? 1 : NV], shv[FORM == kNone ? 1 : NV];
    if (FORM != kNone) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            scv[v] = ld16(scr, v * kWave + lane, nvec);
            shv[v] = ld16(shr, v * kWave + lane, nvec);
        }
    }

    float mean, rstd;
    row_stats<NV>(xv, lane, nvec, dim, a.eps, mean, rstd);
    const float inv = 1.0f / *a.act_scale;

#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = v * kWave + lane;
        if (i >= nvec)
            continue;
        float f[8], sc[8], sh[8];
        unpack8(xv[v], f);
        if (FORM == kNone) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sc[e] = 0.f;
                sh[e] = 0.f;
            }
        } else {
            unpack8(scv[v], sc);
            unpack8(shv[v], sh);
            if (FORM == kTable) {
                float ts[8], th[8];
                load_f32x8(a.table + (int64_t)a.scale_idx * dim + i * 8, ts);
                load_f32x8(a.table + (int64_t)a.shift_idx * dim + i * 8, th);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sc[e] = sc[e] + ts[e];
                    sh[e] = sh[e] + th[e];
                }
            }
        }
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xhat = (f[e] - mean) * rstd;
            const float y = (xhat * (1.0f + sc[e])) + sh[e];
            q[e] = sat448(y * inv);
        }
        uint2 o;
        o.x = pack_e4m3x4(q[0], q[1], q[2], q[3]);
        o.y = pack_e4m3x4(q[4], q[5], q[6], q[7]);
        *reinterpret_cast<uint2*>(a.out + row * dim + (int64_t)i * 8) = o;
    }
    if (lane == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
}

template <int NV>
__global__ __launch_bounds__(256) void k_ln_fp4_wave(Fp4Args a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows)
        return;
    const int dim = a.dim;
    const int nvec = dim >> 3;  // even, since dim % 16 == 0
    const uint16_t* xr = a.x + row * dim;

    uint4 xv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
        xv[v] = ld16(xr, v * kWave + lane, nvec);

    float mean, rstd;
    row_stats<NV>(xv, lane, nvec, dim, a.eps, mean, rstd);

#pragma unroll
    for (int v = 0; v < NV; ++v) {
        // Both lanes of a block pair take the same branch: nvec is even.
        const int i = v * kWave + lane;
        if (i >= nvec)
            continue;
        float f[8], b[8];
        unpack8(xv[v], f);
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            // Normalize, then stage through bf16 (round to nearest even).
            const uint32_t w = pack_bf16x2((f[e] - mean) * rstd, (f[e + 1] - mean) * rstd);
            b[e] = bf16_lo(w);
            b[e + 1] = bf16_hi(w);
            amax = fmaxf(amax, fmaxf(fabsf(b[e]), fabsf(b[e + 1])));
        }
        amax = pair_max(amax);
        const float target = fminf(amax / 6.0f, 448.0f);
        const uint32_t scode = pack_e4m3x4(target, 0.f, 0.f, 0.f) & 0xFFu;
        const float s = e4m3_value(scode);
        uint32_t word = 0;
        if (s != 0.f) {
            const float enc = 1.0f / s;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                word |= e2m1_code(b[e] * enc) << (4 * e);
        }
        *reinterpret_cast<uint32_t*>(a.packed + row * (dim / 2) + (int64_t)i * 4) = word;
        if ((lane & 1) == 0)
            a.sf[row * (dim / 16) + (i >> 1)] = (uint8_t)scode;
    }
    if (lane == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
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

__device__ __forceinline__ void block_row_stats(const uint16_t* xr, int dim, float eps,
                                                float* lds4, float& mean, float& rstd)
{
    float s = 0.f;
    for (int j = threadIdx.x; j < dim; j += 256)
        s += ldbf(xr, j);
    mean = block_sum(s, lds4) / (float)dim;
    float q = 0.f;
    for (int j = threadIdx.x; j < dim; j += 256) {
        const float d = ldbf(xr, j) - mean;
        q = __builtin_fmaf(d, d, q);
    }
    const float var = block_sum(q, lds4) / (float)dim;
    rstd = (float)(1.0 / sqrt((double)var + (double)eps));
}

__global__ __launch_bounds__(256) void k_adaln_fp8_block(Fp8Args a, int form)
{
    __shared__ float lds4[4];
    const int64_t row = blockIdx.x;
    const int dim = a.dim;
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.eps, lds4, mean, rstd);
    const float inv = 1.0f / *a.act_scale;
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
        }
        const float xhat = (ldbf(xr, j) - mean) * rstd;
        const float y = (xhat * (1.0f + sc)) + sh;
        a.out[row * dim + j] = (uint8_t)(pack_e4m3x4(sat448(y * inv), 0.f, 0.f, 0.f) & 0xFFu);
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
    }
}

// One thread per 16-element block.
__global__ __launch_bounds__(256) void k_ln_fp4_block(Fp4Args a)
{
    __shared__ float lds4[4];
    const int64_t row = blockIdx.x;
    const int dim = a.dim;
    const uint16_t* xr = a.x + row * dim;
    float mean, rstd;
    block_row_stats(xr, dim, a.eps, lds4, mean, rstd);
    for (int k = threadIdx.x; k < dim / 16; k += 256) {
        float b[16];
        float amax = 0.f;
        for (int e = 0; e < 16; e += 2) {
            const int j = 16 * k + e;
            const uint32_t w = pack_bf16x2((ldbf(xr, j) - mean) * rstd, (ldbf(xr, j + 1) - mean) * rstd);
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
        a.sf[row * (dim / 16) + k] = (uint8_t)scode;
    }
    if (threadIdx.x == 0) {
        if (a.row_mean) a.row_mean[row] = mean;
        if (a.row_rstd) a.row_rstd[row] = rstd;
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

template <int FORM>
static hipError_t launch_fp8_wave(const Fp8Args& a, int nv, hipStream_t s)
{
    const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
    switch (nv) {
#define ALNP_CASE(N) \
    case N: hipLaunchKernelGGL((k_adaln_fp8_wave<N, FORM>), grid, block, 0, s, a); break;
        ALNP_CASE(1) ALNP_CASE(2) ALNP_CASE(3) ALNP_CASE(4) ALNP_CASE(5) ALNP_CASE(6)
        ALNP_CASE(7) ALNP_CASE(8) ALNP_CASE(9) ALNP_CASE(10) ALNP_CASE(11) ALNP_CASE(12)
        ALNP_CASE(13) ALNP_CASE(14) ALNP_CASE(15) ALNP_CASE(16)
#undef ALNP_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_adaln_fp8(const Fp8Args& a, int form, bool fast, hipStream_t s)
{
    if (fast) {
        const int nv = (a.dim / 8 + kWave - 1) / kWave;
        switch (form) {
        case kNone: return launch_fp8_wave<kNone>(a, nv, s);
        case kBcast: return launch_fp8_wave<kBcast>(a, nv, s);
        case kPtok: return launch_fp8_wave<kPtok>(a, nv, s);
        case kTable: return launch_fp8_wave<kTable>(a, nv, s);
        default: return hipErrorInvalidValue;
        }
    }
    hipLaunchKernelGGL(k_adaln_fp8_block, dim3((unsigned)a.rows), dim3(256), 0, s, a, form);
    return hipGetLastError();
}

hipError_t launch_ln_fp4(const Fp4Args& a, bool fast, hipStream_t s)
{
    if (fast) {
        const int nv = (a.dim / 8 + kWave - 1) / kWave;
        const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
        switch (nv) {
#define ALNP_CASE(N) \
    case N: hipLaunchKernelGGL((k_ln_fp4_wave<N>), grid, block, 0, s, a); break;
            ALNP_CASE(1) ALNP_CASE(2) ALNP_CASE(3) ALNP_CASE(4) ALNP_CASE(5) ALNP_CASE(6)
            ALNP_CASE(7) ALNP_CASE(8) ALNP_CASE(9) ALNP_CASE(10) ALNP_CASE(11) ALNP_CASE(12)
            ALNP_CASE(13) ALNP_CASE(14) ALNP_CASE(15) ALNP_CASE(16)
#undef ALNP_CASE
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_ln_fp4_block, dim3((unsigned)a.rows), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quant_fp8(const float* v, const float* act, int64_t n, uint8_t* out,
                            hipStream_t s)
{
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_quant_fp8, dim3((unsigned)blocks), dim3(256), 0, s, v, act, n, out);
    return hipGetLastError();
}

}  // namespace alnp
