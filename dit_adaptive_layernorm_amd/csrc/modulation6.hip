// modulation6.hip -- six-way DiT modulation producer for gfx950.
//
// out_k[t, :] = bf16_rne(params[t, k, :] + mod[k, :]) for k = 0..5
// ("adaptive-layernorm-producers" README, "Tensor Contract": FP32
// (batch, sequence, 6, dim) parameters plus FP32 (6, dim) layer modulation,
// six BF16 (batch, sequence, dim) outputs).
//
// A pure stream: 4 bytes read and 2 written per element, one add.  One
// 256-thread workgroup per token; each thread moves 8 elements per step
// (two 16-byte loads of params, two of the 72 KiB table, which stays in L2,
// one 16-byte store).  Consecutive threads take consecutive 8-element
// vectors of the token's 6*dim span, so loads and stores are contiguous
// across the wave.
#include "device_common.hpp"
#include "kernels.hpp"

namespace alnp {

__device__ __forceinline__ uint16_t* select_out(const Mod6Args& a, int k)
{
    uint16_t* p = a.out[0];
    p = k == 1 ? a.out[1] : p;
    p = k == 2 ? a.out[2] : p;
    p = k == 3 ? a.out[3] : p;
    p = k == 4 ? a.out[4] : p;
    p = k == 5 ? a.out[5] : p;
    return p;
}

__global__ __launch_bounds__(256) void k_mod6_vec(Mod6Args a)
{
    const int64_t t = blockIdx.x;
    const int dv = a.dim >> 3;             // 8-element vectors per chunk
    const float* pt = a.params + t * 6 * (int64_t)a.dim;
    for (int i = threadIdx.x; i < 6 * dv; i += 256) {
        const int k = (i >= dv) + (i >= 2 * dv) + (i >= 3 * dv) + (i >= 4 * dv) + (i >= 5 * dv);
        const int j8 = i - k * dv;
        const float4 p0 = reinterpret_cast<const float4*>(pt)[2 * i];
        const float4 p1 = reinterpret_cast<const float4*>(pt)[2 * i + 1];
        const float4* mk = reinterpret_cast<const float4*>(a.mod + (int64_t)k * a.dim) + 2 * j8;
        const float4 m0 = mk[0];
        const float4 m1 = mk[1];
        uint4 o;
        o.x = pack_bf16x2(p0.x + m0.x, p0.y + m0.y);
        o.y = pack_bf16x2(p0.z + m0.z, p0.w + m0.w);
        o.z = pack_bf16x2(p1.x + m1.x, p1.y + m1.y);
        o.w = pack_bf16x2(p1.z + m1.z, p1.w + m1.w);
        reinterpret_cast<uint4*>(select_out(a, k) + t * a.dim)[j8] = o;
    }
}

// Any even or odd dim, any element-aligned pointers.
__global__ __launch_bounds__(256) void k_mod6_scalar(Mod6Args a)
{
    const int64_t t = blockIdx.x;
    const int dim = a.dim;
    const float* pt = a.params + t * 6 * (int64_t)dim;
    for (int i = threadIdx.x; i < 6 * dim; i += 256) {
        const int k = (i >= dim) + (i >= 2 * dim) + (i >= 3 * dim) + (i >= 4 * dim) + (i >= 5 * dim);
        const int j = i - k * dim;
        const float s = pt[i] + a.mod[(int64_t)k * dim + j];
        select_out(a, k)[t * dim + j] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xFFFFu);
    }
}

hipError_t launch_modulation6(const Mod6Args& a, bool fast, hipStream_t s)
{
    const dim3 grid((unsigned)a.tokens), block(256);
    if (fast)
        hipLaunchKernelGGL(k_mod6_vec, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(k_mod6_scalar, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace alnp
