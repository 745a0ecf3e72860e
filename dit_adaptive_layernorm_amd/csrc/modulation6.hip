// modulation6.hip -- six-way DiT modulation producer for gfx950.
//
// out_k[t, :] = bf16_rne(params[t, k, :] + mod[k, :]) for k = 0..5
// ("adaptive-layernorm-producers" README, "Tensor Contract": FP32
// (batch, sequence, 6, dim) parameters plus FP32 (6, dim) layer modulation,
// six BF16 (batch, sequence, dim) outputs).
//
// A pure stream: 4 bytes read and 2 written per element, one add.  One
// 256-thread workgroup per token (grid-stride over tokens); each thread moves
// 8 elements per step (two 16-byte non-temporal loads of params, two
// ordinary loads of the 72 KiB table, which stays in L2, one 16-byte
// non-temporal store), up to three steps in flight.  Consecutive threads take
// consecutive 8-element vectors of the token's 6*dim span, so loads and
// stores are contiguous across the wave.
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

__device__ __forceinline__ float4 as_f4(const uint4& u)
{
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}

// One 8-element step: vector i of the token's 6*dim span.
__device__ __forceinline__ void mod6_step(const Mod6Args& a, int64_t t, int dv, int i,
                                          const uint4& p0u, const uint4& p1u)
{
    const int k = (i >= dv) + (i >= 2 * dv) + (i >= 3 * dv) + (i >= 4 * dv) + (i >= 5 * dv);
    const int j8 = i - k * dv;
    const float4* mk = reinterpret_cast<const float4*>(a.mod + (int64_t)k * a.dim) + 2 * j8;
    const float4 m0 = mk[0], m1 = mk[1];
    const float4 p0 = as_f4(p0u), p1 = as_f4(p1u);
    uint4 o;
    o.x = pack_bf16x2(p0.x + m0.x, p0.y + m0.y);
    o.y = pack_bf16x2(p0.z + m0.z, p0.w + m0.w);
    o.z = pack_bf16x2(p1.x + m1.x, p1.y + m1.y);
    o.w = pack_bf16x2(p1.z + m1.z, p1.w + m1.w);
    st_stream(select_out(a, k) + t * a.dim + 8 * (int64_t)j8, o);
}

__global__ __launch_bounds__(256) void k_mod6_vec(Mod6Args a)
{
    const int dv = a.dim >> 3;             // 8-element vectors per chunk
    const int n = 6 * dv;                  // vectors per token
    for (int64_t t = blockIdx.x; t < a.tokens; t += gridDim.x) {
        const float* pt = a.params + t * 6 * (int64_t)a.dim;
        int i = threadIdx.x;
        // Three steps per round, all loads issued before any store.
        for (; i + 512 < n; i += 768) {
            const uint4 a0 = ld_stream(pt + 8 * i), a1 = ld_stream(pt + 8 * i + 4);
            const uint4 b0 = ld_stream(pt + 8 * (i + 256)), b1 = ld_stream(pt + 8 * (i + 256) + 4);
            const uint4 c0 = ld_stream(pt + 8 * (i + 512)), c1 = ld_stream(pt + 8 * (i + 512) + 4);
            mod6_step(a, t, dv, i, a0, a1);
            mod6_step(a, t, dv, i + 256, b0, b1);
            mod6_step(a, t, dv, i + 512, c0, c1);
        }
        for (; i < n; i += 256)
            mod6_step(a, t, dv, i, ld_stream(pt + 8 * i), ld_stream(pt + 8 * i + 4));
    }
}

// Any even or odd dim, any element-aligned pointers.
__global__ __launch_bounds__(256) void k_mod6_scalar(Mod6Args a)
{
    const int dim = a.dim;
    for (int64_t t = blockIdx.x; t < a.tokens; t += gridDim.x) {
        const float* pt = a.params + t * 6 * (int64_t)dim;
        for (int i = threadIdx.x; i < 6 * dim; i += 256) {
            const int k = (i >= dim) + (i >= 2 * dim) + (i >= 3 * dim) + (i >= 4 * dim) + (i >= 5 * dim);
            const int j = i - k * dim;
            const float s = pt[i] + a.mod[(int64_t)k * dim + j];
            select_out(a, k)[t * dim + j] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xFFFFu);
        }
    }
}

hipError_t launch_modulation6(const Mod6Args& a, bool fast, hipStream_t s)
{
    const dim3 grid((unsigned)(a.tokens < (1 << 20) ? a.tokens : (1 << 20))), block(256);
    if (fast)
        hipLaunchKernelGGL(k_mod6_vec, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(k_mod6_scalar, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace alnp
