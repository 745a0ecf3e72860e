// modulation6.hip -- six-way DiT modulation producer for gfx950.
//
// out_k[t, :] = bf16_rne(params[t, k, :] + mod[k, :]) for k = 0..5
// ("adaptive-layernorm-producers" README, "Tensor Contract": fp32 params of
// shape (batch, seq, 6, dim) and an fp32 (6, dim) per-layer table in, six
// bf16 (batch, seq, dim) tensors out).
//
// A pure stream: 4 bytes read and 2 written per element, one add.  Each
// thread owns one 8-element slot of the (6, dim) span and handles it for four
// consecutive tokens: the matching slot of the (6, dim) table is loaded once
// into registers, the eight 16-byte non-temporal params loads are all in
// flight before the first 16-byte non-temporal store.  Consecutive threads
// take consecutive slots, so every wave access is 1 KiB contiguous.  (Reading
// the table per token instead cost 7% extra HBM fetches, as streamed params
// evicted it from L2, and ~20% in time.)
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

// Tokens per thread in the vector kernel.
constexpr int kTokensPerThread = 4;

// A thread owns one 8-element slot i of the token span (chunk k, columns
// 8*j8 .. 8*j8+7) and walks kTokensPerThread consecutive tokens: the table
// slot is read once into registers and reused, and all of the thread's
// params loads are in flight before the first store.  blockIdx.x picks 256
// slots, (blockIdx.y, blockIdx.z) the token group.
__global__ __launch_bounds__(256) void k_mod6_vec(Mod6Args a)
{
    const int dv = a.dim >> 3;  // 8-element vectors per chunk
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= 6 * dv)
        return;
    const int k = (i >= dv) + (i >= 2 * dv) + (i >= 3 * dv) + (i >= 4 * dv) + (i >= 5 * dv);
    const int j8 = i - k * dv;
    uint16_t* out = select_out(a, k);
    const float4* mk = reinterpret_cast<const float4*>(a.mod + (int64_t)k * a.dim) + 2 * j8;
    const float4 m0 = mk[0], m1 = mk[1];
    const int64_t t0 = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * kTokensPerThread;
    uint4 p0[kTokensPerThread], p1[kTokensPerThread];
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
        const int64_t t = t0 + u < a.tokens ? t0 + u : a.tokens - 1;
        const float* pt = a.params + t * 6 * (int64_t)a.dim + 8 * (int64_t)i;
        p0[u] = ld_stream(pt);
        p1[u] = ld_stream(pt + 4);
    }
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
        const int64_t t = t0 + u;
        if (t >= a.tokens)
            break;
        const float4 q0 = as_f4(p0[u]), q1 = as_f4(p1[u]);
        uint4 o;
        o.x = pack_bf16x2(q0.x + m0.x, q0.y + m0.y);
        o.y = pack_bf16x2(q0.z + m0.z, q0.w + m0.w);
        o.z = pack_bf16x2(q1.x + m1.x, q1.y + m1.y);
        o.w = pack_bf16x2(q1.z + m1.z, q1.w + m1.w);
        st_stream(out + t * a.dim + 8 * (int64_t)j8, o);
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
    if (fast) {
        const int64_t slots = 6 * (int64_t)(a.dim >> 3);
        const int64_t groups = (a.tokens + kTokensPerThread - 1) / kTokensPerThread;
        const int64_t gy = groups < 65535 ? groups : 65535;
        const dim3 grid((unsigned)((slots + 255) / 256), (unsigned)gy, (unsigned)((groups + gy - 1) / gy));
        hipLaunchKernelGGL(k_mod6_vec, grid, dim3(256), 0, s, a);
    } else {
        const dim3 grid((unsigned)(a.tokens < (1 << 20) ? a.tokens : (1 << 20)));
        hipLaunchKernelGGL(k_mod6_scalar, grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace alnp
