// modulation6.hip -- six-way DiT modulation producer for gfx950.
//
// out_k[t, :] = bf16_rne(params[t, k, :] + mod[k, :]) for k = 0..5
// ("adaptive-layernorm-producers" README, "Tensor Contract": fp32 params of
// shape (batch, seq, 6, dim) and an fp32 (6, dim) per-layer table in, six
// bf16 (batch, seq, dim) tensors out).
//
// A pure stream: 4 bytes read and 2 written per element, one add.  Each wave
// owns 512 consecutive floats of a token's (6, dim) span and handles them for
// four consecutive tokens: its lanes read them as two contiguous 1 KiB loads
// per token (lane j: floats 4j..4j+3 of each 256-float half), all eight
// 16-byte non-temporal params loads are in flight before the first store, and
// the matching table values are loaded once into registers after them.  A
// lane pair then holds eight consecutive outputs per half; one DPP swap lets
// the even lane store half 0 and the odd lane half 1, 16 bytes each,
// non-temporal.  (Reading the table per token instead cost 7% extra HBM
// fetches, as streamed params evicted it from L2, and ~20% in time.  The
// earlier mapping, a lane per 8-float slot, read 32 bytes per lane as two
// loads that each touched every line of a 2 KiB span half: 97.2 us against
// 90.0 on the 1 x 5070 x 3072 workload, A-B, bit-identical.)
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

// Tokens per thread in the vector kernel (2 and 8 measured slower).
constexpr int kTokensPerThread = 4;

// Wave w of workgroup blockIdx.x covers floats [512 (4 blockIdx.x + w), + 512)
// of the span (6 * dim floats per token, dim % 8 == 0, so a lane pair's eight
// floats lie in one chunk and wholly inside or outside the span); lanes past
// the span load a valid address and store nothing.  (blockIdx.y, blockIdx.z)
// pick the token group.
__global__ __launch_bounds__(256) void k_mod6_vec(Mod6Args a)
{
    const int span = 6 * a.dim;
    const int blk = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 512;
    if (blk >= span)
        return;  // whole wave
    const int lane = threadIdx.x & (kWave - 1);
    int e[2], k[2];
    bool ok[2];
    float4 m[2];
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
    // The table values (L2 hits) after the params loads, which they would
    // otherwise hold up in the CU's load queue (a scheduling barrier keeps
    // them there): 89.2 -> 88.3 us (A-B, bit-identical).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
        m[h] = *reinterpret_cast<const float4*>(a.mod + e[h]);
    const bool odd = lane & 1;
    const int hs = odd ? 1 : 0;                        // the half this lane stores
    uint16_t* out = select_out(a, k[hs]);
    const int js = (odd ? e[1] - 4 : e[0]) - k[hs] * a.dim;  // its pair's first element
#pragma unroll
    for (int u = 0; u < kTokensPerThread; ++u) {
        const int64_t t = t0 + u;
        if (t >= a.tokens)
            break;
        uint2 o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 q = as_f4(p[u][h]);
            o[h].x = pack_bf16x2(q.x + m[h].x, q.y + m[h].y);
            o[h].y = pack_bf16x2(q.z + m[h].z, q.w + m[h].w);
        }
        const uint2 snd = odd ? o[0] : o[1];
        const uint32_t r0 = __builtin_amdgcn_mov_dpp(snd.x, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        const uint32_t r1 = __builtin_amdgcn_mov_dpp(snd.y, 0xB1, 0xF, 0xF, false);
        if (ok[hs])
            st_stream(out + t * a.dim + js, odd ? make_uint4(r0, r1, o[1].x, o[1].y)
                                                : make_uint4(o[0].x, o[0].y, r0, r1));
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
        const int64_t waves = (6 * (int64_t)a.dim + 511) / 512;
        const int64_t groups = (a.tokens + kTokensPerThread - 1) / kTokensPerThread;
        const int64_t gy = groups < 65535 ? groups : 65535;
        const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)gy, (unsigned)((groups + gy - 1) / gy));
        hipLaunchKernelGGL(k_mod6_vec, grid, dim3(256), 0, s, a);
    } else {
        const dim3 grid((unsigned)(a.tokens < (1 << 20) ? a.tokens : (1 << 20)));
        hipLaunchKernelGGL(k_mod6_scalar, grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace alnp
