// residual.hip -- residual gate step for gfx950:
//   out = bf16(residual + bf16(gate * proj))
// the numerical program the h3-blackwell-runtime page fixes for the
// residual-gate epilogue (bf16 projection output, gate multiplication with
// its bf16 boundary, bf16 residual added in the reference order, final bf16
// rounding).  gate is per token (rows, dim) -- a six-way producer output
// chunk -- or broadcast (dim,).
//
// A pure stream (6-8 bytes per element).  With a per-token gate, one
// workgroup per row in the producers' row shape (for dim 3072: two waves,
// three 16-byte vectors of each operand per thread), every load in flight
// before the first store: the plainest streaming layout, and the one whose
// memory-only pass is fastest for these bytes.  With a broadcast gate, a
// thread owns one 8-element column slot and walks four consecutive rows, so
// the gate slot is read once into registers.  Each element is read and
// written by the same thread, so out may be residual itself.
#include "rows.hpp"

namespace alnp {

constexpr int kRowsPerThread = 4;

// Eight bf16 lanes: bf16(r + bf16(g * p)).
__device__ __forceinline__ uint4 gate8(const uint4& r, const uint4& g, const uint4& p)
{
    float rf[8], gf[8], pf[8];
    unpack8(r, rf);
    unpack8(g, gf);
    unpack8(p, pf);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const uint32_t gp = pack_bf16x2(gf[e] * pf[e], gf[e + 1] * pf[e + 1]);
        o[e / 2] = pack_bf16x2(rf[e] + bf16_lo(gp), rf[e + 1] + bf16_hi(gp));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Per-token gate: one row per workgroup, VPT vectors per thread (vector
// i = v * threads + t); only a thread's last slot can lie past the row end
// unless the row fills every slot (FULL).
template <int VPT, int WAVES, bool FULL>
__global__ __launch_bounds__(WAVES * 64) void k_gated_residual_rows(GateArgs a)
{
    constexpr int T = WAVES * 64;
    const int t = threadIdx.x;
    const int64_t row = grid_row();
    if (row >= a.rows)
        return;
    const int nvec = a.dim >> 3;
    const int64_t base = row * a.dim;
    uint4 rv[VPT], gv[VPT], pv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (FULL || v < VPT - 1 || i < nvec) {
            rv[v] = ld_stream(a.residual + base + 8 * (int64_t)i);
            gv[v] = ld_stream(a.gate + base + 8 * (int64_t)i);
            pv[v] = ld_stream(a.proj + base + 8 * (int64_t)i);
        }
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * T + t;
        if (FULL || v < VPT - 1 || i < nvec)
            st_stream(a.out + base + 8 * (int64_t)i, gate8(rv[v], gv[v], pv[v]));
    }
}

// Broadcast gate: blockDim.x threads over the row's 8-element slots.
template <bool BCAST>
__global__ __launch_bounds__(256) void k_gated_residual_vec(GateArgs a)
{
    const int dv = a.dim >> 3;
    const int j8 = blockIdx.x * blockDim.x + threadIdx.x;
    if (j8 >= dv)
        return;
    const int64_t r0 = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * kRowsPerThread;
    uint4 rv[kRowsPerThread], pv[kRowsPerThread], gv[BCAST ? 1 : kRowsPerThread];
    if (BCAST)
        gv[0] = ld_keep(a.gate + 8 * (int64_t)j8);
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int64_t r = r0 + u < a.rows ? r0 + u : a.rows - 1;
        const int64_t off = r * a.dim + 8 * (int64_t)j8;
        rv[u] = ld_stream(a.residual + off);
        pv[u] = ld_stream(a.proj + off);
        if (!BCAST)
            gv[u] = ld_stream(a.gate + off);
    }
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int64_t r = r0 + u;
        if (r >= a.rows)
            break;
        st_stream(a.out + r * a.dim + 8 * (int64_t)j8, gate8(rv[u], gv[BCAST ? 0 : u], pv[u]));
    }
}

// Any dim, element-aligned pointers.
__global__ __launch_bounds__(256) void k_gated_residual_scalar(GateArgs a)
{
    const int64_t n = a.rows * a.dim;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t j = i % a.dim;
        const float g = __uint_as_float((uint32_t)a.gate[a.gate_rows == 1 ? j : i] << 16);
        const float p = __uint_as_float((uint32_t)a.proj[i] << 16);
        const float r = __uint_as_float((uint32_t)a.residual[i] << 16);
        const float gp = bf16_lo(pack_bf16x2(g * p, 0.f));
        a.out[i] = (uint16_t)(pack_bf16x2(r + gp, 0.f) & 0xFFFFu);
    }
}

hipError_t launch_gated_residual(const GateArgs& a, bool fast, hipStream_t s)
{
    const RowShape rs = fast && a.gate_rows != 1 && a.dim <= kMaxFastDim ? row_shape(a.dim)
                                                                         : RowShape{0, 0};
    if (rs.vpt > 0) {
        const dim3 grid = row_grid(a.rows);
        if ((a.dim >> 3) == rs.vpt * rs.threads) {
#define ALNP_LAUNCH(V, W) \
    hipLaunchKernelGGL((k_gated_residual_rows<V, W, true>), grid, dim3(W * 64), 0, s, a)
            ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        } else {
#define ALNP_LAUNCH(V, W) \
    hipLaunchKernelGGL((k_gated_residual_rows<V, W, false>), grid, dim3(W * 64), 0, s, a)
            ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        }
    } else if (fast) {
        // Workgroups of 256 threads over the row's slots, or 128 or 64 when
        // that divides them (dim 3072: three of 128, no idle wave).
        const int64_t dv = a.dim >> 3;
        const int bt = dv % 256 == 0 ? 256 : dv % 128 == 0 ? 128 : dv % 64 == 0 ? 64 : 256;
        const int64_t groups = (a.rows + kRowsPerThread - 1) / kRowsPerThread;
        const int64_t gy = groups < 65535 ? groups : 65535;
        const dim3 grid((unsigned)((dv + bt - 1) / bt), (unsigned)gy, (unsigned)((groups + gy - 1) / gy));
        if (a.gate_rows == 1)
            hipLaunchKernelGGL(k_gated_residual_vec<true>, grid, dim3(bt), 0, s, a);
        else
            hipLaunchKernelGGL(k_gated_residual_vec<false>, grid, dim3(bt), 0, s, a);
    } else {
        const int64_t n = a.rows * a.dim;
        const int64_t blocks = (n + 255) / 256;
        const dim3 grid((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20)));
        hipLaunchKernelGGL(k_gated_residual_scalar, grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace alnp
