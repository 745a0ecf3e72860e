// fp4.hip -- LayerNorm / adaptive-LayerNorm -> FP4 producers for gfx950.
//
// NVFP4 (README "Available Functions": the nvfp4 entries; e4m3 scale per 16
// elements, row-major or the 128x4 tiled layout) and MXFP4 (E8M0 scale per 32
// elements, OCP MX v1.0) from the bf16-staged normalized, optionally
// modulated, row; packed two e2m1 codes per byte, low nibble first.
#include "rows.hpp"

namespace alnp {

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
// row-major).  FULL: the row fills every vector slot, so the last slot needs
// no bounds check (same arithmetic).
template <int VPT, int WAVES, int FORM, bool SWZ, bool MX = false, bool FULL = false>
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
    int64_t row = grid_row();
    if (row >= a.rows)
        return;  // whole workgroup
    if (SWZ && (a.rows & 255) == 0) {
        // In the tiled layout a 128-byte line of scales holds 4 bytes from
        // each of 32 rows (equal r div 128 and (r mod 32) div 8).  Workgroups
        // go to the eight XCDs in turn, so workgroup w takes the row that
        // puts those 32 rows on one XCD, whose L2 then assembles each line
        // whole instead of eight L2s writing parts of it.  A bijection on
        // [0, rows) for rows a multiple of 256: w -> XCD x = w mod 8, its
        // k = w div 8 -> line group g = x + 8 (k div 32), member m = k mod 32.
        const int64_t x = row & 7, k = row >> 3;
        const int64_t g = x + 8 * (k >> 5), m = k & 31;
        row = (g >> 2) * 128 + 32 * (m >> 3) + 8 * (g & 3) + (m & 7);
    }
    // The encode factors 1 / s, staged from the compile-time table into LDS
    // (requested here, written once the row loads are in flight).
    const float recip0 = !MX && t < 128 ? kE4m3Recip.v[t] : 0.f;
    const float recip1 = !MX && T == 64 ? kE4m3Recip.v[t + 64] : 0.f;

    uint4 xv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
        xv[v] = ld_row<true>(a.x + row * dim, v * T + t, nvec, !FULL && v == VPT - 1);
    uint4 scv[NM], shv[NM];
    uint2 sc8[N8], sh8[N8];
    if (FORM == kBcast) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            scv[v] = ld_row<false>(a.scale, v * T + t, nvec, !FULL && v == VPT - 1);
            shv[v] = ld_row<false>(a.shift, v * T + t, nvec, !FULL && v == VPT - 1);
        }
    } else if (FORM == kModFp8) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            sc8[v] = ld_fp8x8(a.scale_fp8, v * T + t, nvec, !FULL && v == VPT - 1);
            sh8[v] = ld_fp8x8(a.shift_fp8, v * T + t, nvec, !FULL && v == VPT - 1);
        }
    }
    const float sdeq = FORM == kModFp8 ? *a.scale_deq : 0.f;
    const float hdeq = FORM == kModFp8 ? *a.shift_deq : 0.f;
    if (!MX && t < 128)
        inv_s[t] = recip0;
    if (!MX && T == 64)
        inv_s[t + 64] = recip1;

    const bool tail_ok = FULL || (VPT - 1) * T + t < nvec;
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
            uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w[0], __builtin_bit_cast(bf16x2, w[0]), xs, 0);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[1]), xs, 1);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[2]), xs, 2);
            word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, w[3]), xs, 3);
            st_stream(a.packed + row * (dim / 2) + (int64_t)i * 4, word);
            a.sf[row * (dim >> 5) + (i >> 2)] = (uint8_t)(E + 127);
            continue;
        }
        // Stage through bf16 (round to nearest even), one convert per element.
#pragma unroll
        for (int e = 0; e < 8; ++e)
            b[e] = bf16_round(y[e]);
        const float amax = pair_max(absmax8(b));
        const uint32_t scode = e4m3_code1(fminf(amax * kSixth, 448.0f));
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

// ---- launchers ----------------------------------------------------------------

template <int FORM, bool SWZ, bool MX = false>
static hipError_t launch_fp4_rows(const Fp4Args& a, RowShape rs, hipStream_t s)
{
    const dim3 grid = row_grid(a.rows);
    // Rows that fill every vector slot (dim 2048, 3072) take the variant
    // without the last slot's bounds check: NVFP4 4096 x 3072 7.29 -> 7.22 us
    // with the single-convert staging (A-B).  For MXFP4 it measured slower
    // (7.19 -> 7.37 us), so MX keeps the checked variant.
    if (!MX && (a.dim >> 3) == rs.vpt * rs.threads) {
#define ALNP_LAUNCH(V, W) hipLaunchKernelGGL((k_fp4_rows<V, W, FORM, SWZ, MX, true>), grid, dim3(W * 64), 0, s, a)
        ALNP_SHAPE_CASES(ALNP_LAUNCH)
#undef ALNP_LAUNCH
        return hipGetLastError();
    }
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
        // MXFP4: LN, broadcast or modfp8 AdaLN, row-major E8M0 scales.
        if (a.sf_layout != kSfRowMajor || (a.form != kNone && a.form != kBcast && a.form != kModFp8))
            return hipErrorInvalidValue;
        if (rs.vpt > 0) {
            switch (a.form) {
            case kBcast: return launch_fp4_rows<kBcast, false, true>(a, rs, s);
            case kModFp8: return launch_fp4_rows<kModFp8, false, true>(a, rs, s);
            default: return launch_fp4_rows<kNone, false, true>(a, rs, s);
            }
        }
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

}  // namespace alnp
