// device_common.hpp -- gfx950 device helpers shared by the producer kernels.
//
// Compiled with -ffp-contract=off: every float expression below is one
// IEEE-rounded operation unless it calls __builtin_fmaf explicitly, so the
// modulation order (xhat * (1 + scale)) + shift is evaluated exactly as
// written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alnp {

constexpr int kWave = 64;

// ---- memory ----------------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16-byte loads.  Streamed operands (read once per call) use the
// non-temporal hint so they do not displace reused data in L2 / Infinity
// Cache; operands shared by every row (broadcast scale/shift, the table) use
// ordinary loads.
__device__ __forceinline__ uint4 ld_stream(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_keep(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Non-temporal stores of 4, 8 and 16 bytes (outputs are not re-read here).
__device__ __forceinline__ void st_stream(void* p, uint32_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_stream(void* p, uint2 v)
{
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_stream(void* p, uint4 v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// ---- bf16 ----------------------------------------------------------------

// bf16 -> fp32 is exact: the pattern is the upper half of the float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 (one 16-byte vector) -> eight floats.
__device__ __forceinline__ void unpack8(const uint4& v, float f[8])
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16, round to nearest even (v_cvt_pk_bf16_f32);
// element a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf16_rne(v) held as a float: one v_cvt_pk_bf16_f32 with a zero low half
// leaves the bf16 pattern in the upper half and zeros below, which is the
// float value of the bf16 (one instruction, where converting a pair and
// unpacking it takes one and a half per element).
__device__ __forceinline__ float bf16_round(float v)
{
    return __uint_as_float(pack_bf16x2(0.f, v));
}

// ---- e4m3 ----------------------------------------------------------------

// Clamp to the e4m3 range, keeping NaN: IEEE 754-2019 minimum and maximum
// (v_minimum3_f32 / v_maximum3_f32), which return NaN for a NaN operand.
__device__ __forceinline__ float sat448(float v)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_minimum(v, 448.0f), -448.0f);
}

// Four floats (already in range) -> four e4m3 codes, element a in byte 0.
// v_cvt_pk_fp8_f32 rounds to nearest even and writes the OCP e4m3 format on
// gfx950.  Each convert writes one half of the word and keeps the other; the
// two together write all of it, so the word they start from is a's own bits
// (a register already held) rather than a zero the compiler would have to
// materialize.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Eight e4m3 codes (bytes of v, byte 0 first) -> eight floats, exact
// (v_cvt_pk_f32_fp8).
__device__ __forceinline__ void unpack_e4m3x8(const uint2& v, float f[8])
{
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
    f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// Value of a non-negative e4m3 code below 0x7F: m * 2^-9 (subnormal) or
// (8 + m) * 2^(e - 10).
__device__ __forceinline__ float e4m3_value(uint32_t code)
{
    uint32_t e = (code >> 3) & 0xF, m = code & 7;
    return e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8 + m), (int)e - 10);
}

// ---- e2m1 ----------------------------------------------------------------

// Round to nearest even onto {0, .5, 1, 1.5, 2, 3, 4, 6}: count the decision
// points passed.  Strict '>' at points whose lower neighbour has the even
// code, '>=' where the upper one does; 6 and above (and inf) give code 7.
// NaN passes no point and keeps only its sign.
__device__ __forceinline__ uint32_t e2m1_code(float v)
{
    float a = fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                 (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Eight floats -> eight e2m1 codes packed low nibble first (element e in
// bits 4e..4e+3), by v_cvt_scalef32_pk_fp4_f32 with scale 1: round to
// nearest even onto the e2m1 grid, saturating at +-6, sign kept (matches
// e2m1_code for every non-NaN input).
__device__ __forceinline__ uint32_t pack_e2m1x8(float a, float b, float c, float d, float e,
                                                float f, float g, float h)
{
    // The four converts write all four bytes: start from a's bits (see
    // pack_e4m3x4).
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(a), a, b, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c, d, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e, f, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, g, h, 1.0f, 3);
    return w;
}

// ---- row arithmetic ---------------------------------------------------------

// Partial sum of eight bf16 values: four v_dot2_f32_bf16 against (1, 1),
// accumulated into `acc` in order.
__device__ __forceinline__ float sum_bf16x8(const uint4& v, float acc)
{
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), one, acc, false);
    return acc;
}

// Partial sum of squares of eight bf16 values: v_dot2_f32_bf16 of each pair
// with itself (the products are exact in fp32).
__device__ __forceinline__ float sumsq_bf16x8(const uint4& v, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, v.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, v.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, v.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, v.w), acc, false);
    return acc;
}

// 1 / sqrt(v): the hardware reciprocal square root (about 1 ulp) refined by
// one Newton step r + (r / 2) (1 - v r^2).  v = 0, +inf and NaN keep the
// hardware result (+inf, 0, NaN), as 1 / sqrt would give.
__device__ __forceinline__ float rsqrt_refined(float v)
{
    const float r = __builtin_amdgcn_rsqf(v);
    const float e = __builtin_fmaf(-(v * r), r, 1.0f);
    const float r1 = __builtin_fmaf(0.5f * r, e, r);
    return (v > 0.f && v < __builtin_inff()) ? r1 : r;
}

// max(0, |b[0]|, ..., |b[7]|) with NaN operands ignored (fmaxf), as a tree of
// three-operand maxima.
__device__ __forceinline__ float absmax8(const float b[8])
{
    const float m0 = fmaxf(fmaxf(fabsf(b[0]), fabsf(b[1])), fabsf(b[2]));
    const float m1 = fmaxf(fmaxf(fabsf(b[3]), fabsf(b[4])), fabsf(b[5]));
    const float m2 = fmaxf(fmaxf(fabsf(b[6]), fabsf(b[7])), 0.0f);
    return fmaxf(fmaxf(m0, m1), m2);
}

// ---- wave reductions ------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane gets the same bits.  DPP butterflies
// inside each row of 16 lanes (xor 1, xor 2, half-mirror, mirror: each lane
// adds the same two operands as its partner, so every lane of a row ends
// with the row's sum r), then two row broadcasts: rows 1 and 3 add the sums
// of rows 0 and 2 (row_bcast:15, rows 0 and 2 add zero), then rows 2 and 3
// add row 1's (row_bcast:31), so lane 63 holds (r3 + r2) + (r1 + r0), which
// one readlane hands to every lane.  IEEE addition is commutative, so this
// is bit for bit the (r0 + r1) + (r2 + r3) of four readlanes, in three
// instructions instead of nine.
__device__ __forceinline__ float wave_sum(float v)
{
    v = v + dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v = v + dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v = v + dpp<0x141>(v);   // row_half_mirror
    v = v + dpp<0x140>(v);   // row_mirror
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the waves of a workgroup (nwaves <= 16), same bits in every
// thread: wave sums, then the per-wave partials added in wave order.  `slot`
// is LDS for 16 floats; the trailing barrier is left to the caller's next
// use of the slot.
__device__ __forceinline__ float group_sum(float v, float* slot, int nwaves)
{
    v = wave_sum(v);
    if (nwaves == 1)
        return v;
    if ((threadIdx.x & (kWave - 1)) == 0)
        slot[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = slot[0];
    for (int k = 1; k < nwaves; ++k)
        r += slot[k];
    return r;
}

// Sum over `nwaves` consecutive waves starting at wave `first` of the
// workgroup (the waves that share one row), same bits in every thread of
// those waves.  Every thread of the workgroup must call it (it holds a
// barrier); `slot` is LDS with one float per wave of the workgroup.
__device__ __forceinline__ float subgroup_sum(float v, float* slot, int first, int nwaves)
{
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0)
        slot[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = slot[first];
    for (int k = 1; k < nwaves; ++k)
        r += slot[first + k];
    return r;
}

// Clamp eight values to the e4m3 range, NaN kept (as sat448).  Scaled
// normalized activations rarely pass 448, so one maximum over the eight
// (NaN ignored: NaN needs no clamp) decides whether the clamps run at all.
__device__ __forceinline__ void sat448x8(float (&v)[8])
{
    if (!(absmax8(v) > 448.0f))
        return;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        v[e] = sat448(v[e]);
}

// Max of two non-negative floats that are not NaN (block maxima from
// absmax8): their bit patterns order as unsigned integers.  One integer max
// takes the DPP operand directly, where fmaxf would also need a zero for the
// DPP move's inactive value and a canonicalizing max.
template <int CTRL>
__device__ __forceinline__ float max_nonneg_dpp(float v)
{
    const uint32_t b = __float_as_uint(v);
    const uint32_t p = __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false);
    return __uint_as_float(b > p ? b : p);
}

// Max over the four lanes of a quad (the lanes holding one 32-element MX
// block): quad_perm [1,0,3,2] then [2,3,0,1].  v >= 0, not NaN.
__device__ __forceinline__ float quad_max(float v)
{
    v = max_nonneg_dpp<0xB1>(v);
    return max_nonneg_dpp<0x4E>(v);
}

// Exponent E of an MX block scale 2^E (OCP Microscaling Formats v1.0):
// floor(log2(amax)) - emax, clamped to [-127, 127]; -127 when amax is 0 and
// 127 when it is infinite.  v_frexp_exp gives e with amax = m * 2^e, m in
// [0.5, 1), so floor(log2(amax)) = e - 1.
__device__ __forceinline__ int mx_scale_exp(float amax, int emax)
{
    const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - emax;
    const int E = amax > 0.f ? min(max(e, -127), 127) : -127;
    return amax == __builtin_inff() ? 127 : E;
}

// Max of a lane and its xor-1 partner (the two lanes holding one 16-element
// FP4 block).  v >= 0, not NaN.
__device__ __forceinline__ float pair_max(float v)
{
    return max_nonneg_dpp<0xB1>(v);
}

// e4m3 code of one float already in range (|v| <= 448), in the low byte:
// one v_cvt_pk_fp8_f32 (the other converted value and the upper half of the
// word are discarded).
__device__ __forceinline__ uint32_t e4m3_code1(float v)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, __float_as_int(v), false) & 0xFFu;
}

}  // namespace alnp
