/*
 * alnp_oracle.c -- plain CPU oracle for the adaptive-LayerNorm producers.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  Shares no code
 * with the HIP library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * On x86-64 float arithmetic is SSE single precision, so every fp32
 * expression below is one correctly rounded IEEE operation.
 *
 * Readings of points the pages leave open (each repeated where it is used):
 *  R1  variance is the biased (1/dim) two-pass variance, eps inside the sqrt
 *      (standard LayerNorm definition; the README only says "LayerNorm ...
 *      no affine" with eps = 1e-5).
 *  R2  modulation is ((xhat * (scale + 1)) + shift) in fp32, each operation
 *      rounded separately, no bf16 rounding on the FP8 path (h3 page,
 *      "Exactness Contract", gives the operation order).
 *  R3  act_scale is a dequantization scale: q = e4m3(y * (1/act_scale)),
 *      the reciprocal taken once per call in fp32.
 *  R4  FP8 quantization saturates: |v| >= 448 and +-inf map to +-448; NaN
 *      maps to the e4m3 NaN code with the sign kept.
 *  R5  table form: operand = bf16 temb chunk + fp32 table row, one fp32 add,
 *      not rounded to bf16.
 *  R6  FP4: normalized row staged through bf16 (README "Validation": staged
 *      BF16-norm); per 16-element block s = e4m3_sat(amax / 6) with global
 *      scale 1; codes = e2m1_rtne(b * (1/s)), IEEE division for both; an
 *      all-zero scale gives all-zero codes.
 *  R7  six-way: out_k = bf16_rtne(params[:, k, :] + mod[k, :]), chunk k to
 *      output k.
 *  R8  NaN inputs to e2m1 are outside the contract; they encode as a zero
 *      magnitude with the sign kept.
 *  R9  modfp8 (README "Available Functions", "Tensor Contract": e4m3 (dim,)
 *      scale/shift with fp32 dequantization scalars): the operand is the e4m3
 *      value times its dequantization scalar, one fp32 multiplication.
 *  R10 AWQ (README: per-channel bf16 inv_s (dim,)): activation-aware smoothing
 *      multiplies the modulated value by inv_s[j] before the static-scale
 *      quantization: q = e4m3((y * inv_s[j]) * (1/act_scale)), each
 *      multiplication rounded.
 *  R11 AdaLN -> FP4: the FP8 path's fp32 modulation, then the LN -> FP4 bf16
 *      stage and block quantization (the pages fix the staging only for the
 *      LN entry; the plainest reading applies it to the modulated value).
 *  R12 Swizzled scales: NVIDIA's documented 128x4 tiled layout for block
 *      scale factors (the pages give only its name).  Pinned against
 *      PyTorch's own implementation of that documented layout.
 *  R13 Residual gate (h3 page, the residual-gate epilogue's numerical
 *      program: bf16 GEMM output, gate multiplication with its bf16
 *      boundary, bf16 residual added, final bf16 rounding):
 *      out = bf16(residual + bf16(gate * proj)), fp32 arithmetic.
 *  R14 RMSNorm modulation (RL-Kernel norm_modulate page: modulated RMSNorm
 *      with a weight and index-selected scale/shift rows; h3 page, "NVFP4
 *      Modulation Producer Fusion", "Exactness Contract": segment-specific
 *      scale and shift, (x * (scale + 1)) + shift order, BF16 rounding):
 *      rstd = 1/sqrt(sum(x^2)/dim + eps), mean of squares with no centring,
 *      in double, rounded once to fp32.  The RMSNorm output is a bf16
 *      tensor: n = bf16((x * rstd) * w), two fp32 operations (w = 1 when
 *      absent).  Each modulation operation is a bf16 tensor operation,
 *      computed in fp32 and rounded once: t = bf16(scale + 1),
 *      u = bf16(n * t), y = bf16(u + shift).  scale and shift are rows seg[r]
 *      of (segments, dim) tables; a row whose index is outside [0, segments)
 *      is all NaN (0x7FC0).
 *  R15 MX block formats (not on the pages: the OCP Microscaling Formats (MX)
 *      v1.0 specification, its conversion of a vector to an MX block; the
 *      block format gfx950's scaled matrix instructions read).  32
 *      consecutive elements of a row share an E8M0 scale X = 2^E with
 *      E = floor(log2(amax)) - emax (emax = 2 for E2M1, 8 for E4M3), clamped
 *      to [-127, 127] and stored as E + 127; each element is v / X rounded to
 *      nearest even and saturated at the element format's largest normal.
 *      amax ignores NaN like the FP4 block maximum; a block without a
 *      non-zero value gets E = -127 (code 0), an infinite amax E = 127.
 *      MXFP4 quantizes the bf16-staged value of R6/R11; MXFP8 the fp32 y of
 *      R2, with no static act_scale (the block scale takes its place).
 */
#include "alnp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16: the upper 16 bits of an IEEE binary32.                              */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of a bf16 pattern as a double, with the infinity pattern standing for
 * 2^128 (the value the next pattern would have with an unbounded exponent),
 * which is what IEEE round-to-nearest compares against at overflow. */
static double bf16_value_for_rounding(uint16_t b)
{
    if ((b & 0x7FFF) == 0x7F80)
        return (b & 0x8000) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    return (double)orc_bf16_to_f32(b);
}

/* Round-to-nearest-even fp32 -> bf16 by comparing distances to the two
 * bf16 neighbours (truncation toward zero, and the next value away from
 * zero).  NaN keeps its sign and becomes quiet. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040);
    if (isinf(f))
        return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1);
    double v = (double)f;
    double dlo = fabs(v - bf16_value_for_rounding(lo));
    double dhi = fabs(bf16_value_for_rounding(hi) - v);
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1) ? hi : lo;
}

/* ------------------------------------------------------------------------ */
/* e4m3fn (OCP FP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no        */
/* infinities; S.1111.111 is NaN; largest finite magnitude 448.              */
/* ------------------------------------------------------------------------ */

static double e4m3_magnitude(int c) /* c in 0..126 */
{
    int e = c >> 3, m = c & 7;
    if (e == 0)
        return ldexp((double)m, -9);          /* subnormal: m/8 * 2^-6 */
    return ldexp((double)(8 + m), e - 10);    /* (1 + m/8) * 2^(e-7)    */
}

double orc_e4m3_decode(uint8_t code)
{
    int c = code & 0x7F;
    double s = (code & 0x80) ? -1.0 : 1.0;
    if (c == 0x7F)
        return s * NAN;
    return s * e4m3_magnitude(c);
}

/* Saturating round-to-nearest-even encode (readings R4). */
uint8_t orc_e4m3_encode_sat(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bestd = a;
    for (int c = 1; c <= 126; ++c) {
        double d = fabs(a - e4m3_magnitude(c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------------ */
/* e2m1 (FP4): 1 sign, 2 exponent, 1 mantissa bit; magnitudes                */
/* {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN or infinity.                         */
/* ------------------------------------------------------------------------ */

static const double kE2m1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t code)
{
    double m = kE2m1Mag[code & 7];
    return (code & 8) ? -m : m;
}

/* Round-to-nearest-even; magnitudes of 6 and above (infinity included)
 * saturate at 6; sign kept, so small negatives give code 8 (-0). */
uint8_t orc_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    if (isnan(v))
        return sign; /* R8 */
    double a = fabs((double)v);
    if (a >= 6.0)
        return (uint8_t)(sign | 7);
    int best = 0;
    double bestd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - kE2m1Mag[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

void orc_bf16_to_f32_n(const uint16_t* in, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_to_f32(in[i]);
}
void orc_f32_to_bf16_n(const float* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(in[i]);
}
void orc_e4m3_decode_n(const uint8_t* in, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(in[i]);
}
void orc_e4m3_encode_sat_n(const float* in, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode_sat(in[i]);
}
void orc_e2m1_decode_n(const uint8_t* in, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_decode(in[i]);
}
void orc_e2m1_encode_n(const float* in, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_encode(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Row statistics (R1): mean and biased variance accumulated in double,       */
/* rstd = 1/sqrt(var + eps) in double, each rounded once to fp32.            */
/* ------------------------------------------------------------------------ */

static void row_stats(const uint16_t* xr, int64_t dim, float eps, float* mean,
                      float* rstd)
{
    double s = 0.0;
    for (int64_t j = 0; j < dim; ++j)
        s += (double)orc_bf16_to_f32(xr[j]);
    double mu = s / (double)dim;
    double q = 0.0;
    for (int64_t j = 0; j < dim; ++j) {
        double d = (double)orc_bf16_to_f32(xr[j]) - mu;
        q += d * d;
    }
    double var = q / (double)dim;
    *mean = (float)mu;
    *rstd = (float)(1.0 / sqrt(var + (double)eps));
}

void orc_ln_stats(const uint16_t* x, int64_t rows, int64_t dim, float eps,
                  float* mean, float* rstd)
{
    for (int64_t r = 0; r < rows; ++r)
        row_stats(x + r * dim, dim, eps, &mean[r], &rstd[r]);
}

/* ------------------------------------------------------------------------ */
/* FP8 producers.  One row: normalize, modulate (R2), scale (R3), quantize    */
/* (R4).  sc/sh are the row's fp32 modulation operands.                       */
/* ------------------------------------------------------------------------ */

static void row_adaln_fp8(const uint16_t* xr, const float* sc, const float* sh,
                          int64_t dim, float inv_act, float mean, float rstd,
                          uint8_t* out, float* y)
{
    for (int64_t j = 0; j < dim; ++j) {
        float xj = orc_bf16_to_f32(xr[j]);
        float centered = xj - mean;
        float xhat = centered * rstd;
        float t = 1.0f + sc[j];
        float u = xhat * t;
        float yj = u + sh[j];
        if (y)
            y[j] = yj;
        out[j] = orc_e4m3_encode_sat(yj * inv_act);
    }
}

/* The reciprocal of the dequantization scale, once per call (R3). */
static float reciprocal(float act_scale) { return 1.0f / act_scale; }

void orc_adaln_fp8_f32ops(const uint16_t* x, const float* scale,
                          const float* shift, float act_scale, float eps,
                          int64_t rows, int64_t dim, uint8_t* out, float* mean,
                          float* rstd, float* y)
{
    float inv = reciprocal(act_scale);
    for (int64_t r = 0; r < rows; ++r) {
        float mu, rs;
        row_stats(x + r * dim, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        row_adaln_fp8(x + r * dim, scale + r * dim, shift + r * dim, dim, inv,
                      mu, rs, out + r * dim, y ? y + r * dim : 0);
    }
}

/* The forms below differ only in where a row's fp32 operands come from:
 * each builds one row's operands into a scratch buffer, then runs the row
 * core on it. */
static void run_rows(const uint16_t* x, int64_t rows, int64_t dim, float inv,
                     float eps, uint8_t* out, float* mean, float* rstd,
                     float* y, int form, const uint16_t* scale,
                     const uint16_t* shift, const uint16_t* temb,
                     const float* table, int64_t chunks, int64_t shift_idx,
                     int64_t scale_idx)
{
    float* sc = (float*)malloc((size_t)dim * sizeof(float));
    float* sh = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        for (int64_t j = 0; j < dim; ++j) {
            switch (form) {
            case 0: /* LN only: modulation off */
                sc[j] = 0.0f;
                sh[j] = 0.0f;
                break;
            case 1: /* broadcast (dim,) */
                sc[j] = orc_bf16_to_f32(scale[j]);
                sh[j] = orc_bf16_to_f32(shift[j]);
                break;
            case 2: /* per-token (rows, dim) */
                sc[j] = orc_bf16_to_f32(scale[r * dim + j]);
                sh[j] = orc_bf16_to_f32(shift[r * dim + j]);
                break;
            default: /* table: temb (rows, chunks, dim) + table (chunks, dim), R5 */
                sc[j] = orc_bf16_to_f32(temb[(r * chunks + scale_idx) * dim + j]) +
                        table[scale_idx * dim + j];
                sh[j] = orc_bf16_to_f32(temb[(r * chunks + shift_idx) * dim + j]) +
                        table[shift_idx * dim + j];
                break;
            }
        }
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        row_adaln_fp8(xr, sc, sh, dim, inv, mu, rs, out + r * dim,
                      y ? y + r * dim : 0);
    }
    free(sc);
    free(sh);
}

void orc_ln_fp8(const uint16_t* x, float act_scale, float eps, int64_t rows,
                int64_t dim, uint8_t* out, float* mean, float* rstd, float* y)
{
    run_rows(x, rows, dim, reciprocal(act_scale), eps, out, mean, rstd, y, 0,
             0, 0, 0, 0, 0, 0, 0);
}

void orc_adaln_fp8_bcast(const uint16_t* x, const uint16_t* scale,
                         const uint16_t* shift, float act_scale, float eps,
                         int64_t rows, int64_t dim, uint8_t* out, float* mean,
                         float* rstd, float* y)
{
    run_rows(x, rows, dim, reciprocal(act_scale), eps, out, mean, rstd, y, 1,
             scale, shift, 0, 0, 0, 0, 0);
}

void orc_adaln_fp8_ptok(const uint16_t* x, const uint16_t* scale,
                        const uint16_t* shift, float act_scale, float eps,
                        int64_t rows, int64_t dim, uint8_t* out, float* mean,
                        float* rstd, float* y)
{
    run_rows(x, rows, dim, reciprocal(act_scale), eps, out, mean, rstd, y, 2,
             scale, shift, 0, 0, 0, 0, 0);
}

void orc_adaln_fp8_table(const uint16_t* x, const uint16_t* temb,
                         const float* table, int64_t chunks, int64_t shift_idx,
                         int64_t scale_idx, float act_scale, float eps,
                         int64_t rows, int64_t dim, uint8_t* out, float* mean,
                         float* rstd, float* y)
{
    run_rows(x, rows, dim, reciprocal(act_scale), eps, out, mean, rstd, y, 3,
             0, 0, temb, table, chunks, shift_idx, scale_idx);
}

/* modfp8 (R9): e4m3 broadcast operands times fp32 dequantization scalars. */
void orc_adaln_fp8_modfp8(const uint16_t* x, const uint8_t* scale_fp8,
                          const uint8_t* shift_fp8, float scale_deq,
                          float shift_deq, float act_scale, float eps,
                          int64_t rows, int64_t dim, uint8_t* out, float* mean,
                          float* rstd, float* y)
{
    float* sc = (float*)malloc((size_t)dim * sizeof(float));
    float* sh = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t j = 0; j < dim; ++j) {
        sc[j] = (float)orc_e4m3_decode(scale_fp8[j]) * scale_deq;
        sh[j] = (float)orc_e4m3_decode(shift_fp8[j]) * shift_deq;
    }
    float inv = reciprocal(act_scale);
    for (int64_t r = 0; r < rows; ++r) {
        float mu, rs;
        row_stats(x + r * dim, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        row_adaln_fp8(x + r * dim, sc, sh, dim, inv, mu, rs, out + r * dim,
                      y ? y + r * dim : 0);
    }
    free(sc);
    free(sh);
}

/* AWQ (R10): per-channel inv_s multiplication before the quantization. */
void orc_awq_adaln_fp8(const uint16_t* x, const uint16_t* scale,
                       const uint16_t* shift, const uint16_t* inv_s,
                       float act_scale, float eps, int64_t rows, int64_t dim,
                       uint8_t* out, float* mean, float* rstd, float* y)
{
    float inv = reciprocal(act_scale);
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            float t = 1.0f + orc_bf16_to_f32(scale[j]);
            float u = xhat * t;
            float yj = u + orc_bf16_to_f32(shift[j]);
            if (y)
                y[r * dim + j] = yj;
            float smoothed = yj * orc_bf16_to_f32(inv_s[j]);
            out[r * dim + j] = orc_e4m3_encode_sat(smoothed * inv);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* FP4 producer (R6).                                                         */
/* ------------------------------------------------------------------------ */

void orc_fp4_block_quant(const float* b, uint8_t* codes, uint8_t* scale_code)
{
    float amax = 0.0f;
    for (int j = 0; j < 16; ++j)
        amax = fmaxf(amax, fabsf(b[j]));
    float target = amax / 6.0f;
    uint8_t sc = orc_e4m3_encode_sat(target);
    float s = (float)orc_e4m3_decode(sc);
    *scale_code = sc;
    if (s == 0.0f) {
        for (int j = 0; j < 16; ++j)
            codes[j] = 0;
        return;
    }
    float enc = 1.0f / s;
    for (int j = 0; j < 16; ++j)
        codes[j] = orc_e2m1_encode(b[j] * enc);
}

void orc_fp4_block_quant_n(const float* b, int64_t nblocks, uint8_t* codes,
                           uint8_t* scale_codes)
{
    for (int64_t k = 0; k < nblocks; ++k)
        orc_fp4_block_quant(b + 16 * k, codes + 16 * k, scale_codes + k);
}

void orc_fp4_pack(const uint8_t* codes, int64_t n, uint8_t* packed)
{
    for (int64_t i = 0; i < n / 2; ++i)
        packed[i] = (uint8_t)((codes[2 * i] & 0xF) | ((codes[2 * i + 1] & 0xF) << 4));
}

void orc_ln_fp4(const uint16_t* x, float eps, int64_t rows, int64_t dim,
                uint8_t* packed, uint8_t* sf, float* mean, float* rstd,
                float* b)
{
    float* staged = (float*)malloc((size_t)dim * sizeof(float));
    uint8_t* codes = (uint8_t*)malloc((size_t)dim);
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            staged[j] = orc_bf16_to_f32(orc_f32_to_bf16(xhat));
            if (b)
                b[r * dim + j] = staged[j];
        }
        for (int64_t k = 0; k < dim / 16; ++k)
            orc_fp4_block_quant(staged + 16 * k, codes + 16 * k,
                                &sf[r * (dim / 16) + k]);
        orc_fp4_pack(codes, dim, packed + r * (dim / 2));
    }
    free(staged);
    free(codes);
}

/* AdaLN -> FP4 with fp32 modulation operands (R11): the FP8 path's fp32
 * modulation, then the bf16 stage and the block quantization. */
static void adaln_fp4_f32ops(const uint16_t* x, const float* sc, const float* sh, float eps,
                             int64_t rows, int64_t dim, uint8_t* packed, uint8_t* sf,
                             float* mean, float* rstd, float* b)
{
    float* staged = (float*)malloc((size_t)dim * sizeof(float));
    uint8_t* codes = (uint8_t*)malloc((size_t)dim);
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            float t = 1.0f + sc[j];
            float u = xhat * t;
            float yj = u + sh[j];
            staged[j] = orc_bf16_to_f32(orc_f32_to_bf16(yj));
            if (b)
                b[r * dim + j] = staged[j];
        }
        for (int64_t k = 0; k < dim / 16; ++k)
            orc_fp4_block_quant(staged + 16 * k, codes + 16 * k,
                                &sf[r * (dim / 16) + k]);
        orc_fp4_pack(codes, dim, packed + r * (dim / 2));
    }
    free(staged);
    free(codes);
}

/* Broadcast bf16 operands (exact in fp32). */
void orc_adaln_fp4(const uint16_t* x, const uint16_t* scale,
                   const uint16_t* shift, float eps, int64_t rows, int64_t dim,
                   uint8_t* packed, uint8_t* sf, float* mean, float* rstd,
                   float* b)
{
    float* sc = (float*)malloc((size_t)dim * sizeof(float));
    float* sh = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t j = 0; j < dim; ++j) {
        sc[j] = orc_bf16_to_f32(scale[j]);
        sh[j] = orc_bf16_to_f32(shift[j]);
    }
    adaln_fp4_f32ops(x, sc, sh, eps, rows, dim, packed, sf, mean, rstd, b);
    free(sc);
    free(sh);
}

/* modfp8 operands (R9) on the AdaLN -> FP4 path (R11): e4m3 value times its
 * dequantization scalar, one fp32 multiplication. */
void orc_adaln_fp4_modfp8(const uint16_t* x, const uint8_t* scale_fp8,
                          const uint8_t* shift_fp8, float scale_deq, float shift_deq,
                          float eps, int64_t rows, int64_t dim, uint8_t* packed,
                          uint8_t* sf, float* mean, float* rstd, float* b)
{
    float* sc = (float*)malloc((size_t)dim * sizeof(float));
    float* sh = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t j = 0; j < dim; ++j) {
        sc[j] = (float)orc_e4m3_decode(scale_fp8[j]) * scale_deq;
        sh[j] = (float)orc_e4m3_decode(shift_fp8[j]) * shift_deq;
    }
    adaln_fp4_f32ops(x, sc, sh, eps, rows, dim, packed, sf, mean, rstd, b);
    free(sc);
    free(sh);
}

/* ------------------------------------------------------------------------ */
/* 128x4 tiled block-scale layout (R12).                                       */
/* The (rows, cols) scale matrix is cut into tiles of 128 rows x 4 columns,   */
/* stored one after another (tile row-major: all column tiles of the first    */
/* 128 rows, then the next 128 rows), 512 bytes each.  Inside a tile the      */
/* byte for (r, c) sits at (r mod 32) * 16 + (r div 32) * 4 + c: the four     */
/* 32-row groups are interleaved so that one 16-byte unit holds the four      */
/* column scales of rows r, r + 32, r + 64 and r + 96.                        */
/* ------------------------------------------------------------------------ */

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t orc_sf_swizzled_size(int64_t rows, int64_t cols)
{
    return round_up(rows, 128) * round_up(cols, 4);
}

int64_t orc_sf_swizzled_offset(int64_t r, int64_t c, int64_t cols)
{
    int64_t col_tiles = round_up(cols, 4) / 4;
    int64_t tile = (r / 128) * col_tiles + (c / 4);
    int64_t rr = r % 128, cc = c % 4;
    return tile * 512 + (rr % 32) * 16 + (rr / 32) * 4 + cc;
}

void orc_sf_swizzle(const uint8_t* sf_rowmajor, int64_t rows, int64_t cols,
                    uint8_t* out)
{
    memset(out, 0, (size_t)orc_sf_swizzled_size(rows, cols));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[orc_sf_swizzled_offset(r, c, cols)] = sf_rowmajor[r * cols + c];
}

/* ------------------------------------------------------------------------ */
/* Residual gate (R13).                                                       */
/* ------------------------------------------------------------------------ */

void orc_gated_residual(const uint16_t* residual, const uint16_t* gate,
                        const uint16_t* proj, int64_t rows, int64_t dim,
                        int64_t gate_rows, uint16_t* out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* g = gate + (gate_rows == 1 ? 0 : r * dim);
        for (int64_t j = 0; j < dim; ++j) {
            float gated = orc_bf16_to_f32(g[j]) * orc_bf16_to_f32(proj[r * dim + j]);
            float gated_bf16 = orc_bf16_to_f32(orc_f32_to_bf16(gated));
            float sum = orc_bf16_to_f32(residual[r * dim + j]) + gated_bf16;
            out[r * dim + j] = orc_f32_to_bf16(sum);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Six-way modulation (R7).                                                   */
/* ------------------------------------------------------------------------ */

void orc_modulation6(const float* params, const float* mod, int64_t tokens,
                     int64_t dim, uint16_t* out)
{
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t k = 0; k < 6; ++k)
            for (int64_t j = 0; j < dim; ++j) {
                float s = params[(t * 6 + k) * dim + j] + mod[k * dim + j];
                out[(k * tokens + t) * dim + j] = orc_f32_to_bf16(s);
            }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm with segment-selected modulation (R14).                            */
/* ------------------------------------------------------------------------ */

float orc_rms_rstd(const uint16_t* xr, int64_t dim, float eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < dim; ++j) {
        double v = (double)orc_bf16_to_f32(xr[j]);
        ss += v * v;
    }
    return (float)(1.0 / sqrt(ss / (double)dim + (double)eps));
}

uint16_t orc_bf16_modulate(uint16_t n, uint16_t scale, uint16_t shift)
{
    float t = orc_bf16_to_f32(orc_f32_to_bf16(orc_bf16_to_f32(scale) + 1.0f));
    float u = orc_bf16_to_f32(orc_f32_to_bf16(orc_bf16_to_f32(n) * t));
    return orc_f32_to_bf16(u + orc_bf16_to_f32(shift));
}

void orc_bf16_modulate_n(const uint16_t* n, const uint16_t* scale, const uint16_t* shift,
                         int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = orc_bf16_modulate(n[i], scale[i], shift[i]);
}

void orc_rms_modulate_seg(const uint16_t* x, const uint16_t* weight, const uint16_t* scale,
                          const uint16_t* shift, const int32_t* seg, int64_t segments,
                          float eps, int64_t rows, int64_t dim, uint16_t* out,
                          float* rstd_out, uint16_t* n_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float rstd = orc_rms_rstd(xr, dim, eps);
        if (rstd_out)
            rstd_out[r] = rstd;
        int64_t s = seg[r];
        int in_range = s >= 0 && s < segments;
        for (int64_t j = 0; j < dim; ++j) {
            float v = orc_bf16_to_f32(xr[j]) * rstd;
            if (weight)
                v = v * orc_bf16_to_f32(weight[j]);
            uint16_t n = orc_f32_to_bf16(v);
            if (n_out)
                n_out[r * dim + j] = n;
            out[r * dim + j] = in_range ? orc_bf16_modulate(n, scale[s * dim + j], shift[s * dim + j])
                                        : (uint16_t)0x7FC0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MX block formats (R15).                                                    */
/* ------------------------------------------------------------------------ */

uint8_t orc_e8m0_scale(float amax, int emax)
{
    if (isinf(amax))
        return 254;
    if (!(amax > 0.0f))
        return 0;
    int e;
    frexp((double)amax, &e); /* amax = m * 2^e with m in [0.5, 1): floor(log2) = e - 1 */
    int E = (e - 1) - emax;
    if (E < -127)
        E = -127;
    if (E > 127)
        E = 127;
    return (uint8_t)(E + 127);
}

double orc_e8m0_decode(uint8_t code)
{
    return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

void orc_mx_block_quant(const float* v, int64_t n, int fp4, uint8_t* codes,
                        uint8_t* scale_code)
{
    float amax = 0.0f;
    for (int64_t j = 0; j < n; ++j)
        amax = fmaxf(amax, fabsf(v[j]));
    uint8_t sc = orc_e8m0_scale(amax, fp4 ? 2 : 8);
    *scale_code = sc;
    int E = (int)sc - 127;
    for (int64_t j = 0; j < n; ++j) {
        /* Division by a power of two: exact in double; the float rounding can
         * only touch values far below every non-zero code. */
        float q = (float)ldexp((double)v[j], -E);
        codes[j] = fp4 ? orc_e2m1_encode(q) : orc_e4m3_encode_sat(q);
    }
}

void orc_mx_block_quant_n(const float* v, int64_t nblocks, int fp4, uint8_t* codes,
                          uint8_t* scale_codes)
{
    for (int64_t k = 0; k < nblocks; ++k)
        orc_mx_block_quant(v + 32 * k, 32, fp4, codes + 32 * k, scale_codes + k);
}

/* LayerNorm or broadcast AdaLN (scale/shift non-NULL) -> bf16 stage -> MXFP4. */
void orc_adaln_mxfp4(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                     float eps, int64_t rows, int64_t dim, uint8_t* packed,
                     uint8_t* scales, float* mean, float* rstd, float* b)
{
    float* staged = (float*)malloc((size_t)dim * sizeof(float));
    uint8_t* codes = (uint8_t*)malloc((size_t)dim);
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            float yj = xhat;
            if (scale) {
                float t = 1.0f + orc_bf16_to_f32(scale[j]);
                float u = xhat * t;
                yj = u + orc_bf16_to_f32(shift[j]);
            }
            staged[j] = orc_bf16_to_f32(orc_f32_to_bf16(yj));
            if (b)
                b[r * dim + j] = staged[j];
        }
        orc_mx_block_quant_n(staged, dim / 32, 1, codes, scales + r * (dim / 32));
        orc_fp4_pack(codes, dim, packed + r * (dim / 2));
    }
    free(staged);
    free(codes);
}

/* LayerNorm, broadcast or per-token AdaLN -> MXFP8: the fp32 y of R2. */
void orc_adaln_mxfp8(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                     int per_token, float eps, int64_t rows, int64_t dim, uint8_t* out,
                     uint8_t* scales, float* mean, float* rstd, float* y)
{
    float* yr = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        const uint16_t* scr = scale ? scale + (per_token ? r * dim : 0) : 0;
        const uint16_t* shr = shift ? shift + (per_token ? r * dim : 0) : 0;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            float t = 1.0f + (scr ? orc_bf16_to_f32(scr[j]) : 0.0f);
            float u = xhat * t;
            yr[j] = u + (shr ? orc_bf16_to_f32(shr[j]) : 0.0f);
            if (y)
                y[r * dim + j] = yr[j];
        }
        orc_mx_block_quant_n(yr, dim / 32, 0, out + r * dim, scales + r * (dim / 32));
    }
    free(yr);
}

/* Table form -> MXFP8: operands temb chunk + fp32 table row (R5), the fp32 y
 * of R2, then MX blocks (R15). */
void orc_adaln_mxfp8_table(const uint16_t* x, const uint16_t* temb, const float* table,
                           int64_t chunks, int64_t shift_idx, int64_t scale_idx, float eps,
                           int64_t rows, int64_t dim, uint8_t* out, uint8_t* scales,
                           float* mean, float* rstd, float* y)
{
    float* yr = (float*)malloc((size_t)dim * sizeof(float));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * dim;
        float mu, rs;
        row_stats(xr, dim, eps, &mu, &rs);
        if (mean)
            mean[r] = mu;
        if (rstd)
            rstd[r] = rs;
        for (int64_t j = 0; j < dim; ++j) {
            float sc = orc_bf16_to_f32(temb[(r * chunks + scale_idx) * dim + j]) +
                       table[scale_idx * dim + j];
            float sh = orc_bf16_to_f32(temb[(r * chunks + shift_idx) * dim + j]) +
                       table[shift_idx * dim + j];
            float centered = orc_bf16_to_f32(xr[j]) - mu;
            float xhat = centered * rs;
            float t = 1.0f + sc;
            float u = xhat * t;
            yr[j] = u + sh;
            if (y)
                y[r * dim + j] = yr[j];
        }
        orc_mx_block_quant_n(yr, dim / 32, 0, out + r * dim, scales + r * (dim / 32));
    }
    free(yr);
}
