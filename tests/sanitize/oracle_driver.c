/*
 * Every function of the CPU oracle run under the address and
 * undefined-behaviour sanitizers.  Each array is its own heap block of exactly
 * the size the function's contract states, so that a read or write one
 * element past any operand is reported.  Inputs cover ordinary values and the
 * degenerate rows the producers meet: all zeros (zero variance), a constant
 * row, the largest and smallest bf16 magnitudes, infinities and NaN, eps 0,
 * the last table chunk, and segment indices outside the table.  Exit status 0
 * when no sanitizer fired and the few exact facts checked below hold.
 */
#include "alnp_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int failures;

#define CHECK(cond)                                                 \
    do {                                                            \
        if (!(cond)) {                                              \
            printf("line %d: check failed: %s\n", __LINE__, #cond); \
            ++failures;                                             \
        }                                                           \
    } while (0)

/* One heap block of exactly n elements (n >= 1). */
static void* block(size_t n, size_t elem)
{
    void* p = malloc(n * elem);
    if (!p) {
        printf("out of memory\n");
        exit(2);
    }
    memset(p, 0xA5, n * elem);
    return p;
}
#define NEW(type, n) ((type*)block((size_t)(n), sizeof(type)))

static uint32_t lcg = 12345u;
static uint32_t next_u32(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return lcg;
}
static float uniform_pm(float a) /* uniform in [-a, a) */
{
    return a * ((float)(next_u32() >> 8) / 8388608.0f - 1.0f);
}

/* Row r of a (rows, dim) bf16 input: pattern r % 6. */
static void fill_x(uint16_t* x, int64_t rows, int64_t dim)
{
    static const uint16_t extremes[4] = {0x7F7F, 0xFF7F, 0x0001, 0x8001};
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < dim; ++j) {
            uint16_t v;
            switch (r % 6) {
            case 0: v = orc_f32_to_bf16(uniform_pm(3.0f)); break;
            case 1: v = 0x0000; break;                         /* zero variance */
            case 2: v = 0x3FC0; break;                         /* constant 1.5 */
            case 3: v = extremes[j % 4]; break;
            case 4: v = j == 0 ? 0x7F80 : orc_f32_to_bf16(uniform_pm(1.0f)); break; /* +inf */
            default: v = j == 1 ? 0x7FC0 : 0xFF80; break;      /* NaN, -inf */
            }
            x[r * dim + j] = v;
        }
}

static void fill_bf16(uint16_t* p, int64_t n, float a)
{
    for (int64_t i = 0; i < n; ++i)
        p[i] = orc_f32_to_bf16(uniform_pm(a));
}

static void fill_f32(float* p, int64_t n, float a)
{
    for (int64_t i = 0; i < n; ++i)
        p[i] = uniform_pm(a);
}

static void fill_u8(uint8_t* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        p[i] = (uint8_t)next_u32();
}

static void formats(void)
{
    for (int c = 0; c < 256; ++c) {
        double v = orc_e4m3_decode((uint8_t)c);
        if ((c & 0x7F) != 0x7F)
            CHECK(orc_e4m3_encode_sat((float)v) == c);
        double w = orc_e2m1_decode((uint8_t)(c & 0xF));
        CHECK(orc_e2m1_encode((float)w) == (c & 0xF));
        (void)orc_e8m0_decode((uint8_t)c);
    }
    for (uint32_t b = 0; b < 65536; ++b) {
        float f = orc_bf16_to_f32((uint16_t)b);
        uint16_t back = orc_f32_to_bf16(f);
        if (!isnan(f))
            CHECK(back == b);
    }
    static const float specials[] = {0.0f, -0.0f, 1e-45f, 3.4028235e38f, -3.4028235e38f,
                                     INFINITY, -INFINITY, NAN, 448.0f, 464.0f, 6.0f, 7.0f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        (void)orc_f32_to_bf16(specials[i]);
        (void)orc_e4m3_encode_sat(specials[i]);
        (void)orc_e2m1_encode(specials[i]);
        for (int emax = 2; emax <= 8; emax += 6)
            (void)orc_e8m0_scale(fabsf(specials[i]), emax);
    }
    enum { N = 37 };
    float* f = NEW(float, N);
    uint16_t* h = NEW(uint16_t, N);
    uint8_t* c8 = NEW(uint8_t, N);
    double* d = NEW(double, N);
    fill_f32(f, N, 500.0f);
    orc_f32_to_bf16_n(f, N, h);
    orc_bf16_to_f32_n(h, N, f);
    orc_e4m3_encode_sat_n(f, N, c8);
    orc_e4m3_decode_n(c8, N, d);
    orc_e2m1_encode_n(f, N, c8);
    orc_e2m1_decode_n(c8, N, d);
    free(f);
    free(h);
    free(c8);
    free(d);
}

static void fp8_forms(int64_t rows, int64_t dim, float eps)
{
    const int64_t n = rows * dim, chunks = 6;
    uint16_t* x = NEW(uint16_t, n);
    uint16_t* sc = NEW(uint16_t, n);
    uint16_t* sh = NEW(uint16_t, n);
    uint16_t* inv_s = NEW(uint16_t, dim);
    uint16_t* temb = NEW(uint16_t, rows * chunks * dim);
    float* table = NEW(float, chunks * dim);
    float* scf = NEW(float, n);
    float* shf = NEW(float, n);
    uint8_t* s8 = NEW(uint8_t, dim);
    uint8_t* h8 = NEW(uint8_t, dim);
    uint8_t* out = NEW(uint8_t, n);
    float* mean = NEW(float, rows);
    float* rstd = NEW(float, rows);
    float* y = NEW(float, n);
    fill_x(x, rows, dim);
    fill_bf16(sc, n, 0.5f);
    fill_bf16(sh, n, 0.5f);
    fill_bf16(inv_s, dim, 2.0f);
    fill_bf16(temb, rows * chunks * dim, 0.5f);
    fill_f32(table, chunks * dim, 0.5f);
    fill_f32(scf, n, 0.5f);
    fill_f32(shf, n, 0.5f);
    fill_u8(s8, dim);
    fill_u8(h8, dim);
    const float act = 0.05f;

    orc_ln_stats(x, rows, dim, eps, mean, rstd);
    CHECK(mean[1 % rows] == 0.0f || rows == 1);
    for (int with_opt = 0; with_opt < 2; ++with_opt) {
        float* m = with_opt ? mean : NULL;
        float* r = with_opt ? rstd : NULL;
        float* yy = with_opt ? y : NULL;
        orc_ln_fp8(x, act, eps, rows, dim, out, m, r, yy);
        orc_adaln_fp8_bcast(x, sc, sh, act, eps, rows, dim, out, m, r, yy);
        orc_adaln_fp8_ptok(x, sc, sh, act, eps, rows, dim, out, m, r, yy);
        orc_adaln_fp8_table(x, temb, table, chunks, 0, chunks - 1, act, eps, rows, dim, out, m,
                            r, yy);
        orc_adaln_fp8_f32ops(x, scf, shf, act, eps, rows, dim, out, m, r, yy);
        orc_adaln_fp8_modfp8(x, s8, h8, 0.5f, 0.25f, act, eps, rows, dim, out, m, r, yy);
        orc_awq_adaln_fp8(x, sc, sh, inv_s, act, eps, rows, dim, out, m, r, yy);
    }
    free(x), free(sc), free(sh), free(inv_s), free(temb), free(table), free(scf), free(shf);
    free(s8), free(h8), free(out), free(mean), free(rstd), free(y);
}

static void fp4_forms(int64_t rows, int64_t dim, float eps)
{
    const int64_t n = rows * dim, cols = dim / 16;
    uint16_t* x = NEW(uint16_t, n);
    uint16_t* sc = NEW(uint16_t, dim);
    uint16_t* sh = NEW(uint16_t, dim);
    uint8_t* s8 = NEW(uint8_t, dim);
    uint8_t* h8 = NEW(uint8_t, dim);
    uint8_t* packed = NEW(uint8_t, n / 2);
    uint8_t* sf = NEW(uint8_t, rows * cols);
    uint8_t* swz = NEW(uint8_t, orc_sf_swizzled_size(rows, cols));
    float* mean = NEW(float, rows);
    float* rstd = NEW(float, rows);
    float* b = NEW(float, n);
    uint8_t* codes = NEW(uint8_t, n);
    fill_x(x, rows, dim);
    fill_bf16(sc, dim, 0.5f);
    fill_bf16(sh, dim, 0.5f);
    fill_u8(s8, dim);
    fill_u8(h8, dim);
    for (int with_opt = 0; with_opt < 2; ++with_opt) {
        float* m = with_opt ? mean : NULL;
        float* r = with_opt ? rstd : NULL;
        float* bb = with_opt ? b : NULL;
        orc_ln_fp4(x, eps, rows, dim, packed, sf, m, r, bb);
        orc_adaln_fp4(x, sc, sh, eps, rows, dim, packed, sf, m, r, bb);
        orc_adaln_fp4_modfp8(x, s8, h8, 0.5f, 0.25f, eps, rows, dim, packed, sf, m, r, bb);
    }
    orc_sf_swizzle(sf, rows, cols, swz);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t off = orc_sf_swizzled_offset(r, c, cols);
            CHECK(off >= 0 && off < orc_sf_swizzled_size(rows, cols));
        }
    orc_fp4_block_quant_n(b, n / 16, codes, sf);
    orc_fp4_pack(codes, n, packed);
    free(x), free(sc), free(sh), free(s8), free(h8), free(packed), free(sf), free(swz);
    free(mean), free(rstd), free(b), free(codes);
}

static void mx_forms(int64_t rows, int64_t dim, float eps)
{
    const int64_t n = rows * dim, chunks = 6;
    uint16_t* x = NEW(uint16_t, n);
    uint16_t* sc = NEW(uint16_t, n);
    uint16_t* sh = NEW(uint16_t, n);
    uint16_t* temb = NEW(uint16_t, rows * chunks * dim);
    float* table = NEW(float, chunks * dim);
    uint8_t* out = NEW(uint8_t, n);
    uint8_t* packed = NEW(uint8_t, n / 2);
    uint8_t* scales = NEW(uint8_t, n / 32);
    float* mean = NEW(float, rows);
    float* rstd = NEW(float, rows);
    float* y = NEW(float, n);
    uint8_t* codes = NEW(uint8_t, n);
    fill_x(x, rows, dim);
    fill_bf16(sc, n, 0.5f);
    fill_bf16(sh, n, 0.5f);
    fill_bf16(temb, rows * chunks * dim, 0.5f);
    fill_f32(table, chunks * dim, 0.5f);
    for (int with_opt = 0; with_opt < 2; ++with_opt) {
        float* m = with_opt ? mean : NULL;
        float* r = with_opt ? rstd : NULL;
        float* yy = with_opt ? y : NULL;
        orc_adaln_mxfp4(x, NULL, NULL, eps, rows, dim, packed, scales, m, r, yy);
        orc_adaln_mxfp4(x, sc, sh, eps, rows, dim, packed, scales, m, r, yy);
        orc_adaln_mxfp8(x, NULL, NULL, 0, eps, rows, dim, out, scales, m, r, yy);
        orc_adaln_mxfp8(x, sc, sh, 0, eps, rows, dim, out, scales, m, r, yy);
        orc_adaln_mxfp8(x, sc, sh, 1, eps, rows, dim, out, scales, m, r, yy);
        orc_adaln_mxfp8_table(x, temb, table, chunks, chunks - 1, 0, eps, rows, dim, out, scales,
                              m, r, yy);
    }
    for (int fp4 = 0; fp4 < 2; ++fp4) {
        orc_mx_block_quant_n(y, n / 32, fp4, codes, scales);
        orc_mx_block_quant(y, 7, fp4, codes, scales); /* a short final block */
    }
    free(x), free(sc), free(sh), free(temb), free(table), free(out), free(packed), free(scales);
    free(mean), free(rstd), free(y), free(codes);
}

static void other_forms(int64_t rows, int64_t dim, float eps)
{
    const int64_t n = rows * dim, segments = 3;
    uint16_t* x = NEW(uint16_t, n);
    uint16_t* gate = NEW(uint16_t, n);
    uint16_t* proj = NEW(uint16_t, n);
    uint16_t* out = NEW(uint16_t, n);
    uint16_t* nrm = NEW(uint16_t, n);
    uint16_t* weight = NEW(uint16_t, dim);
    uint16_t* sc = NEW(uint16_t, segments * dim);
    uint16_t* sh = NEW(uint16_t, segments * dim);
    int32_t* seg = NEW(int32_t, rows);
    float* rstd = NEW(float, rows);
    float* params = NEW(float, rows * 6 * dim);
    float* mod = NEW(float, 6 * dim);
    uint16_t* planes = NEW(uint16_t, 6 * n);
    fill_x(x, rows, dim);
    fill_bf16(gate, n, 1.0f);
    fill_bf16(proj, n, 4.0f);
    fill_bf16(weight, dim, 1.5f);
    fill_bf16(sc, segments * dim, 0.5f);
    fill_bf16(sh, segments * dim, 0.5f);
    fill_f32(params, rows * 6 * dim, 1.0f);
    fill_f32(mod, 6 * dim, 1.0f);
    static const int32_t seg_cycle[5] = {0, 2, -1, 3, 1}; /* -1 and 3 lie outside */
    for (int64_t r = 0; r < rows; ++r)
        seg[r] = seg_cycle[r % 5];

    orc_gated_residual(x, gate, proj, rows, dim, 1, out);
    orc_gated_residual(x, gate, proj, rows, dim, rows, out);
    memcpy(out, x, (size_t)n * sizeof(uint16_t));
    orc_gated_residual(out, gate, proj, rows, dim, rows, out); /* in place */
    orc_modulation6(params, mod, rows, dim, planes);
    (void)orc_rms_rstd(x, dim, eps);
    orc_rms_modulate_seg(x, weight, sc, sh, seg, segments, eps, rows, dim, out, rstd, nrm);
    orc_rms_modulate_seg(x, NULL, sc, sh, seg, segments, eps, rows, dim, out, NULL, NULL);
    for (int64_t r = 0; r < rows; ++r)
        if (seg[r] < 0 || seg[r] >= segments)
            CHECK(out[r * dim] == 0x7FC0);
    orc_bf16_modulate_n(nrm, gate, proj, n, out);
    free(x), free(gate), free(proj), free(out), free(nrm), free(weight), free(sc), free(sh);
    free(seg), free(rstd), free(params), free(mod), free(planes);
}

int main(void)
{
    formats();
    static const int64_t row_counts[] = {1, 6, 7};
    static const int64_t dims[] = {32, 96, 160};
    static const float epss[] = {1e-6f, 0.0f};
    for (size_t a = 0; a < 3; ++a)
        for (size_t b = 0; b < 3; ++b)
            for (size_t c = 0; c < 2; ++c) {
                fp8_forms(row_counts[a], dims[b], epss[c]);
                fp4_forms(row_counts[a], dims[b], epss[c]);
                mx_forms(row_counts[a], dims[b], epss[c]);
                other_forms(row_counts[a], dims[b], epss[c]);
            }
    fp4_forms(129, 48, 1e-6f); /* scale rows past one 128-row tile, a ragged column tile */
    printf("%d failures\n", failures);
    return failures ? 1 : 0;
}
