/*
 * alnp_oracle.h -- plain, slow CPU oracle for the adaptive-LayerNorm producers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this code; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * source with the HIP path.
 *
 * Every function is the step-by-step definition of what the producers compute,
 * written with scalar loops, separately rounded fp32 operations (compiled with
 * -ffp-contract=off, no fast-math) and double-accumulated row statistics.
 * Conversions to bf16 / e4m3 / e2m1 are done by nearest-value search over the
 * format's finite values, not by bit tricks, so that a reader can check them
 * against the format definitions by eye.
 *
 * Sources (web pages; cited by title and section):
 *  - "adaptive-layernorm-producers" README, sections "Available Functions",
 *    "Tensor Contract", "Minimal Usage", "Validation".
 *  - "adaptive-layernorm-producers Benchmark Results", section
 *    "Six-way modulation producer".
 *  - h3-blackwell-runtime compare page: "NVFP4 Modulation Producer Fusion",
 *    subsection "Exactness Contract" (operation order (x*(scale+1))+shift);
 *    benchmarks/gb10-cute-p1-stream-a-summary.json, object
 *    "numerical_contract" (block scale amax/6, clamp at 448, E2M1
 *    round-to-nearest-even); benchmarks/gb10-cute-nvfp4-conversion-contract.json
 *    (low nibble first packing).
 *
 * bf16 values travel as uint16_t bit patterns, e4m3 and packed e2m1 as
 * uint8_t.  All arrays are contiguous, row-major.
 */
#ifndef ALNP_ORACLE_H
#define ALNP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);
double   orc_e4m3_decode(uint8_t code);
uint8_t  orc_e4m3_encode_sat(float v);
double   orc_e2m1_decode(uint8_t code);
uint8_t  orc_e2m1_encode(float v);

void orc_bf16_to_f32_n(const uint16_t* in, int64_t n, float* out);
void orc_f32_to_bf16_n(const float* in, int64_t n, uint16_t* out);
void orc_e4m3_decode_n(const uint8_t* in, int64_t n, double* out);
void orc_e4m3_encode_sat_n(const float* in, int64_t n, uint8_t* out);
void orc_e2m1_decode_n(const uint8_t* in, int64_t n, double* out);
void orc_e2m1_encode_n(const float* in, int64_t n, uint8_t* out);

/* ---- row statistics ---------------------------------------------------- */
void orc_ln_stats(const uint16_t* x, int64_t rows, int64_t dim, float eps,
                  float* mean, float* rstd);

/* ---- FP8 producers ----------------------------------------------------- */
/* y (nullable) receives the fp32 pre-quantization value, (rows, dim). */
void orc_ln_fp8(const uint16_t* x, float act_scale, float eps, int64_t rows,
                int64_t dim, uint8_t* out, float* mean, float* rstd, float* y);
void orc_adaln_fp8_bcast(const uint16_t* x, const uint16_t* scale,
                         const uint16_t* shift, float act_scale, float eps,
                         int64_t rows, int64_t dim, uint8_t* out, float* mean,
                         float* rstd, float* y);
void orc_adaln_fp8_ptok(const uint16_t* x, const uint16_t* scale,
                        const uint16_t* shift, float act_scale, float eps,
                        int64_t rows, int64_t dim, uint8_t* out, float* mean,
                        float* rstd, float* y);
void orc_adaln_fp8_table(const uint16_t* x, const uint16_t* temb,
                         const float* table, int64_t chunks, int64_t shift_idx,
                         int64_t scale_idx, float act_scale, float eps,
                         int64_t rows, int64_t dim, uint8_t* out, float* mean,
                         float* rstd, float* y);
/* Per-token core fed fp32 operands directly, (rows, dim) each. */
void orc_adaln_fp8_f32ops(const uint16_t* x, const float* scale,
                          const float* shift, float act_scale, float eps,
                          int64_t rows, int64_t dim, uint8_t* out, float* mean,
                          float* rstd, float* y);

/* FP8 variants of the README's function list.
 * modfp8: broadcast modulation stored as e4m3 (dim,) with fp32 dequantization
 * scalars: scale_j = e4m3(scale_fp8[j]) * scale_deq, same for shift.
 * awq: broadcast bf16 scale/shift plus a per-channel bf16 inv_s (dim,):
 * q = e4m3((y * inv_s[j]) * (1/act_scale)). */
void orc_adaln_fp8_modfp8(const uint16_t* x, const uint8_t* scale_fp8,
                          const uint8_t* shift_fp8, float scale_deq,
                          float shift_deq, float act_scale, float eps,
                          int64_t rows, int64_t dim, uint8_t* out, float* mean,
                          float* rstd, float* y);
void orc_awq_adaln_fp8(const uint16_t* x, const uint16_t* scale,
                       const uint16_t* shift, const uint16_t* inv_s,
                       float act_scale, float eps, int64_t rows, int64_t dim,
                       uint8_t* out, float* mean, float* rstd, float* y);

/* ---- FP4 producer ------------------------------------------------------ */
/* One block of 16 values -> 16 e2m1 codes (4-bit, sign in bit 3) and one
 * e4m3 block-scale code. */
void orc_fp4_block_quant(const float* b, uint8_t* codes, uint8_t* scale_code);
void orc_fp4_block_quant_n(const float* b, int64_t nblocks, uint8_t* codes,
                           uint8_t* scale_codes);
/* codes (n even, one per byte) -> n/2 bytes, element 2i in the low nibble. */
void orc_fp4_pack(const uint8_t* codes, int64_t n, uint8_t* packed);
/* b (nullable) receives the bf16-staged normalized row as fp32, (rows, dim). */
void orc_ln_fp4(const uint16_t* x, float eps, int64_t rows, int64_t dim,
                uint8_t* packed, uint8_t* sf, float* mean, float* rstd,
                float* b);

/* Broadcast AdaLN -> FP4: y = (xhat * (1 + scale)) + shift in fp32 as on the
 * FP8 path, then the same bf16 stage and block quantization as orc_ln_fp4.
 * b (nullable) receives the bf16-staged y as fp32. */
void orc_adaln_fp4(const uint16_t* x, const uint16_t* scale,
                   const uint16_t* shift, float eps, int64_t rows, int64_t dim,
                   uint8_t* packed, uint8_t* sf, float* mean, float* rstd,
                   float* b);
/* ada_layer_norm_quant_nvfp4_swizzled_modfp8 arithmetic with row-major scales:
 * operands e4m3(code) * deq (R9), then as orc_adaln_fp4. */
void orc_adaln_fp4_modfp8(const uint16_t* x, const uint8_t* scale_fp8,
                          const uint8_t* shift_fp8, float scale_deq, float shift_deq,
                          float eps, int64_t rows, int64_t dim, uint8_t* packed,
                          uint8_t* sf, float* mean, float* rstd, float* b);

/* 128x4 tiled ("swizzled") block-scale layout.  The pages name the layout
 * but do not define it; this is the tiled layout NVIDIA documents for
 * block-scaled GEMM operands (see the function comment).  The tests pin it
 * byte for byte to PyTorch's own implementation of that documented layout;
 * agreement with the pages' kernels' bytes cannot be checked.
 * cols = dim / 16 scale columns. */
int64_t orc_sf_swizzled_size(int64_t rows, int64_t cols);
int64_t orc_sf_swizzled_offset(int64_t r, int64_t c, int64_t cols);
/* Scatter a row-major (rows, cols) scale matrix into the swizzled buffer;
 * every byte the layout does not cover by a real scale (padding rows and
 * columns) is set to 0. */
void orc_sf_swizzle(const uint8_t* sf_rowmajor, int64_t rows, int64_t cols,
                    uint8_t* out);

/* ---- residual gate ----------------------------------------------------- */
/* out = bf16(residual + bf16(gate * proj)), elementwise over (rows, dim);
 * gate is (gate_rows, dim) with gate_rows 1 (broadcast) or rows (per token).
 * out may be residual itself. */
void orc_gated_residual(const uint16_t* residual, const uint16_t* gate,
                        const uint16_t* proj, int64_t rows, int64_t dim,
                        int64_t gate_rows, uint16_t* out);

/* ---- six-way modulation ------------------------------------------------ */
/* params (tokens, 6, dim) fp32, mod (6, dim) fp32 -> out (6, tokens, dim)
 * bf16 planes; plane k holds chunk k. */
void orc_modulation6(const float* params, const float* mod, int64_t tokens,
                     int64_t dim, uint16_t* out);

/* ---- RMSNorm with segment-selected modulation (R14) ----------------------- */
/* rstd of one row: 1/sqrt(sum(x^2)/dim + eps), double, rounded to fp32. */
float orc_rms_rstd(const uint16_t* xr, int64_t dim, float eps);
/* bf16((bf16(n * bf16(scale + 1))) + shift), each operation fp32 then bf16. */
uint16_t orc_bf16_modulate(uint16_t n, uint16_t scale, uint16_t shift);
void orc_bf16_modulate_n(const uint16_t* n, const uint16_t* scale, const uint16_t* shift,
                         int64_t count, uint16_t* out);
/* x (rows, dim) bf16; weight (dim,) bf16 or NULL; scale, shift (segments, dim)
 * bf16; seg (rows,) int32 -> out (rows, dim) bf16, rstd (rows,) (nullable),
 * n = the bf16 RMSNorm output (rows, dim) (nullable test hook). */
void orc_rms_modulate_seg(const uint16_t* x, const uint16_t* weight, const uint16_t* scale,
                          const uint16_t* shift, const int32_t* seg, int64_t segments,
                          float eps, int64_t rows, int64_t dim, uint16_t* out,
                          float* rstd_out, uint16_t* n_out);

/* ---- MX block formats (R15) ------------------------------------------------ */
/* E8M0 code of the shared scale for a block maximum and the element format's
 * emax (2 for E2M1, 8 for E4M3); value of a code (255 is NaN). */
uint8_t orc_e8m0_scale(float amax, int emax);
double  orc_e8m0_decode(uint8_t code);
/* n values -> n element codes (e2m1 when fp4, else e4m3) and one scale code. */
void orc_mx_block_quant(const float* v, int64_t n, int fp4, uint8_t* codes,
                        uint8_t* scale_code);
void orc_mx_block_quant_n(const float* v, int64_t nblocks, int fp4, uint8_t* codes,
                          uint8_t* scale_codes);
/* LN (scale = shift = NULL) or broadcast AdaLN -> bf16 stage -> MXFP4: packed
 * (rows, dim/2), scales (rows, dim/32) E8M0. */
void orc_adaln_mxfp4(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                     float eps, int64_t rows, int64_t dim, uint8_t* packed,
                     uint8_t* scales, float* mean, float* rstd, float* b);
/* LN, broadcast or per-token AdaLN -> MXFP8: out (rows, dim) e4m3, scales
 * (rows, dim/32) E8M0; y (nullable) receives the fp32 values quantized. */
void orc_adaln_mxfp8(const uint16_t* x, const uint16_t* scale, const uint16_t* shift,
                     int per_token, float eps, int64_t rows, int64_t dim, uint8_t* out,
                     uint8_t* scales, float* mean, float* rstd, float* y);
/* Table form (temb (rows, chunks, dim) bf16 + table (chunks, dim) fp32) -> MXFP8. */
void orc_adaln_mxfp8_table(const uint16_t* x, const uint16_t* temb, const float* table,
                           int64_t chunks, int64_t shift_idx, int64_t scale_idx, float eps,
                           int64_t rows, int64_t dim, uint8_t* out, uint8_t* scales,
                           float* mean, float* rstd, float* y);

#ifdef __cplusplus
}
#endif
#endif
