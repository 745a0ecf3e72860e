/*
 * alnp.h -- C ABI of the adaptive-LayerNorm producers for AMD MI355X (gfx950).
 *
 * The producers fuse the work in front of a low-precision GEMM in a DiT /
 * Wan-style block: per row of a bf16 (rows, dim) activation, LayerNorm
 * without affine weights, the DiT modulation xhat * (1 + scale) + shift, and
 * quantization to FP8 e4m3 (static scale) or FP4 e2m1 (e4m3 scale per 16
 * elements); plus the six-way modulation producer.  Sources: the
 * "adaptive-layernorm-producers" README ("Available Functions", "Tensor
 * Contract", "Minimal Usage") and its "Benchmark Results" page.
 *
 * Conventions shared by every entry point
 *  - Types: bf16 tensors are passed as uint16_t bit patterns, e4m3 and
 *    packed e2m1 as uint8_t, fp32 as float.  All tensors are contiguous and
 *    row-major; pointers are DEVICE pointers unless a parameter says
 *    otherwise.
 *  - Ownership: the caller allocates every buffer and keeps it alive until
 *    the work queued on `stream` has finished.  The library never allocates,
 *    frees or synchronizes; each call validates its arguments on the host,
 *    enqueues one kernel on `stream` (a hipStream_t; NULL is the null stream)
 *    and returns.  Calls can be captured into a HIP graph.
 *  - Errors: a negative status is returned and NOTHING is launched (outputs
 *    untouched) for: a NULL required pointer (ALNP_ERR_NULL); rows < 0,
 *    dim <= 0 or sizes past the limits below (ALNP_ERR_SHAPE); dim odd for
 *    FP8, not a multiple of 16 for FP4 or of 32 for MX (ALNP_ERR_DIM); a chunk index
 *    outside [0, chunks) (ALNP_ERR_INDEX); a pointer not aligned to its
 *    element size (ALNP_ERR_ALIGN); a negative or non-finite eps
 *    (ALNP_ERR_ARG).  rows == 0 is a valid no-op.  If the launch itself
 *    fails, ALNP_ERR_LAUNCH is returned.  Device scalars (act_scale) are not
 *    inspected on the host.
 *  - Devices: every pointer of a call must be memory of the GPU that is the
 *    calling thread's current HIP device, and `stream` must belong to it;
 *    the kernel is launched there.  The library does not inspect pointers to
 *    find their device (that would cost microseconds per call), so this is
 *    the caller's to ensure; the package's Python functions run each call on
 *    the device of its first tensor and reject tensors from another.
 *  - Aliasing: outputs must not overlap inputs or each other.
 *  - Limits: rows (and batch * seq) <= 2^24 - 1; dim <= 2^24;
 *    alnp_quant_fp8_static_f32 takes n <= 2^31.
 *  - Numerics (identical for every operand form):
 *      mean = sum(x) / dim, var = sum((x - mean)^2) / dim   (fp32, biased)
 *      rstd = 1 / sqrt(var + eps)
 *      xhat = (x - mean) * rstd
 *      y    = (xhat * (1 + scale)) + shift   (fp32, each op rounded,
 *                                             no fused multiply-add)
 *      q    = e4m3(y * (1 / act_scale))     (round to nearest even,
 *                                             saturating at +-448; a NaN
 *                                             gives a NaN code, 0x7F or
 *                                             0xFF: the sign is not kept)
 *    The operation order (x * (scale + 1)) + shift is the one the
 *    h3-blackwell-runtime page states ("NVFP4 Modulation Producer Fusion",
 *    "Exactness Contract").
 *  - Optional outputs row_mean / row_rstd (fp32, (rows,)) receive the row
 *    statistics when non-NULL.
 */
#ifndef ALNP_H
#define ALNP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum alnp_status {
    ALNP_OK = 0,
    ALNP_ERR_NULL = -1,
    ALNP_ERR_SHAPE = -2,
    ALNP_ERR_DIM = -3,
    ALNP_ERR_INDEX = -4,
    ALNP_ERR_ALIGN = -5,
    ALNP_ERR_LAUNCH = -6,
    ALNP_ERR_ARG = -7
};

/* Version of this ABI; bumped on any signature change. */
int alnp_abi_version(void);

/* Static string for a status code; never NULL. */
const char* alnp_status_string(int status);

/*
 * Broadcast AdaLN -> FP8 (README "Available Functions":
 * ada_layer_norm_quant_fp8_bf16; "Tensor Contract": broadcast scale/shift).
 *   x          (rows, dim) bf16
 *   scale      (dim,) bf16, shared by every row
 *   shift      (dim,) bf16, shared by every row
 *   act_scale  device fp32 scalar, the dequantization scale
 *   eps        LayerNorm epsilon (the pages use 1e-5)
 *   out        (rows, dim) e4m3 codes
 *   row_mean, row_rstd  optional (rows,) fp32
 * dim must be even.
 */
int alnp_ada_layer_norm_quant_fp8_bf16(const uint16_t* x, const uint16_t* scale,
                                       const uint16_t* shift,
                                       const float* act_scale, float eps,
                                       int64_t rows, int64_t dim, uint8_t* out,
                                       float* row_mean, float* row_rstd,
                                       void* stream);

/*
 * Per-token AdaLN -> FP8 (README "Available Functions":
 * ada_layer_norm_quant_fp8_ptok_bf16; each activation row has its own
 * scale/shift row, read directly instead of from a broadcast copy).
 *   scale, shift  (rows, dim) bf16, one row of operands per activation row.
 * Other arguments as for the broadcast form.
 */
int alnp_ada_layer_norm_quant_fp8_ptok_bf16(const uint16_t* x,
                                            const uint16_t* scale,
                                            const uint16_t* shift,
                                            const float* act_scale, float eps,
                                            int64_t rows, int64_t dim,
                                            uint8_t* out, float* row_mean,
                                            float* row_rstd, void* stream);

/*
 * Table-form per-token AdaLN -> FP8 (README "Available Functions":
 * ada_layer_norm_quant_fp8_ptok_table_bf16; the kernel picks the scale and
 * shift chunks of temb itself and adds the fp32 table row to each).
 *   temb       (rows, chunks, dim) bf16
 *   table      (chunks, dim) fp32
 *   shift_idx, scale_idx  chunk indices in [0, chunks); they may be equal
 * The operands are scale[r, j] = temb[r, scale_idx, j] + table[scale_idx, j]
 * and likewise shift, each one fp32 addition (not rounded to bf16).  Only the
 * two selected chunks of temb are read.
 */
int alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(
    const uint16_t* x, const uint16_t* temb, const float* table, int64_t chunks,
    int64_t shift_idx, int64_t scale_idx, const float* act_scale, float eps,
    int64_t rows, int64_t dim, uint8_t* out, float* row_mean, float* row_rstd,
    void* stream);

/*
 * LayerNorm (no affine) -> FP8 (README:
 * layer_norm_no_affine_quant_fp8_static_bf16).  Same arithmetic as the
 * AdaLN forms with scale = shift = 0, so the result equals the broadcast
 * form called with zero operands, bit for bit.
 */
int alnp_layer_norm_no_affine_quant_fp8_static_bf16(
    const uint16_t* x, const float* act_scale, float eps, int64_t rows,
    int64_t dim, uint8_t* out, float* row_mean, float* row_rstd, void* stream);

/*
 * Broadcast AdaLN -> FP8 with modulation stored as e4m3 (README:
 * ada_layer_norm_quant_fp8_modfp8_bf16; "Tensor Contract": scale_fp8,
 * shift_fp8 e4m3 (dim,); scale_deq, shift_deq device fp32 scalars).
 *   scale[j] = e4m3(scale_fp8[j]) * (*scale_deq), one fp32 multiplication;
 *   shift likewise; then the same normalize / modulate / quantize as above.
 * dim must be even.
 */
int alnp_ada_layer_norm_quant_fp8_modfp8_bf16(const uint16_t* x,
                                              const uint8_t* scale_fp8,
                                              const uint8_t* shift_fp8,
                                              const float* scale_deq,
                                              const float* shift_deq,
                                              const float* act_scale, float eps,
                                              int64_t rows, int64_t dim,
                                              uint8_t* out, float* row_mean,
                                              float* row_rstd, void* stream);

/*
 * Broadcast AdaLN -> per-channel AWQ smoothing -> FP8 (README:
 * awq_ada_layer_norm_quant_fp8_bf16; "Tensor Contract": inv_s bf16 (dim,)).
 *   q = e4m3((y * inv_s[j]) * (1 / act_scale)), each multiplication rounded.
 * dim must be even.
 */
int alnp_awq_ada_layer_norm_quant_fp8_bf16(const uint16_t* x, const uint16_t* scale,
                                           const uint16_t* shift, const uint16_t* inv_s,
                                           const float* act_scale, float eps,
                                           int64_t rows, int64_t dim, uint8_t* out,
                                           float* row_mean, float* row_rstd,
                                           void* stream);

/*
 * LayerNorm (no affine) -> FP4 (README:
 * layer_norm_no_affine_quant_nvfp4_swizzled_bf16, with the block scales in
 * plain row-major order instead of the 128x4 swizzle).
 *   packed  (rows, dim/2) uint8: two e2m1 codes per byte, element 2i in the
 *           low nibble (low-nibble-first, as the conversion-contract example
 *           on the h3-blackwell-runtime page prints)
 *   sf      (rows, dim/16) e4m3 block scales, row-major; size from
 *           alnp_sf_size()
 * Per row: xhat as above, rounded to bf16 (the README's staged BF16 norm);
 * per block of 16: s = e4m3(amax / 6) (IEEE division, saturating at 448);
 * codes = e2m1(b * (1 / s)) rounded to nearest even, saturating at +-6; a
 * block whose scale is 0 gets all-zero codes.  dim % 16 == 0.
 */
int alnp_layer_norm_no_affine_quant_nvfp4_bf16(const uint16_t* x, float eps,
                                               int64_t rows, int64_t dim,
                                               uint8_t* packed, uint8_t* sf,
                                               float* row_mean,
                                               float* row_rstd, void* stream);

/* Bytes of the row-major block-scale buffer for an FP4 output: rows*dim/16.
 * Returns a negative status for invalid sizes. */
int64_t alnp_sf_size(int64_t rows, int64_t dim);

/*
 * LayerNorm (no affine) -> FP4 with the block scales in the 128x4 tiled
 * ("swizzled") layout (README: layer_norm_no_affine_quant_nvfp4_swizzled_bf16;
 * "Tensor Contract": scale bytes in a 128x4 tiled layout, sized by
 * swizzled_sf_size).  The pages name the layout without defining it; this is
 * the tiled layout NVIDIA documents for block-scaled GEMM operands:
 *   cols = dim / 16 scales per row; tiles of 128 rows x 4 scales, 512 bytes
 *   each, stored tile-row-major; scale (r, c) lives at
 *     ((r / 128) * ceil(cols / 4) + c / 4) * 512
 *       + (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4).
 *   sf_swizzled holds alnp_swizzled_sf_size(rows, dim) bytes.  Padding
 *   columns (cols rounded up to 4) of every written row are set to 0; padding
 *   rows (rows rounded up to 128) are not written.
 * packed, numerics and errors as for the row-major entry.
 */
int alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16(
    const uint16_t* x, float eps, int64_t rows, int64_t dim, uint8_t* packed,
    uint8_t* sf_swizzled, float* row_mean, float* row_rstd, void* stream);

/*
 * Broadcast AdaLN -> FP4 (README: ada_layer_norm_quant_nvfp4_swizzled_bf16,
 * here with row-major scales; the _swizzled entry below takes the tiled
 * layout).  scale, shift (dim,) bf16.  Per row: y = (xhat * (1 + scale)) +
 * shift in fp32 exactly as on the FP8 path, then y is rounded to bf16 and
 * quantized in blocks of 16 as for the LayerNorm entry.
 */
int alnp_ada_layer_norm_quant_nvfp4_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps,
                                         int64_t rows, int64_t dim,
                                         uint8_t* packed, uint8_t* sf,
                                         float* row_mean, float* row_rstd,
                                         void* stream);
int alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16(
    const uint16_t* x, const uint16_t* scale, const uint16_t* shift, float eps,
    int64_t rows, int64_t dim, uint8_t* packed, uint8_t* sf_swizzled,
    float* row_mean, float* row_rstd, void* stream);

/*
 * AdaLN -> FP4 with e4m3 modulation operands (README "Available Functions":
 * ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16; "Tensor Contract":
 * scale_fp8/shift_fp8 e4m3 (dim,), scale_deq/shift_deq fp32 device scalars).
 * The operands are e4m3(code) * deq (one fp32 multiplication each), then the
 * broadcast AdaLN -> FP4 arithmetic above, with the block scales written in
 * the 128x4 tiled layout (buffer of alnp_swizzled_sf_size bytes).
 *   scale_fp8, shift_fp8  (dim,) e4m3 codes
 *   scale_deq, shift_deq  device fp32 scalars (4-byte aligned)
 */
int alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
    const uint16_t* x, const uint8_t* scale_fp8, const uint8_t* shift_fp8,
    const float* scale_deq, const float* shift_deq, float eps, int64_t rows, int64_t dim,
    uint8_t* packed, uint8_t* sf_swizzled, float* row_mean, float* row_rstd, void* stream);

/* Bytes of the tiled block-scale buffer (README: swizzled_sf_size):
 * ceil(rows / 128) * 128 * ceil(dim / 64) * 4.  Negative status for invalid
 * sizes. */
int64_t alnp_swizzled_sf_size(int64_t rows, int64_t dim);

/*
 * Six-way DiT modulation (README: adaln_modulation6_bf16; "Tensor Contract":
 * fp32 params of shape (batch, seq, 6, dim) and an fp32 (6, dim) per-layer
 * table in, six bf16 (batch, seq, dim) tensors out).
 *   params     (batch, seq, 6, dim) fp32
 *   layer_mod  (6, dim) fp32
 *   out        HOST array of 6 device pointers; out[k] is (batch, seq, dim)
 *              bf16 and receives bf16_rne(params[b, s, k, :] + layer_mod[k, :])
 * NaN sums give a quiet NaN, overflow gives +-inf.
 */
int alnp_adaln_modulation6_bf16(const float* params, const float* layer_mod,
                                int64_t batch, int64_t seq, int64_t dim,
                                uint16_t* const out[6], void* stream);

/*
 * Residual gate step (the residual-gate epilogue whose numerical program the
 * h3-blackwell-runtime page fixes: bf16 projection output, gate
 * multiplication with its bf16 boundary, bf16 residual added, final bf16
 * rounding).  The gate is a six-way producer output chunk (per token) or a
 * (dim,) vector:
 *   out[r, j] = bf16_rne(residual[r, j] + bf16_rne(gate[g, j] * proj[r, j]))
 * with g = r when gate_rows == rows and g = 0 when gate_rows == 1.
 *   residual, proj, out  (rows, dim) bf16; out may be residual itself
 *                        (in-place x += gate * proj); no other overlap.
 *   gate                 (gate_rows, dim) bf16, gate_rows 1 or rows.
 * Other gate_rows values return ALNP_ERR_SHAPE.
 */
int alnp_gated_residual_bf16(const uint16_t* residual, const uint16_t* gate,
                             const uint16_t* proj, int64_t rows, int64_t dim,
                             int64_t gate_rows, uint16_t* out, void* stream);

/*
 * MX block formats: MXFP8 (E4M3 elements) and MXFP4 (E2M1 elements, packed
 * as above) with one E8M0 scale per 32 consecutive row elements, the operand
 * format of gfx950's scaled matrix instructions.  The pages do not cover MX;
 * the block rule is the OCP Microscaling Formats (MX) v1.0 specification's
 * conversion of a vector to an MX block:
 *   X = 2^E, E = floor(log2(amax)) - emax   (emax 8 for E4M3, 2 for E2M1),
 *   E clamped to [-127, 127] (-127 for a block without a non-zero value,
 *   127 for an infinite amax); scale byte = E + 127;
 *   element = round_to_nearest_even(v / X), saturated at +-448 (E4M3) or
 *   +-6 (E2M1); amax ignores NaN.
 * MXFP8 quantizes the FP8 path's fp32 y (no act_scale: the block scales take
 * its place); MXFP4 quantizes the bf16-staged value of the FP4 entries.  The
 * operand forms are those of the FP8 entries (LayerNorm, broadcast,
 * per-token, table, modfp8, AWQ) for MXFP8, and of the FP4 entries
 * (LayerNorm, broadcast, modfp8) for MXFP4, with the same operand arguments.
 *   out      (rows, dim) e4m3 codes (MXFP8); packed (rows, dim/2) (MXFP4)
 *   scales   (rows, dim/32) E8M0 bytes, row-major
 * dim must be a multiple of 32 (ALNP_ERR_DIM).  Codes for NaN elements are
 * unspecified.  Other arguments and errors as for the FP8 / FP4 entries.
 */
int alnp_layer_norm_no_affine_quant_mxfp8_bf16(const uint16_t* x, float eps,
                                               int64_t rows, int64_t dim, uint8_t* out,
                                               uint8_t* scales, float* row_mean,
                                               float* row_rstd, void* stream);
int alnp_ada_layer_norm_quant_mxfp8_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps, int64_t rows,
                                         int64_t dim, uint8_t* out, uint8_t* scales,
                                         float* row_mean, float* row_rstd, void* stream);
int alnp_ada_layer_norm_quant_mxfp8_ptok_bf16(const uint16_t* x, const uint16_t* scale,
                                              const uint16_t* shift, float eps, int64_t rows,
                                              int64_t dim, uint8_t* out, uint8_t* scales,
                                              float* row_mean, float* row_rstd, void* stream);
/* Table form: operands temb[:, idx] + table[idx] as for the FP8 table entry
 * (chunk indices outside [0, chunks) give ALNP_ERR_INDEX). */
int alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(
    const uint16_t* x, const uint16_t* temb, const float* table, int64_t chunks,
    int64_t shift_idx, int64_t scale_idx, float eps, int64_t rows, int64_t dim, uint8_t* out,
    uint8_t* scales, float* row_mean, float* row_rstd, void* stream);
/* modfp8 form: e4m3 (dim,) scale / shift times fp32 device dequantization
 * scalars, as for alnp_ada_layer_norm_quant_fp8_modfp8_bf16. */
int alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16(const uint16_t* x, const uint8_t* scale_fp8,
                                                const uint8_t* shift_fp8, const float* scale_deq,
                                                const float* shift_deq, float eps, int64_t rows,
                                                int64_t dim, uint8_t* out, uint8_t* scales,
                                                float* row_mean, float* row_rstd, void* stream);
/* AWQ form: broadcast modulation, then y * inv_s[j] (bf16 (dim,)) before the
 * block quantization, as for alnp_awq_ada_layer_norm_quant_fp8_bf16. */
int alnp_awq_ada_layer_norm_quant_mxfp8_bf16(const uint16_t* x, const uint16_t* scale,
                                             const uint16_t* shift, const uint16_t* inv_s,
                                             float eps, int64_t rows, int64_t dim, uint8_t* out,
                                             uint8_t* scales, float* row_mean, float* row_rstd,
                                             void* stream);
int alnp_layer_norm_no_affine_quant_mxfp4_bf16(const uint16_t* x, float eps,
                                               int64_t rows, int64_t dim, uint8_t* packed,
                                               uint8_t* scales, float* row_mean,
                                               float* row_rstd, void* stream);
int alnp_ada_layer_norm_quant_mxfp4_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps, int64_t rows,
                                         int64_t dim, uint8_t* packed, uint8_t* scales,
                                         float* row_mean, float* row_rstd, void* stream);
/* modfp8 form, as for alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16,
 * with row-major E8M0 scales. */
int alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16(const uint16_t* x, const uint8_t* scale_fp8,
                                                const uint8_t* shift_fp8, const float* scale_deq,
                                                const float* shift_deq, float eps, int64_t rows,
                                                int64_t dim, uint8_t* packed, uint8_t* scales,
                                                float* row_mean, float* row_rstd, void* stream);
/* Bytes of an MX scale buffer: rows * dim / 32; negative status otherwise. */
int64_t alnp_mx_scale_size(int64_t rows, int64_t dim);

/*
 * RMSNorm with segment-selected AdaLN modulation -> bf16.  Sources: the
 * RL-Kernel norm_modulate page (a modulated RMSNorm with an RMSNorm weight and
 * scale/shift rows picked per token by index_select) and the
 * h3-blackwell-runtime page ("Implementation Phases": an RMSNorm whose output
 * is modulated with AdaLN scale/shift chosen per segment; "NVFP4 Modulation
 * Producer Fusion", "Exactness Contract": per-segment operands, the
 * (x * (scale + 1)) + shift order, BF16 rounding).  Per row r, s = seg[r]:
 *   rstd = 1 / sqrt(sum_j x[r, j]^2 / dim + eps)     (fp32; no centring)
 *   n    = bf16_rne((x * rstd) * weight[j])          (weight 1 if NULL)
 *   t    = bf16_rne(scale[s, j] + 1)
 *   u    = bf16_rne(n * t)
 *   out  = bf16_rne(u + shift[s, j])
 * Every bf16 step is one fp32 operation rounded to bf16, as a bf16 tensor
 * operation is.
 *   x             (rows, dim) bf16
 *   weight        (dim,) bf16, or NULL for no RMSNorm weight
 *   scale, shift  (segments, dim) bf16 tables, segments >= 1
 *   seg           (rows,) int32 table row of each row (DEVICE; not read on the
 *                 host).  A row whose index is outside [0, segments) reads no
 *                 table row and is written as quiet NaN (0x7FC0).
 *   out           (rows, dim) bf16
 *   row_rstd      (rows,) fp32 or NULL
 * Any dim in 1 .. 2^24 (no parity rule); segments outside 1 .. 2^31 - 1
 * returns ALNP_ERR_SHAPE.
 */
int alnp_rms_norm_modulate_seg_bf16(const uint16_t* x, const uint16_t* weight,
                                    const uint16_t* scale, const uint16_t* shift,
                                    const int32_t* seg, int64_t segments, float eps,
                                    int64_t rows, int64_t dim, uint16_t* out,
                                    float* row_rstd, void* stream);

/*
 * Static-scale FP8 quantizer on its own, the last stage of every FP8
 * producer: out[i] = e4m3(v[i] * (1 / act_scale)), same rounding and
 * saturation as above.  n >= 0 elements of fp32 input.
 */
int alnp_quant_fp8_static_f32(const float* v, const float* act_scale,
                              int64_t n, uint8_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ALNP_H */
