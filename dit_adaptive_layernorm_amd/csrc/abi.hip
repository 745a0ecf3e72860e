// abi.hip -- the C entry points of libalnp: host-side validation, then one
// kernel launch on the caller's stream.  Nothing here allocates, frees or
// synchronizes.  Argument conventions and error codes are documented in
// include/alnp.h.
#include "alnp.h"
#include "kernels.hpp"

#include <cmath>

namespace {

using alnp::Fp4Args;
using alnp::Fp8Args;
using alnp::Mod6Args;

Fp8Args fp8_args(const uint16_t* x, const float* act_scale, float eps, int64_t rows,
                       int64_t dim, uint8_t* out, float* row_mean, float* row_rstd)
{
    Fp8Args a{};
    a.x = x;
    a.act_scale = act_scale;
    a.eps = eps;
    a.rows = rows;
    a.dim = (int)dim;
    a.out = out;
    a.row_mean = row_mean;
    a.row_rstd = row_rstd;
    return a;
}

constexpr int64_t kMaxRows = (int64_t(1) << 24) - 1;
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxQuantN = int64_t(1) << 31;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status(hipError_t e) { return e == hipSuccess ? ALNP_OK : ALNP_ERR_LAUNCH; }

// Checks shared by the LayerNorm producers.  Returns ALNP_OK to go on, or a
// status to return (1 = valid no-op for rows == 0).
int check_rows_dim(int64_t rows, int64_t dim, int64_t dim_multiple)
{
    if (rows < 0 || rows > kMaxRows || dim <= 0 || dim > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (dim % dim_multiple != 0)
        return ALNP_ERR_DIM;
    return rows == 0 ? 1 : ALNP_OK;
}

int check_eps(float eps) { return (std::isfinite(eps) && eps >= 0.f) ? ALNP_OK : ALNP_ERR_ARG; }

// Common tail of the FP8 producers: null/alignment/eps checks, choice of
// kernel, launch.
int run_fp8(Fp8Args a, int form, void* stream)
{
    if (!a.x || !a.act_scale || !a.out)
        return ALNP_ERR_NULL;
    if ((form == alnp::kBcast || form == alnp::kPtok || form == alnp::kAwq) &&
        (!a.scale || !a.shift))
        return ALNP_ERR_NULL;
    if (form == alnp::kAwq && !a.inv_s)
        return ALNP_ERR_NULL;
    if (form == alnp::kTable && (!a.temb || !a.table))
        return ALNP_ERR_NULL;
    if (form == alnp::kModFp8 && (!a.scale_fp8 || !a.shift_fp8 || !a.scale_deq || !a.shift_deq))
        return ALNP_ERR_NULL;
    if (!aligned(a.x, 2) || !aligned(a.act_scale, 4) || !aligned(a.scale, 2) ||
        !aligned(a.shift, 2) || !aligned(a.temb, 2) || !aligned(a.table, 4) ||
        !aligned(a.inv_s, 2) || !aligned(a.scale_deq, 4) || !aligned(a.shift_deq, 4) ||
        !aligned(a.row_mean, 4) || !aligned(a.row_rstd, 4))
        return ALNP_ERR_ALIGN;
    if (int st = check_eps(a.eps))
        return st;
    const bool fast = a.dim % 8 == 0 && a.dim <= alnp::kMaxFastDim && aligned(a.x, 16) &&
                      aligned(a.scale, 16) && aligned(a.shift, 16) && aligned(a.temb, 16) &&
                      aligned(a.table, 16) && aligned(a.inv_s, 16) && aligned(a.scale_fp8, 8) &&
                      aligned(a.shift_fp8, 8) && aligned(a.out, 8);
    return launch_status(alnp::launch_adaln_fp8(a, form, fast, as_stream(stream)));
}

// MXFP8 producers (no act_scale; a.mx_scales receives the block scales).
int run_mxfp8(Fp8Args a, int form, void* stream)
{
    if (int st = check_rows_dim(a.rows, a.dim, 32))
        return st > 0 ? ALNP_OK : st;
    if (!a.x || !a.out || !a.mx_scales ||
        ((form == alnp::kBcast || form == alnp::kPtok || form == alnp::kAwq) &&
         (!a.scale || !a.shift)) ||
        (form == alnp::kAwq && !a.inv_s) ||
        (form == alnp::kTable && (!a.temb || !a.table)) ||
        (form == alnp::kModFp8 && (!a.scale_fp8 || !a.shift_fp8 || !a.scale_deq || !a.shift_deq)))
        return ALNP_ERR_NULL;
    if (!aligned(a.x, 2) || !aligned(a.scale, 2) || !aligned(a.shift, 2) || !aligned(a.temb, 2) ||
        !aligned(a.table, 4) || !aligned(a.inv_s, 2) || !aligned(a.scale_deq, 4) ||
        !aligned(a.shift_deq, 4) || !aligned(a.row_mean, 4) || !aligned(a.row_rstd, 4))
        return ALNP_ERR_ALIGN;
    if (int st = check_eps(a.eps))
        return st;
    const bool fast = a.dim <= alnp::kMaxFastDim && aligned(a.x, 16) && aligned(a.scale, 16) &&
                      aligned(a.shift, 16) && aligned(a.temb, 16) && aligned(a.table, 16) &&
                      aligned(a.inv_s, 16) && aligned(a.scale_fp8, 8) &&
                      aligned(a.shift_fp8, 8) && aligned(a.out, 8);
    return launch_status(alnp::launch_mxfp8(a, form, fast, as_stream(stream)));
}

}  // namespace

extern "C" {

int alnp_abi_version(void) { return 1; }

const char* alnp_status_string(int status)
{
    switch (status) {
    case ALNP_OK: return "ok";
    case ALNP_ERR_NULL: return "a required pointer is NULL";
    case ALNP_ERR_SHAPE: return "rows/dim out of range";
    case ALNP_ERR_DIM: return "dim must be even (FP8), a multiple of 16 (FP4) or of 32 (MX)";
    case ALNP_ERR_INDEX: return "chunk index outside [0, chunks)";
    case ALNP_ERR_ALIGN: return "pointer not aligned to its element size";
    case ALNP_ERR_LAUNCH: return "kernel launch failed";
    case ALNP_ERR_ARG: return "eps must be finite and >= 0";
    default: return "unknown status";
    }
}

int alnp_ada_layer_norm_quant_fp8_bf16(const uint16_t* x, const uint16_t* scale,
                                       const uint16_t* shift, const float* act_scale, float eps,
                                       int64_t rows, int64_t dim, uint8_t* out, float* row_mean,
                                       float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    a.scale = scale;
    a.shift = shift;
    return run_fp8(a, alnp::kBcast, stream);
}

int alnp_ada_layer_norm_quant_fp8_ptok_bf16(const uint16_t* x, const uint16_t* scale,
                                            const uint16_t* shift, const float* act_scale,
                                            float eps, int64_t rows, int64_t dim, uint8_t* out,
                                            float* row_mean, float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    a.scale = scale;
    a.shift = shift;
    return run_fp8(a, alnp::kPtok, stream);
}

int alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(const uint16_t* x, const uint16_t* temb,
                                                  const float* table, int64_t chunks,
                                                  int64_t shift_idx, int64_t scale_idx,
                                                  const float* act_scale, float eps, int64_t rows,
                                                  int64_t dim, uint8_t* out, float* row_mean,
                                                  float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    if (chunks <= 0 || chunks > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (shift_idx < 0 || shift_idx >= chunks || scale_idx < 0 || scale_idx >= chunks)
        return ALNP_ERR_INDEX;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    a.temb = temb;
    a.table = table;
    a.chunks = chunks;
    a.shift_idx = shift_idx;
    a.scale_idx = scale_idx;
    return run_fp8(a, alnp::kTable, stream);
}

int alnp_layer_norm_no_affine_quant_fp8_static_bf16(const uint16_t* x, const float* act_scale,
                                                    float eps, int64_t rows, int64_t dim,
                                                    uint8_t* out, float* row_mean,
                                                    float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    return run_fp8(a, alnp::kNone, stream);
}

int alnp_ada_layer_norm_quant_fp8_modfp8_bf16(const uint16_t* x, const uint8_t* scale_fp8,
                                              const uint8_t* shift_fp8, const float* scale_deq,
                                              const float* shift_deq, const float* act_scale,
                                              float eps, int64_t rows, int64_t dim, uint8_t* out,
                                              float* row_mean, float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    a.scale_fp8 = scale_fp8;
    a.shift_fp8 = shift_fp8;
    a.scale_deq = scale_deq;
    a.shift_deq = shift_deq;
    return run_fp8(a, alnp::kModFp8, stream);
}

int alnp_awq_ada_layer_norm_quant_fp8_bf16(const uint16_t* x, const uint16_t* scale,
                                           const uint16_t* shift, const uint16_t* inv_s,
                                           const float* act_scale, float eps, int64_t rows,
                                           int64_t dim, uint8_t* out, float* row_mean,
                                           float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 2))
        return st > 0 ? ALNP_OK : st;
    Fp8Args a = fp8_args(x, act_scale, eps, rows, dim, out, row_mean, row_rstd);
    a.scale = scale;
    a.shift = shift;
    a.inv_s = inv_s;
    return run_fp8(a, alnp::kAwq, stream);
}

}  // extern "C"

namespace {

// Common tail of the FP4 producers (scale/shift null for LayerNorm only).
Fp4Args fp4_args(const uint16_t* x, float eps, int64_t rows, int64_t dim, uint8_t* packed,
                 uint8_t* sf, int layout, float* row_mean, float* row_rstd)
{
    Fp4Args a{};
    a.x = x;
    a.eps = eps;
    a.rows = rows;
    a.dim = (int)dim;
    a.packed = packed;
    a.sf = sf;
    a.sf_layout = layout;
    a.row_mean = row_mean;
    a.row_rstd = row_rstd;
    a.form = alnp::kNone;
    return a;
}

// Common tail of the FP4 producers: null/alignment/eps checks, choice of
// kernel, launch.  a.form selects the operands that must be present.
int run_fp4(Fp4Args a, void* stream)
{
    if (int st = check_rows_dim(a.rows, a.dim, a.mx ? 32 : 16))
        return st > 0 ? ALNP_OK : st;
    if (!a.x || !a.packed || !a.sf || (a.form == alnp::kBcast && (!a.scale || !a.shift)) ||
        (a.form == alnp::kModFp8 &&
         (!a.scale_fp8 || !a.shift_fp8 || !a.scale_deq || !a.shift_deq)))
        return ALNP_ERR_NULL;
    if (!aligned(a.x, 2) || !aligned(a.scale, 2) || !aligned(a.shift, 2) ||
        !aligned(a.scale_deq, 4) || !aligned(a.shift_deq, 4) || !aligned(a.row_mean, 4) ||
        !aligned(a.row_rstd, 4))
        return ALNP_ERR_ALIGN;
    if (int st = check_eps(a.eps))
        return st;
    const bool fast = a.dim <= alnp::kMaxFastDim && aligned(a.x, 16) && aligned(a.scale, 16) &&
                      aligned(a.shift, 16) && aligned(a.scale_fp8, 8) &&
                      aligned(a.shift_fp8, 8) && aligned(a.packed, 4);
    return launch_status(alnp::launch_fp4(a, fast, as_stream(stream)));
}

}  // namespace

extern "C" {

int alnp_layer_norm_no_affine_quant_nvfp4_bf16(const uint16_t* x, float eps, int64_t rows,
                                               int64_t dim, uint8_t* packed, uint8_t* sf,
                                               float* row_mean, float* row_rstd, void* stream)
{
    return run_fp4(fp4_args(x, eps, rows, dim, packed, sf, alnp::kSfRowMajor, row_mean, row_rstd),
                   stream);
}

int alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16(const uint16_t* x, float eps,
                                                        int64_t rows, int64_t dim,
                                                        uint8_t* packed, uint8_t* sf_swizzled,
                                                        float* row_mean, float* row_rstd,
                                                        void* stream)
{
    return run_fp4(fp4_args(x, eps, rows, dim, packed, sf_swizzled, alnp::kSfSwizzled, row_mean,
                            row_rstd),
                   stream);
}

int alnp_ada_layer_norm_quant_nvfp4_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps, int64_t rows,
                                         int64_t dim, uint8_t* packed, uint8_t* sf,
                                         float* row_mean, float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, sf, alnp::kSfRowMajor, row_mean, row_rstd);
    a.form = alnp::kBcast;
    a.scale = scale;
    a.shift = shift;
    return run_fp4(a, stream);
}

int alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16(const uint16_t* x, const uint16_t* scale,
                                                  const uint16_t* shift, float eps,
                                                  int64_t rows, int64_t dim, uint8_t* packed,
                                                  uint8_t* sf_swizzled, float* row_mean,
                                                  float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, sf_swizzled, alnp::kSfSwizzled, row_mean,
                         row_rstd);
    a.form = alnp::kBcast;
    a.scale = scale;
    a.shift = shift;
    return run_fp4(a, stream);
}

int alnp_layer_norm_no_affine_quant_mxfp4_bf16(const uint16_t* x, float eps, int64_t rows,
                                               int64_t dim, uint8_t* packed, uint8_t* scales,
                                               float* row_mean, float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, scales, alnp::kSfRowMajor, row_mean, row_rstd);
    a.mx = 1;
    return run_fp4(a, stream);
}

int alnp_ada_layer_norm_quant_mxfp4_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps, int64_t rows,
                                         int64_t dim, uint8_t* packed, uint8_t* scales,
                                         float* row_mean, float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, scales, alnp::kSfRowMajor, row_mean, row_rstd);
    a.mx = 1;
    a.form = alnp::kBcast;
    a.scale = scale;
    a.shift = shift;
    return run_fp4(a, stream);
}

int alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16(const uint16_t* x, const uint8_t* scale_fp8,
                                                const uint8_t* shift_fp8, const float* scale_deq,
                                                const float* shift_deq, float eps, int64_t rows,
                                                int64_t dim, uint8_t* packed, uint8_t* scales,
                                                float* row_mean, float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, scales, alnp::kSfRowMajor, row_mean, row_rstd);
    a.mx = 1;
    a.form = alnp::kModFp8;
    a.scale_fp8 = scale_fp8;
    a.shift_fp8 = shift_fp8;
    a.scale_deq = scale_deq;
    a.shift_deq = shift_deq;
    return run_fp4(a, stream);
}

int alnp_layer_norm_no_affine_quant_mxfp8_bf16(const uint16_t* x, float eps, int64_t rows,
                                               int64_t dim, uint8_t* out, uint8_t* scales,
                                               float* row_mean, float* row_rstd, void* stream)
{
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    return run_mxfp8(a, alnp::kNone, stream);
}

int alnp_ada_layer_norm_quant_mxfp8_bf16(const uint16_t* x, const uint16_t* scale,
                                         const uint16_t* shift, float eps, int64_t rows,
                                         int64_t dim, uint8_t* out, uint8_t* scales,
                                         float* row_mean, float* row_rstd, void* stream)
{
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    a.scale = scale;
    a.shift = shift;
    return run_mxfp8(a, alnp::kBcast, stream);
}

int alnp_ada_layer_norm_quant_mxfp8_ptok_bf16(const uint16_t* x, const uint16_t* scale,
                                              const uint16_t* shift, float eps, int64_t rows,
                                              int64_t dim, uint8_t* out, uint8_t* scales,
                                              float* row_mean, float* row_rstd, void* stream)
{
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    a.scale = scale;
    a.shift = shift;
    return run_mxfp8(a, alnp::kPtok, stream);
}

int alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16(const uint16_t* x, const uint8_t* scale_fp8,
                                                const uint8_t* shift_fp8, const float* scale_deq,
                                                const float* shift_deq, float eps, int64_t rows,
                                                int64_t dim, uint8_t* out, uint8_t* scales,
                                                float* row_mean, float* row_rstd, void* stream)
{
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    a.scale_fp8 = scale_fp8;
    a.shift_fp8 = shift_fp8;
    a.scale_deq = scale_deq;
    a.shift_deq = shift_deq;
    return run_mxfp8(a, alnp::kModFp8, stream);
}

int alnp_awq_ada_layer_norm_quant_mxfp8_bf16(const uint16_t* x, const uint16_t* scale,
                                             const uint16_t* shift, const uint16_t* inv_s,
                                             float eps, int64_t rows, int64_t dim, uint8_t* out,
                                             uint8_t* scales, float* row_mean, float* row_rstd,
                                             void* stream)
{
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    a.scale = scale;
    a.shift = shift;
    a.inv_s = inv_s;
    return run_mxfp8(a, alnp::kAwq, stream);
}

int alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(
    const uint16_t* x, const uint16_t* temb, const float* table, int64_t chunks, int64_t shift_idx,
    int64_t scale_idx, float eps, int64_t rows, int64_t dim, uint8_t* out, uint8_t* scales,
    float* row_mean, float* row_rstd, void* stream)
{
    if (int st = check_rows_dim(rows, dim, 32))
        return st > 0 ? ALNP_OK : st;
    if (chunks < 1 || chunks > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (shift_idx < 0 || shift_idx >= chunks || scale_idx < 0 || scale_idx >= chunks)
        return ALNP_ERR_INDEX;
    Fp8Args a = fp8_args(x, nullptr, eps, rows, dim, out, row_mean, row_rstd);
    a.mx_scales = scales;
    a.temb = temb;
    a.table = table;
    a.chunks = chunks;
    a.shift_idx = shift_idx;
    a.scale_idx = scale_idx;
    return run_mxfp8(a, alnp::kTable, stream);
}

int64_t alnp_mx_scale_size(int64_t rows, int64_t dim)
{
    if (rows < 0 || rows > kMaxRows || dim <= 0 || dim > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (dim % 32 != 0)
        return ALNP_ERR_DIM;
    return rows * (dim / 32);
}

int alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
    const uint16_t* x, const uint8_t* scale_fp8, const uint8_t* shift_fp8,
    const float* scale_deq, const float* shift_deq, float eps, int64_t rows, int64_t dim,
    uint8_t* packed, uint8_t* sf_swizzled, float* row_mean, float* row_rstd, void* stream)
{
    Fp4Args a = fp4_args(x, eps, rows, dim, packed, sf_swizzled, alnp::kSfSwizzled, row_mean,
                         row_rstd);
    a.form = alnp::kModFp8;
    a.scale_fp8 = scale_fp8;
    a.shift_fp8 = shift_fp8;
    a.scale_deq = scale_deq;
    a.shift_deq = shift_deq;
    return run_fp4(a, stream);
}

int64_t alnp_sf_size(int64_t rows, int64_t dim)
{
    if (rows < 0 || rows > kMaxRows || dim <= 0 || dim > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (dim % 16 != 0)
        return ALNP_ERR_DIM;
    return rows * (dim / 16);
}

int64_t alnp_swizzled_sf_size(int64_t rows, int64_t dim)
{
    if (rows < 0 || rows > kMaxRows || dim <= 0 || dim > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (dim % 16 != 0)
        return ALNP_ERR_DIM;
    return alnp::sf_swizzled_size(rows, dim / 16);
}

int alnp_adaln_modulation6_bf16(const float* params, const float* layer_mod, int64_t batch,
                                int64_t seq, int64_t dim, uint16_t* const out[6], void* stream)
{
    if (batch < 0 || seq < 0 || dim <= 0 || dim > kMaxDim)
        return ALNP_ERR_SHAPE;
    if (seq != 0 && batch > kMaxRows / seq)
        return ALNP_ERR_SHAPE;
    const int64_t tokens = batch * seq;
    if (tokens == 0)
        return ALNP_OK;
    if (!params || !layer_mod || !out)
        return ALNP_ERR_NULL;
    Mod6Args a{params, layer_mod, tokens, (int)dim, {}};
    bool fast = dim % 8 == 0 && aligned(params, 16) && aligned(layer_mod, 16);
    for (int k = 0; k < 6; ++k) {
        if (!out[k])
            return ALNP_ERR_NULL;
        if (!aligned(out[k], 2))
            return ALNP_ERR_ALIGN;
        fast = fast && aligned(out[k], 16);
        a.out[k] = out[k];
    }
    if (!aligned(params, 4) || !aligned(layer_mod, 4))
        return ALNP_ERR_ALIGN;
    return launch_status(alnp::launch_modulation6(a, fast, as_stream(stream)));
}

int alnp_gated_residual_bf16(const uint16_t* residual, const uint16_t* gate,
                             const uint16_t* proj, int64_t rows, int64_t dim, int64_t gate_rows,
                             uint16_t* out, void* stream)
{
    if (rows < 0 || rows > kMaxRows || dim <= 0 || dim > kMaxDim ||
        (gate_rows != 1 && gate_rows != rows))
        return ALNP_ERR_SHAPE;
    if (rows == 0)
        return ALNP_OK;
    if (!residual || !gate || !proj || !out)
        return ALNP_ERR_NULL;
    if (!aligned(residual, 2) || !aligned(gate, 2) || !aligned(proj, 2) || !aligned(out, 2))
        return ALNP_ERR_ALIGN;
    alnp::GateArgs a{residual, gate, proj, rows, (int)dim, gate_rows, out};
    const bool fast = dim % 8 == 0 && aligned(residual, 16) && aligned(gate, 16) &&
                      aligned(proj, 16) && aligned(out, 16);
    return launch_status(alnp::launch_gated_residual(a, fast, as_stream(stream)));
}

int alnp_rms_norm_modulate_seg_bf16(const uint16_t* x, const uint16_t* weight,
                                    const uint16_t* scale, const uint16_t* shift,
                                    const int32_t* seg, int64_t segments, float eps,
                                    int64_t rows, int64_t dim, uint16_t* out, float* row_rstd,
                                    void* stream)
{
    if (int st = check_rows_dim(rows, dim, 1))
        return st > 0 ? ALNP_OK : st;
    if (segments < 1 || segments > INT32_MAX)
        return ALNP_ERR_SHAPE;
    if (!x || !scale || !shift || !seg || !out)
        return ALNP_ERR_NULL;
    if (!aligned(x, 2) || (weight && !aligned(weight, 2)) || !aligned(scale, 2) ||
        !aligned(shift, 2) || !aligned(seg, 4) || !aligned(out, 2) ||
        (row_rstd && !aligned(row_rstd, 4)))
        return ALNP_ERR_ALIGN;
    if (int st = check_eps(eps))
        return st;
    alnp::RmsArgs a{x, weight, scale, shift, seg, segments, eps, rows, (int)dim, out, row_rstd,
                    0.f};
    const bool fast = dim % 8 == 0 && dim <= alnp::kMaxFastDim && aligned(x, 16) &&
                      (!weight || aligned(weight, 16)) && aligned(scale, 16) &&
                      aligned(shift, 16) && aligned(out, 16);
    return launch_status(alnp::launch_rms_modulate(a, fast, as_stream(stream)));
}

int alnp_quant_fp8_static_f32(const float* v, const float* act_scale, int64_t n, uint8_t* out,
                              void* stream)
{
    if (n < 0 || n > kMaxQuantN)
        return ALNP_ERR_SHAPE;
    if (n == 0)
        return ALNP_OK;
    if (!v || !act_scale || !out)
        return ALNP_ERR_NULL;
    if (!aligned(v, 4) || !aligned(act_scale, 4))
        return ALNP_ERR_ALIGN;
    return launch_status(alnp::launch_quant_fp8(v, act_scale, n, out, as_stream(stream)));
}

}  // extern "C"
