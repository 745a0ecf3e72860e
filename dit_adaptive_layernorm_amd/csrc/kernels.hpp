// kernels.hpp -- kernel argument blocks and launchers (internal to libalnp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alnp {

// Operand forms of the FP8 producers.
enum Form {
    kNone = 0,    // LayerNorm only: scale = shift = 0
    kBcast = 1,   // bf16 (dim,) scale / shift
    kPtok = 2,    // bf16 (rows, dim) scale / shift
    kTable = 3,   // bf16 temb (rows, chunks, dim) chunk + fp32 table (chunks, dim) row
    kModFp8 = 4,  // e4m3 (dim,) scale / shift times fp32 dequantization scalars
    kAwq = 5      // bf16 (dim,) scale / shift, then y * inv_s[j] (bf16 (dim,))
};

// Arguments of the FP8 producers.  Unused operand pointers are null.
struct Fp8Args {
    const uint16_t* x;
    const uint16_t* scale;      // broadcast (dim,) or per-token (rows, dim)
    const uint16_t* shift;
    const uint16_t* temb;       // table form: (rows, chunks, dim)
    const float* table;         // table form: (chunks, dim)
    int64_t chunks;
    int64_t shift_idx;
    int64_t scale_idx;
    const uint8_t* scale_fp8;   // modfp8 form: e4m3 (dim,)
    const uint8_t* shift_fp8;
    const float* scale_deq;     // modfp8 form: device fp32 scalars
    const float* shift_deq;
    const uint16_t* inv_s;      // AWQ form: bf16 (dim,)
    const float* act_scale;     // device scalar
    float eps;
    int64_t rows;
    int dim;
    uint8_t* out;
    float* row_mean;
    float* row_rstd;
    float inv_dim;              // 1 / dim in fp32, set by the launcher
    uint8_t* mx_scales;         // MXFP8: (rows, dim/32) E8M0 block scales; null otherwise
};

// Block-scale layouts of the FP4 producers.
enum SfLayout {
    kSfRowMajor = 0,  // (rows, dim/16)
    kSfSwizzled = 1   // 128x4 tiles (see sf_swizzled_offset)
};

struct Fp4Args {
    const uint16_t* x;
    const uint16_t* scale;   // broadcast form: (dim,) bf16
    const uint16_t* shift;
    float eps;
    int64_t rows;
    int dim;
    uint8_t* packed;
    uint8_t* sf;
    int sf_layout;
    float* row_mean;
    float* row_rstd;
    float inv_dim;           // 1 / dim in fp32, set by the launcher
    int form;                // kNone, kBcast (scale/shift) or kModFp8 (the fields below)
    int mx;                  // 1: MXFP4, sf = (rows, dim/32) E8M0 scales (sf_layout row-major)
    const uint8_t* scale_fp8;  // modfp8 form: e4m3 (dim,)
    const uint8_t* shift_fp8;
    const float* scale_deq;    // modfp8 form: device fp32 scalars
    const float* shift_deq;
};

struct Mod6Args {
    const float* params;     // (tokens, 6, dim)
    const float* mod;        // (6, dim)
    int64_t tokens;
    int dim;
    uint16_t* out[6];
};

struct GateArgs {
    const uint16_t* residual;  // (rows, dim)
    const uint16_t* gate;      // (gate_rows, dim), gate_rows 1 or rows
    const uint16_t* proj;      // (rows, dim)
    int64_t rows;
    int dim;
    int64_t gate_rows;
    uint16_t* out;             // (rows, dim), may be residual
};

struct RmsArgs {
    const uint16_t* x;         // (rows, dim)
    const uint16_t* weight;    // (dim,) or null
    const uint16_t* scale;     // (segments, dim)
    const uint16_t* shift;     // (segments, dim)
    const int32_t* seg;        // (rows,) table row per row
    int64_t segments;
    float eps;
    int64_t rows;
    int dim;
    uint16_t* out;             // (rows, dim)
    float* row_rstd;           // (rows,) or null
    float inv_dim;             // 1 / dim in fp32, set by the launcher
};

// Largest row (elements) the register-resident row kernels take: 8 waves,
// 8 vectors of 8 elements per thread.
constexpr int kMaxFastDim = 8 * 64 * 8 * 8;

// Launch shape of the row kernels for a row of dim elements (dim % 8 == 0,
// dim <= kMaxFastDim): threads per workgroup and 16-byte vectors per thread.
struct RowShape {
    int threads;
    int vpt;
};
RowShape row_shape(int dim);

// Bytes of the 128x4 tiled block-scale buffer for (rows, cols = dim/16)
// scales: both dimensions rounded up to the tile.
inline int64_t sf_swizzled_size(int64_t rows, int64_t cols)
{
    return (rows + 127) / 128 * 128 * ((cols + 3) / 4 * 4);
}

// form: a Form.
// fast: row kernel (dim % 8 == 0, dim <= kMaxFastDim, operands
// 16-byte aligned); otherwise the workgroup-per-row kernel.
hipError_t launch_adaln_fp8(const Fp8Args& a, int form, bool fast, hipStream_t s);
// LayerNorm, broadcast AdaLN or modfp8 AdaLN (a.form) -> FP4, row-major or
// tiled scales (the modfp8 form only with tiled scales).
hipError_t launch_fp4(const Fp4Args& a, bool fast, hipStream_t s);
hipError_t launch_modulation6(const Mod6Args& a, bool fast, hipStream_t s);
// fast: dim % 8 == 0 and every pointer 16-byte aligned.
hipError_t launch_gated_residual(const GateArgs& a, bool fast, hipStream_t s);
hipError_t launch_quant_fp8(const float* v, const float* act, int64_t n, uint8_t* out,
                            hipStream_t s);
// MXFP8 (a.mx_scales non-null, act_scale unused): form kNone, kBcast, kPtok or kTable.
hipError_t launch_mxfp8(const Fp8Args& a, int form, bool fast, hipStream_t s);
// fast: as for launch_adaln_fp8 (x, out, weight and tables 16-byte aligned).
hipError_t launch_rms_modulate(const RmsArgs& a, bool fast, hipStream_t s);

}  // namespace alnp
