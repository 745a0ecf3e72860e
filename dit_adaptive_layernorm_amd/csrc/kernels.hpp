// kernels.hpp -- kernel argument blocks and launchers (internal to libalnp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alnp {

// Arguments of the FP8 producers.  Unused operand pointers are null.
struct Fp8Args {
    const uint16_t* x;
    const uint16_t* scale;   // broadcast (dim,) or per-token (rows, dim)
    const uint16_t* shift;
    const uint16_t* temb;    // table form: (rows, chunks, dim)
    const float* table;      // table form: (chunks, dim)
    int64_t chunks;
    int64_t shift_idx;
    int64_t scale_idx;
    const float* act_scale;  // device scalar
    float eps;
    int64_t rows;
    int dim;
    uint8_t* out;
    float* row_mean;
    float* row_rstd;
};

struct Fp4Args {
    const uint16_t* x;
    float eps;
    int64_t rows;
    int dim;
    uint8_t* packed;
    uint8_t* sf;
    float* row_mean;
    float* row_rstd;
};

struct Mod6Args {
    const float* params;     // (tokens, 6, dim)
    const float* mod;        // (6, dim)
    int64_t tokens;
    int dim;
    uint16_t* out[6];
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

// form: 0 LayerNorm only, 1 broadcast, 2 per-token, 3 table.
// fast: row kernel (dim % 8 == 0, dim <= kMaxFastDim, operands
// 16-byte aligned); otherwise the workgroup-per-row kernel.
hipError_t launch_adaln_fp8(const Fp8Args& a, int form, bool fast, hipStream_t s);
hipError_t launch_ln_fp4(const Fp4Args& a, bool fast, hipStream_t s);
hipError_t launch_modulation6(const Mod6Args& a, bool fast, hipStream_t s);
hipError_t launch_quant_fp8(const float* v, const float* act, int64_t n, uint8_t* out,
                            hipStream_t s);

}  // namespace alnp
