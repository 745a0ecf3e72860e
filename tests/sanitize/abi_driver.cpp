// Every C-ABI entry point called with arguments that fail each validation
// rule, with valid arguments (the launchers are stand-ins), and with extreme
// sizes, under the address and undefined-behaviour sanitizers.  Exit status 0
// when every call returned the expected status.
#include "alnp.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

namespace {

alignas(256) unsigned char buf[1 << 16];
int failures = 0;

void expect(int got, int want, const char* what, int line)
{
    if (got != want) {
        std::printf("line %d: %s returned %d, expected %d\n", line, what, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

template <typename T>
T* P(int off = 0) { return reinterpret_cast<T*>(buf + off); }

const uint16_t* X = P<const uint16_t>(0);
const uint16_t* S = P<const uint16_t>(4096);
const uint16_t* H = P<const uint16_t>(8192);
const float* F = P<const float>(12288);
uint8_t* O = P<uint8_t>(16384);
uint8_t* SC = P<uint8_t>(20480);
const uint8_t* E8 = P<const uint8_t>(24576);
uint16_t* B16 = P<uint16_t>(28672);
const int32_t* SEG = P<const int32_t>(32768);
const float NaN = std::numeric_limits<float>::quiet_NaN();
const int64_t kBig = std::numeric_limits<int64_t>::max();

void fp8_family()
{
    EXPECT(alnp_ada_layer_norm_quant_fp8_bf16(X, S, H, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_fp8_bf16(X, nullptr, H, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_ada_layer_norm_quant_fp8_bf16(X, S, H, F, 1e-5f, 4, 63, O, nullptr, nullptr, nullptr), ALNP_ERR_DIM);
    EXPECT(alnp_ada_layer_norm_quant_fp8_bf16(X, S, H, F, NaN, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_ARG);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_bf16(X + 1, S, H, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_bf16(X, S, H, F, 1e-5f, -1, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_bf16(X, S, H, F, 1e-5f, kBig, kBig, O, nullptr, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_bf16(X, S, H, F, 1e-5f, 4, 64, O, P<float>(2), nullptr, nullptr), ALNP_ERR_ALIGN);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(X, S, F, 6, 0, 5, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(X, S, F, 6, 6, 5, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_INDEX);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(X, S, F, kBig, 0, 1, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(X, S, F, 6, -kBig, 1, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_INDEX);
    EXPECT(alnp_layer_norm_no_affine_quant_fp8_static_bf16(X, F, 1e-5f, 513, 3072, O, P<float>(0), P<float>(4096), nullptr), ALNP_OK);
    EXPECT(alnp_layer_norm_no_affine_quant_fp8_static_bf16(X, nullptr, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_ada_layer_norm_quant_fp8_modfp8_bf16(X, E8, E8, F, F, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_fp8_modfp8_bf16(X, E8, nullptr, F, F, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_awq_ada_layer_norm_quant_fp8_bf16(X, S, H, S, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_awq_ada_layer_norm_quant_fp8_bf16(X, S, H, nullptr, F, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_quant_fp8_static_f32(F, F, 1000, O, nullptr), ALNP_OK);
    EXPECT(alnp_quant_fp8_static_f32(F, F, kBig, O, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_quant_fp8_static_f32(F, F, 0, nullptr, nullptr), ALNP_OK);
}

void fp4_and_mx_family()
{
    EXPECT(alnp_layer_norm_no_affine_quant_nvfp4_bf16(X, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_layer_norm_no_affine_quant_nvfp4_bf16(X, 1e-5f, 4, 40, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_DIM);
    EXPECT(alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16(X, 1e-5f, 130, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_nvfp4_bf16(X, S, nullptr, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16(X, S, H, -1.0f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_ARG);
    EXPECT(alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(X, E8, E8, F, F, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(X, E8, E8, F, P<const float>(2), 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_ALIGN);
    EXPECT(alnp_layer_norm_no_affine_quant_mxfp8_bf16(X, 1e-5f, 4, 96, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_mxfp8_bf16(X, S, H, 1e-5f, 4, 48, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_DIM);
    EXPECT(alnp_ada_layer_norm_quant_mxfp8_ptok_bf16(X, S, H, 1e-5f, 4, 64, O, nullptr, nullptr, nullptr, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(X, S, F, 6, 2, 3, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(X, S, F, 6, 2, 7, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_INDEX);
    EXPECT(alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16(X, E8, E8, F, F, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_awq_ada_layer_norm_quant_mxfp8_bf16(X, S, H, S, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_layer_norm_no_affine_quant_mxfp4_bf16(X, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_ada_layer_norm_quant_mxfp4_bf16(X, S, H, 1e-5f, kBig, 64, O, SC, nullptr, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16(X, E8, E8, F, F, 1e-5f, 4, 64, O, SC, nullptr, nullptr, nullptr), ALNP_OK);
    const int64_t extents[] = {0, 1, 16, 32, 40, 129, -16, kBig, -kBig};
    for (int64_t r : extents)
        for (int64_t d : extents) {
            (void)alnp_sf_size(r, d);
            (void)alnp_swizzled_sf_size(r, d);
            (void)alnp_mx_scale_size(r, d);
        }
    EXPECT((int)alnp_sf_size(4, 64), 16);
    EXPECT((int)alnp_swizzled_sf_size(129, 64), 2 * 512);
    EXPECT((int)alnp_mx_scale_size(4, 64), 8);
}

void other_entries()
{
    uint16_t* outs[6] = {B16, B16 + 512, B16 + 1024, B16 + 1536, B16 + 2048, B16 + 2560};
    EXPECT(alnp_adaln_modulation6_bf16(F, F, 1, 51, 1536, outs, nullptr), ALNP_OK);
    EXPECT(alnp_adaln_modulation6_bf16(F, F, kBig, kBig, 1536, outs, nullptr), ALNP_ERR_SHAPE);
    outs[3] = nullptr;
    EXPECT(alnp_adaln_modulation6_bf16(F, F, 1, 51, 1536, outs, nullptr), ALNP_ERR_NULL);
    EXPECT(alnp_gated_residual_bf16(X, S, H, 4, 64, 1, B16, nullptr), ALNP_OK);
    EXPECT(alnp_gated_residual_bf16(X, S, H, 4, 64, 2, B16, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_gated_residual_bf16(X, S, H, kBig, 64, 1, B16, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_rms_norm_modulate_seg_bf16(X, S, S, H, SEG, 3, 1e-6f, 4, 5376, B16, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_rms_norm_modulate_seg_bf16(X, nullptr, S, H, SEG, 3, 1e-6f, 4097, 64, B16, nullptr, nullptr), ALNP_OK);
    EXPECT(alnp_rms_norm_modulate_seg_bf16(X, S, S, H, SEG, 0, 1e-6f, 4, 64, B16, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_rms_norm_modulate_seg_bf16(X, S, S, H, SEG, kBig, 1e-6f, 4, 64, B16, nullptr, nullptr), ALNP_ERR_SHAPE);
    EXPECT(alnp_rms_norm_modulate_seg_bf16(X, S, S, H, P<const int32_t>(2), 3, 1e-6f, 4, 64, B16, nullptr, nullptr), ALNP_ERR_ALIGN);
    for (int s = -8; s <= 1; ++s)
        (void)alnp_status_string(s);
    EXPECT(alnp_abi_version(), 1);
}

}  // namespace

int main()
{
    fp8_family();
    fp4_and_mx_family();
    other_entries();
    std::printf("%d failures\n", failures);
    return failures ? 1 : 0;
}
