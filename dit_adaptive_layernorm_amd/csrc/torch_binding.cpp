// torch_binding.cpp -- the package's functions as compiled code.
//
// Every function takes torch tensors, runs on the device of its first tensor
// (as torch's own operators do), checks them (GPU, that device, dtype, shape,
// contiguity), allocates the outputs it is not given, and calls the C ABI of
// libalnp.so (include/alnp.h) on torch's current stream of that device.
// Doing this in C++ saves the Python-level checks and ctypes marshalling,
// about 3 us per call.  Nothing here computes; errors raise ValueError,
// TypeError, or the package's AlnpError for a status from the library.  The
// tests check every function against an independent ctypes marshalling.
#include <torch/extension.h>
#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPFunctions.h>
#include <c10/hip/HIPStream.h>

#include <string>
#include <vector>

#include "alnp.h"

namespace py = pybind11;
using at::Tensor;
using OptT = c10::optional<Tensor>;

namespace {

py::object g_error;  // the package's AlnpError class, registered at import

[[noreturn]] void fail(const char* fn, int status)
{
    if (g_error) {
        py::object e = g_error(fn, status);
        PyErr_SetObject(g_error.ptr(), e.ptr());
        throw py::error_already_set();
    }
    throw std::runtime_error(std::string(fn) + ": " + alnp_status_string(status));
}

inline void check(const char* fn, int status)
{
    if (status != 0)
        fail(fn, status);
}

std::string shape_str(at::IntArrayRef s)
{
    std::string r = "(";
    for (size_t i = 0; i < s.size(); ++i)
        r += (i ? ", " : "") + std::to_string(s[i]) + (s.size() == 1 ? "," : "");
    return r + ")";
}

// Index of the GPU the running call is on (set by CallDevice, read by the
// tensor checks without asking the runtime again for every tensor).
thread_local int t_call_device = -1;

// The device a call runs on: that of its first tensor, as for torch's own
// operators.  A guard makes it the current device for the call (nothing to
// switch when it already is) and restores the previous one afterwards.
class CallDevice {
public:
    explicit CallDevice(const Tensor& first)
        : guard_(first.is_cuda() ? c10::make_optional(first.device()) : c10::nullopt),
          saved_(t_call_device)
    {
        t_call_device = first.is_cuda() ? first.get_device() : -1;
    }
    ~CallDevice() { t_call_device = saved_; }
    CallDevice(const CallDevice&) = delete;
    CallDevice& operator=(const CallDevice&) = delete;

private:
    c10::OptionalDeviceGuard guard_;
    int saved_;
};

// A GPU tensor on the call's device, else ValueError.  A first tensor that
// is not on the GPU leaves no call device (-1); the call then fails on that
// tensor's own check, which every function makes.
void on_call_device(const Tensor& t, const char* name)
{
    if (!t.is_cuda())
        throw py::value_error(std::string(name) + " must be on the GPU");
    if (t_call_device >= 0 && t.get_device() != t_call_device)
        throw py::value_error(std::string(name) + " must be on cuda:" +
                              std::to_string(t_call_device) + ", the device of the call, got " +
                              t.device().str());
}

// GPU, device, dtype, (shape,) contiguity, in that order (the order of the
// first failing check decides the error).
void dev(const Tensor& t, const char* name, at::ScalarType dt)
{
    on_call_device(t, name);
    if (t.scalar_type() != dt)
        throw py::type_error(std::string(name) + " must be " + c10::toString(dt) + ", got " +
                             c10::toString(t.scalar_type()));
    if (!t.is_contiguous())
        throw py::value_error(std::string(name) + " must be contiguous");
}

void dev(const Tensor& t, const char* name, at::ScalarType dt, at::IntArrayRef shape)
{
    on_call_device(t, name);
    if (t.scalar_type() != dt)
        throw py::type_error(std::string(name) + " must be " + c10::toString(dt) + ", got " +
                             c10::toString(t.scalar_type()));
    if (t.sizes() != shape)
        throw py::value_error(std::string(name) + " must have shape " + shape_str(shape) +
                              ", got " + shape_str(t.sizes()));
    if (!t.is_contiguous())
        throw py::value_error(std::string(name) + " must be contiguous");
}

template <typename T>
T* ptr(const Tensor& t) { return static_cast<T*>(t.data_ptr()); }

void* stream() { return c10::hip::getCurrentHIPStream().stream(); }

// x: (rows, dim) bf16.
void check_x(const Tensor& x, int64_t& rows, int64_t& dim)
{
    dev(x, "x", at::kBFloat16);
    if (x.dim() != 2)
        throw py::value_error("x must be 2-D (rows, dim)");
    rows = x.size(0);
    dim = x.size(1);
}

const float* act(const Tensor& t, const char* name = "act_scale")
{
    dev(t, name, at::kFloat);
    if (t.numel() != 1)
        throw py::value_error(std::string(name) + " must hold one fp32 value");
    return ptr<const float>(t);
}

float* opt_f32(const OptT& t, const char* name, int64_t rows)
{
    if (!t)
        return nullptr;
    dev(*t, name, at::kFloat, {rows});
    return ptr<float>(*t);
}

Tensor fp8_out(const OptT& out, const Tensor& x)
{
    Tensor o = out ? *out : at::empty(x.sizes(), x.options().dtype(at::kFloat8_e4m3fn));
    dev(o, "out", at::kFloat8_e4m3fn, x.sizes());
    return o;
}

// ---- FP8 producers ----------------------------------------------------------------

Tensor ada_fp8_bcast(const Tensor& x, const Tensor& scale, const Tensor& shift,
                     const Tensor& act_scale, double eps, const OptT& out, const OptT& row_mean,
                     const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor o = fp8_out(out, x);
    dev(scale, "scale", at::kBFloat16, {dim});
    dev(shift, "shift", at::kBFloat16, {dim});
    check("alnp_ada_layer_norm_quant_fp8_bf16",
          alnp_ada_layer_norm_quant_fp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(scale), ptr<const uint16_t>(shift),
              act(act_scale), (float)eps, rows, dim, ptr<uint8_t>(o),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor ada_fp8_ptok(const Tensor& x, const Tensor& scale, const Tensor& shift,
                    const Tensor& act_scale, double eps, const OptT& out, const OptT& row_mean,
                    const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor o = fp8_out(out, x);
    dev(scale, "scale", at::kBFloat16, {rows, dim});
    dev(shift, "shift", at::kBFloat16, {rows, dim});
    check("alnp_ada_layer_norm_quant_fp8_ptok_bf16",
          alnp_ada_layer_norm_quant_fp8_ptok_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(scale), ptr<const uint16_t>(shift),
              act(act_scale), (float)eps, rows, dim, ptr<uint8_t>(o),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor ada_fp8_table(const Tensor& x, const Tensor& temb, const Tensor& table,
                     const Tensor& act_scale, int64_t shift_idx, int64_t scale_idx, double eps,
                     const OptT& out, const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    if (temb.dim() != 3)
        throw py::value_error("temb must be (rows, chunks, dim)");
    const int64_t chunks = temb.size(1);
    Tensor o = fp8_out(out, x);
    dev(temb, "temb", at::kBFloat16, {rows, chunks, dim});
    dev(table, "table", at::kFloat, {chunks, dim});
    check("alnp_ada_layer_norm_quant_fp8_ptok_table_bf16",
          alnp_ada_layer_norm_quant_fp8_ptok_table_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(temb), ptr<const float>(table), chunks,
              shift_idx, scale_idx, act(act_scale), (float)eps, rows, dim, ptr<uint8_t>(o),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor ada_fp8_modfp8(const Tensor& x, const Tensor& scale_fp8, const Tensor& shift_fp8,
                      const Tensor& scale_deq, const Tensor& shift_deq, const Tensor& act_scale,
                      double eps, const OptT& out, const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor o = fp8_out(out, x);
    dev(scale_fp8, "scale_fp8", at::kFloat8_e4m3fn, {dim});
    dev(shift_fp8, "shift_fp8", at::kFloat8_e4m3fn, {dim});
    check("alnp_ada_layer_norm_quant_fp8_modfp8_bf16",
          alnp_ada_layer_norm_quant_fp8_modfp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint8_t>(scale_fp8), ptr<const uint8_t>(shift_fp8),
              act(scale_deq, "scale_deq"), act(shift_deq, "shift_deq"), act(act_scale),
              (float)eps, rows, dim, ptr<uint8_t>(o), opt_f32(row_mean, "row_mean", rows),
              opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor awq_fp8(const Tensor& x, const Tensor& scale, const Tensor& shift, const Tensor& inv_s,
               const Tensor& act_scale, double eps, const OptT& out, const OptT& row_mean,
               const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor o = fp8_out(out, x);
    dev(scale, "scale", at::kBFloat16, {dim});
    dev(shift, "shift", at::kBFloat16, {dim});
    dev(inv_s, "inv_s", at::kBFloat16, {dim});
    check("alnp_awq_ada_layer_norm_quant_fp8_bf16",
          alnp_awq_ada_layer_norm_quant_fp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(scale), ptr<const uint16_t>(shift),
              ptr<const uint16_t>(inv_s), act(act_scale), (float)eps, rows, dim, ptr<uint8_t>(o),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor ln_fp8(const Tensor& x, const Tensor& act_scale, double eps, const OptT& out,
              const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor o = fp8_out(out, x);
    check("alnp_layer_norm_no_affine_quant_fp8_static_bf16",
          alnp_layer_norm_no_affine_quant_fp8_static_bf16(
              ptr<const uint16_t>(x), act(act_scale), (float)eps, rows, dim, ptr<uint8_t>(o),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

Tensor quant_fp8(const Tensor& v, const Tensor& act_scale, const OptT& out)
{
    const CallDevice call(v);
    dev(v, "v", at::kFloat);
    Tensor o = out ? *out : at::empty(v.sizes(), v.options().dtype(at::kFloat8_e4m3fn));
    dev(o, "out", at::kFloat8_e4m3fn, v.sizes());
    check("alnp_quant_fp8_static_f32",
          alnp_quant_fp8_static_f32(ptr<const float>(v), act(act_scale), v.numel(),
                                    ptr<uint8_t>(o), stream()));
    return o;
}

// ---- FP4 producers ----------------------------------------------------------------

int64_t size_or_fail(const char* fn, int64_t n)
{
    if (n < 0)
        fail(fn, (int)n);
    return n;
}

// Outputs of the NVFP4 functions.  strict_sf: the (rows, dim // 16) shape is
// required (row-major LN entry); otherwise only the byte count is.
std::pair<Tensor, Tensor> fp4_outputs(const Tensor& x, int64_t rows, int64_t dim, const OptT& packed,
                                      const OptT& sf, bool swizzled, bool strict_sf)
{
    if (dim % 16)
        throw py::value_error("dim must be a multiple of 16");
    Tensor p = packed ? *packed : at::empty({rows, dim / 2}, x.options().dtype(at::kByte));
    const int64_t n_sf = swizzled ? size_or_fail("alnp_swizzled_sf_size", alnp_swizzled_sf_size(rows, dim))
                                  : size_or_fail("alnp_sf_size", alnp_sf_size(rows, dim));
    Tensor s;
    if (sf)
        s = *sf;
    else if (strict_sf)
        s = at::empty({rows, dim / 16}, x.options().dtype(at::kFloat8_e4m3fn));
    else if (swizzled)
        s = at::empty({n_sf}, x.options().dtype(at::kByte));
    else
        s = at::empty({rows, dim / 16}, x.options().dtype(at::kByte));
    dev(p, "packed", at::kByte, {rows, dim / 2});
    if (s.scalar_type() != at::kByte && s.scalar_type() != at::kFloat8_e4m3fn)
        throw py::type_error("sf must be uint8 or float8_e4m3fn");
    if (strict_sf) {
        dev(s, "sf", s.scalar_type(), {rows, dim / 16});
    } else {
        dev(s, "sf", s.scalar_type());
        if (s.numel() != n_sf)
            throw py::value_error("sf must hold " + std::to_string(n_sf) + " bytes, got " +
                                  std::to_string(s.numel()));
    }
    return {p, s};
}

py::tuple ln_nvfp4(const Tensor& x, double eps, const OptT& packed, const OptT& sf,
                   const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    auto [p, s] = fp4_outputs(x, rows, dim, packed, sf, false, true);
    check("alnp_layer_norm_no_affine_quant_nvfp4_bf16",
          alnp_layer_norm_no_affine_quant_nvfp4_bf16(
              ptr<const uint16_t>(x), (float)eps, rows, dim, ptr<uint8_t>(p), ptr<uint8_t>(s),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(p, s);
}

py::tuple ln_nvfp4_swizzled(const Tensor& x, double eps, const OptT& packed, const OptT& sf,
                            const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    auto [p, s] = fp4_outputs(x, rows, dim, packed, sf, true, false);
    check("alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16",
          alnp_layer_norm_no_affine_quant_nvfp4_swizzled_bf16(
              ptr<const uint16_t>(x), (float)eps, rows, dim, ptr<uint8_t>(p), ptr<uint8_t>(s),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(p, s);
}

py::tuple ada_nvfp4(const Tensor& x, const Tensor& scale, const Tensor& shift, double eps,
                    const OptT& packed, const OptT& sf, const OptT& row_mean, const OptT& row_rstd,
                    bool swizzled)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    auto [p, s] = fp4_outputs(x, rows, dim, packed, sf, swizzled, false);
    dev(scale, "scale", at::kBFloat16, {dim});
    dev(shift, "shift", at::kBFloat16, {dim});
    auto fn = swizzled ? alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16 : alnp_ada_layer_norm_quant_nvfp4_bf16;
    check(swizzled ? "alnp_ada_layer_norm_quant_nvfp4_swizzled_bf16" : "alnp_ada_layer_norm_quant_nvfp4_bf16",
          fn(ptr<const uint16_t>(x), ptr<const uint16_t>(scale), ptr<const uint16_t>(shift),
             (float)eps, rows, dim, ptr<uint8_t>(p), ptr<uint8_t>(s),
             opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(p, s);
}

py::tuple ada_nvfp4_swizzled_modfp8(const Tensor& x, const Tensor& scale_fp8,
                                    const Tensor& shift_fp8, const Tensor& scale_deq,
                                    const Tensor& shift_deq, double eps, const OptT& packed,
                                    const OptT& sf, const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    auto [p, s] = fp4_outputs(x, rows, dim, packed, sf, true, false);
    dev(scale_fp8, "scale_fp8", at::kFloat8_e4m3fn, {dim});
    dev(shift_fp8, "shift_fp8", at::kFloat8_e4m3fn, {dim});
    check("alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16",
          alnp_ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint8_t>(scale_fp8), ptr<const uint8_t>(shift_fp8),
              act(scale_deq, "scale_deq"), act(shift_deq, "shift_deq"), (float)eps, rows, dim,
              ptr<uint8_t>(p), ptr<uint8_t>(s), opt_f32(row_mean, "row_mean", rows),
              opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(p, s);
}

// ---- MX block formats ---------------------------------------------------------------

Tensor mx_scales(const Tensor& x, int64_t rows, int64_t dim, const OptT& scales)
{
    if (dim % 32)
        throw py::value_error("dim must be a multiple of 32");
    Tensor s = scales ? *scales : at::empty({rows, dim / 32}, x.options().dtype(at::kByte));
    if (s.scalar_type() != at::kByte && s.scalar_type() != at::kFloat8_e8m0fnu)
        throw py::type_error("scales must be uint8 (E8M0 bytes)");
    dev(s, "scales", s.scalar_type(), {rows, dim / 32});
    return s;
}

// form: 0 LN, 1 broadcast (dim,), 2 per-token (rows, dim)
py::tuple mxfp8(const Tensor& x, const c10::optional<Tensor>& scale,
                const c10::optional<Tensor>& shift, double eps, const OptT& out,
                const OptT& scales, const OptT& row_mean, const OptT& row_rstd, int form)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor o = fp8_out(out, x);
    float* mp = opt_f32(row_mean, "row_mean", rows);
    float* rp = opt_f32(row_rstd, "row_rstd", rows);
    if (form == 0) {
        check("alnp_layer_norm_no_affine_quant_mxfp8_bf16",
              alnp_layer_norm_no_affine_quant_mxfp8_bf16(ptr<const uint16_t>(x), (float)eps, rows,
                                                         dim, ptr<uint8_t>(o), ptr<uint8_t>(s), mp,
                                                         rp, stream()));
        return py::make_tuple(o, s);
    }
    const Tensor& sc = *scale;
    const Tensor& sh = *shift;
    if (form == 1) {
        dev(sc, "scale", at::kBFloat16, {dim});
        dev(sh, "shift", at::kBFloat16, {dim});
        check("alnp_ada_layer_norm_quant_mxfp8_bf16",
              alnp_ada_layer_norm_quant_mxfp8_bf16(ptr<const uint16_t>(x), ptr<const uint16_t>(sc),
                                                   ptr<const uint16_t>(sh), (float)eps, rows, dim,
                                                   ptr<uint8_t>(o), ptr<uint8_t>(s), mp, rp, stream()));
    } else {
        dev(sc, "scale", at::kBFloat16, {rows, dim});
        dev(sh, "shift", at::kBFloat16, {rows, dim});
        check("alnp_ada_layer_norm_quant_mxfp8_ptok_bf16",
              alnp_ada_layer_norm_quant_mxfp8_ptok_bf16(
                  ptr<const uint16_t>(x), ptr<const uint16_t>(sc), ptr<const uint16_t>(sh),
                  (float)eps, rows, dim, ptr<uint8_t>(o), ptr<uint8_t>(s), mp, rp, stream()));
    }
    return py::make_tuple(o, s);
}

py::tuple mxfp8_table(const Tensor& x, const Tensor& temb, const Tensor& table, int64_t shift_idx,
                      int64_t scale_idx, double eps, const OptT& out, const OptT& scales,
                      const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    if (temb.dim() != 3)
        throw py::value_error("temb must be (rows, chunks, dim)");
    const int64_t chunks = temb.size(1);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor o = fp8_out(out, x);
    dev(temb, "temb", at::kBFloat16, {rows, chunks, dim});
    dev(table, "table", at::kFloat, {chunks, dim});
    check("alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16",
          alnp_ada_layer_norm_quant_mxfp8_ptok_table_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(temb), ptr<const float>(table), chunks,
              shift_idx, scale_idx, (float)eps, rows, dim, ptr<uint8_t>(o), ptr<uint8_t>(s),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(o, s);
}

py::tuple mxfp8_modfp8(const Tensor& x, const Tensor& scale_fp8, const Tensor& shift_fp8,
                       const Tensor& scale_deq, const Tensor& shift_deq, double eps,
                       const OptT& out, const OptT& scales, const OptT& row_mean,
                       const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor o = fp8_out(out, x);
    dev(scale_fp8, "scale_fp8", at::kFloat8_e4m3fn, {dim});
    dev(shift_fp8, "shift_fp8", at::kFloat8_e4m3fn, {dim});
    check("alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16",
          alnp_ada_layer_norm_quant_mxfp8_modfp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint8_t>(scale_fp8), ptr<const uint8_t>(shift_fp8),
              act(scale_deq, "scale_deq"), act(shift_deq, "shift_deq"), (float)eps, rows, dim,
              ptr<uint8_t>(o), ptr<uint8_t>(s), opt_f32(row_mean, "row_mean", rows),
              opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(o, s);
}

py::tuple awq_mxfp8(const Tensor& x, const Tensor& scale, const Tensor& shift, const Tensor& inv_s,
                    double eps, const OptT& out, const OptT& scales, const OptT& row_mean,
                    const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor o = fp8_out(out, x);
    dev(scale, "scale", at::kBFloat16, {dim});
    dev(shift, "shift", at::kBFloat16, {dim});
    dev(inv_s, "inv_s", at::kBFloat16, {dim});
    check("alnp_awq_ada_layer_norm_quant_mxfp8_bf16",
          alnp_awq_ada_layer_norm_quant_mxfp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint16_t>(scale), ptr<const uint16_t>(shift),
              ptr<const uint16_t>(inv_s), (float)eps, rows, dim, ptr<uint8_t>(o), ptr<uint8_t>(s),
              opt_f32(row_mean, "row_mean", rows), opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(o, s);
}

py::tuple mxfp4_modfp8(const Tensor& x, const Tensor& scale_fp8, const Tensor& shift_fp8,
                       const Tensor& scale_deq, const Tensor& shift_deq, double eps,
                       const OptT& packed, const OptT& scales, const OptT& row_mean,
                       const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor p = packed ? *packed : at::empty({rows, dim / 2}, x.options().dtype(at::kByte));
    dev(p, "packed", at::kByte, {rows, dim / 2});
    dev(scale_fp8, "scale_fp8", at::kFloat8_e4m3fn, {dim});
    dev(shift_fp8, "shift_fp8", at::kFloat8_e4m3fn, {dim});
    check("alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16",
          alnp_ada_layer_norm_quant_mxfp4_modfp8_bf16(
              ptr<const uint16_t>(x), ptr<const uint8_t>(scale_fp8), ptr<const uint8_t>(shift_fp8),
              act(scale_deq, "scale_deq"), act(shift_deq, "shift_deq"), (float)eps, rows, dim,
              ptr<uint8_t>(p), ptr<uint8_t>(s), opt_f32(row_mean, "row_mean", rows),
              opt_f32(row_rstd, "row_rstd", rows), stream()));
    return py::make_tuple(p, s);
}

py::tuple mxfp4(const Tensor& x, const c10::optional<Tensor>& scale,
                const c10::optional<Tensor>& shift, double eps, const OptT& packed,
                const OptT& scales, const OptT& row_mean, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    Tensor s = mx_scales(x, rows, dim, scales);
    Tensor p = packed ? *packed : at::empty({rows, dim / 2}, x.options().dtype(at::kByte));
    dev(p, "packed", at::kByte, {rows, dim / 2});
    float* mp = opt_f32(row_mean, "row_mean", rows);
    float* rp = opt_f32(row_rstd, "row_rstd", rows);
    if (!scale) {
        check("alnp_layer_norm_no_affine_quant_mxfp4_bf16",
              alnp_layer_norm_no_affine_quant_mxfp4_bf16(ptr<const uint16_t>(x), (float)eps, rows,
                                                         dim, ptr<uint8_t>(p), ptr<uint8_t>(s), mp,
                                                         rp, stream()));
        return py::make_tuple(p, s);
    }
    dev(*scale, "scale", at::kBFloat16, {dim});
    dev(*shift, "shift", at::kBFloat16, {dim});
    check("alnp_ada_layer_norm_quant_mxfp4_bf16",
          alnp_ada_layer_norm_quant_mxfp4_bf16(ptr<const uint16_t>(x), ptr<const uint16_t>(*scale),
                                               ptr<const uint16_t>(*shift), (float)eps, rows, dim,
                                               ptr<uint8_t>(p), ptr<uint8_t>(s), mp, rp, stream()));
    return py::make_tuple(p, s);
}

// ---- six-way modulation, residual gate, RMSNorm modulation --------------------------

py::tuple modulation6(const Tensor& params, const Tensor& mod, const c10::optional<std::vector<Tensor>>& out)
{
    const CallDevice call(params);
    if (params.dim() != 4 || params.size(2) != 6)
        throw py::value_error("adaln_params must be (batch, seq, 6, dim)");
    const int64_t B = params.size(0), S = params.size(1), D = params.size(3);
    dev(params, "adaln_params", at::kFloat);
    dev(mod, "layer_modulation", at::kFloat, {6, D});
    std::vector<Tensor> outs;
    if (out) {
        outs = *out;
    } else {
        for (int k = 0; k < 6; ++k)
            outs.push_back(at::empty({B, S, D}, params.options().dtype(at::kBFloat16)));
    }
    if (outs.size() != 6)
        throw py::value_error("out must hold six tensors");
    uint16_t* ptrs[6];
    for (int k = 0; k < 6; ++k) {
        const std::string name = "out[" + std::to_string(k) + "]";
        dev(outs[k], name.c_str(), at::kBFloat16, {B, S, D});
        ptrs[k] = ptr<uint16_t>(outs[k]);
    }
    check("alnp_adaln_modulation6_bf16",
          alnp_adaln_modulation6_bf16(ptr<const float>(params), ptr<const float>(mod), B, S, D, ptrs,
                                      stream()));
    return py::make_tuple(outs[0], outs[1], outs[2], outs[3], outs[4], outs[5]);
}

Tensor gated_residual(const Tensor& residual, const Tensor& gate, const Tensor& proj, const OptT& out)
{
    const CallDevice call(residual);
    if (residual.dim() != 2)
        throw py::value_error("residual must be 2-D (rows, dim)");
    const int64_t rows = residual.size(0), dim = residual.size(1);
    dev(residual, "residual", at::kBFloat16);
    dev(proj, "proj", at::kBFloat16, {rows, dim});
    int64_t gate_rows;
    if (gate.sizes() == at::IntArrayRef{dim})
        gate_rows = 1;
    else if (gate.sizes() == at::IntArrayRef{rows, dim})
        gate_rows = rows;
    else
        throw py::value_error("gate must be (" + std::to_string(dim) + ",) or (" +
                              std::to_string(rows) + ", " + std::to_string(dim) + ")");
    dev(gate, "gate", at::kBFloat16);
    Tensor o = out ? *out : at::empty_like(residual);
    dev(o, "out", at::kBFloat16, {rows, dim});
    check("alnp_gated_residual_bf16",
          alnp_gated_residual_bf16(ptr<const uint16_t>(residual), ptr<const uint16_t>(gate),
                                   ptr<const uint16_t>(proj), rows, dim, gate_rows,
                                   ptr<uint16_t>(o), stream()));
    return o;
}

Tensor rms_modulate(const Tensor& x, const OptT& weight, const Tensor& scale, const Tensor& shift,
                    const Tensor& seg, double eps, const OptT& out, const OptT& row_rstd)
{
    const CallDevice call(x);
    int64_t rows, dim;
    check_x(x, rows, dim);
    if (scale.dim() != 2)
        throw py::value_error("scale must be (segments, dim)");
    const int64_t segments = scale.size(0);
    const uint16_t* wp = nullptr;
    if (weight) {
        dev(*weight, "weight", at::kBFloat16, {dim});
        wp = ptr<const uint16_t>(*weight);
    }
    Tensor o = out ? *out : at::empty_like(x);
    dev(scale, "scale", at::kBFloat16, {segments, dim});
    dev(shift, "shift", at::kBFloat16, {segments, dim});
    dev(seg, "seg", at::kInt, {rows});
    dev(o, "out", at::kBFloat16, {rows, dim});
    check("alnp_rms_norm_modulate_seg_bf16",
          alnp_rms_norm_modulate_seg_bf16(ptr<const uint16_t>(x), wp, ptr<const uint16_t>(scale),
                                          ptr<const uint16_t>(shift), ptr<const int32_t>(seg),
                                          segments, (float)eps, rows, dim, ptr<uint16_t>(o),
                                          opt_f32(row_rstd, "row_rstd", rows), stream()));
    return o;
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m)
{
    m.doc() = "Compiled argument checks and C-ABI calls for the adaptive-LayerNorm producers.";
    m.def("set_error_class", [](py::object cls) { g_error = cls; });
    const auto none = py::none();
    m.def("ada_layer_norm_quant_fp8_bf16", &ada_fp8_bcast, py::arg("x"), py::arg("scale"),
          py::arg("shift"), py::arg("act_scale"), py::arg("eps") = 1e-5, py::arg("out") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Broadcast AdaLN -> FP8: scale, shift (dim,) bf16.");
    m.def("ada_layer_norm_quant_fp8_ptok_bf16", &ada_fp8_ptok, py::arg("x"), py::arg("scale"),
          py::arg("shift"), py::arg("act_scale"), py::arg("eps") = 1e-5, py::arg("out") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Per-token AdaLN -> FP8: scale, shift (rows, dim) bf16.");
    m.def("ada_layer_norm_quant_fp8_ptok_table_bf16", &ada_fp8_table, py::arg("x"), py::arg("temb"),
          py::arg("table"), py::arg("act_scale"), py::arg("shift_idx"), py::arg("scale_idx"),
          py::arg("eps") = 1e-5, py::arg("out") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none,
          "Table-form per-token AdaLN -> FP8: temb (rows, chunks, dim) bf16, table (chunks, dim) "
          "fp32; operands temb[:, idx] + table[idx].");
    m.def("ada_layer_norm_quant_fp8_modfp8_bf16", &ada_fp8_modfp8, py::arg("x"),
          py::arg("scale_fp8"), py::arg("shift_fp8"), py::arg("scale_deq"), py::arg("shift_deq"),
          py::arg("act_scale"), py::arg("eps") = 1e-5, py::arg("out") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Broadcast AdaLN -> FP8 with e4m3 (dim,) scale/shift and fp32 device dequantization "
          "scalars.");
    m.def("awq_ada_layer_norm_quant_fp8_bf16", &awq_fp8, py::arg("x"), py::arg("scale"),
          py::arg("shift"), py::arg("inv_s"), py::arg("act_scale"), py::arg("eps") = 1e-5,
          py::arg("out") = none, py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Broadcast AdaLN -> per-channel inv_s (dim,) bf16 -> FP8.");
    m.def("layer_norm_no_affine_quant_fp8_static_bf16", &ln_fp8, py::arg("x"),
          py::arg("act_scale"), py::arg("eps") = 1e-5, py::arg("out") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none, "LayerNorm (no affine) -> FP8.");
    m.def("quant_fp8_static_f32", &quant_fp8, py::arg("v"), py::arg("act_scale"),
          py::arg("out") = none, "e4m3(v * (1 / act_scale)), saturating; v fp32 of any shape.");
    m.def("layer_norm_no_affine_quant_nvfp4_bf16", &ln_nvfp4, py::arg("x"), py::arg("eps") = 1e-5,
          py::arg("packed") = none, py::arg("sf") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none,
          "LayerNorm (no affine) -> e2m1 packed (rows, dim // 2) uint8 (low nibble first) + e4m3 "
          "block scales (rows, dim // 16), row-major.");
    m.def("layer_norm_no_affine_quant_nvfp4_swizzled_bf16", &ln_nvfp4_swizzled, py::arg("x"),
          py::arg("eps") = 1e-5, py::arg("packed") = none, py::arg("sf_swizzled") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "LayerNorm (no affine) -> e2m1 packed + e4m3 block scales in the 128x4 tiled layout.");
    m.def("ada_layer_norm_quant_nvfp4_bf16",
          [](const Tensor& x, const Tensor& scale, const Tensor& shift, double eps,
             const OptT& packed, const OptT& sf, const OptT& row_mean, const OptT& row_rstd) {
              return ada_nvfp4(x, scale, shift, eps, packed, sf, row_mean, row_rstd, false);
          },
          py::arg("x"), py::arg("scale"), py::arg("shift"), py::arg("eps") = 1e-5,
          py::arg("packed") = none, py::arg("sf") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none,
          "Broadcast AdaLN -> e2m1 packed + row-major e4m3 block scales.");
    m.def("ada_layer_norm_quant_nvfp4_swizzled_bf16",
          [](const Tensor& x, const Tensor& scale, const Tensor& shift, double eps,
             const OptT& packed, const OptT& sf, const OptT& row_mean, const OptT& row_rstd) {
              return ada_nvfp4(x, scale, shift, eps, packed, sf, row_mean, row_rstd, true);
          },
          py::arg("x"), py::arg("scale"), py::arg("shift"), py::arg("eps") = 1e-5,
          py::arg("packed") = none, py::arg("sf_swizzled") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none,
          "Broadcast AdaLN -> e2m1 packed + e4m3 block scales in the 128x4 tiled layout.");
    m.def("ada_layer_norm_quant_nvfp4_swizzled_modfp8_bf16", &ada_nvfp4_swizzled_modfp8,
          py::arg("x"), py::arg("scale_fp8"), py::arg("shift_fp8"), py::arg("scale_deq"),
          py::arg("shift_deq"), py::arg("eps") = 1e-5, py::arg("packed") = none,
          py::arg("sf_swizzled") = none, py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars -> e2m1 "
          "packed + e4m3 block scales in the 128x4 tiled layout.");
    m.def("layer_norm_no_affine_quant_mxfp8_bf16",
          [](const Tensor& x, double eps, const OptT& out, const OptT& scales, const OptT& row_mean,
             const OptT& row_rstd) {
              return mxfp8(x, c10::nullopt, c10::nullopt, eps, out, scales, row_mean, row_rstd, 0);
          },
          py::arg("x"), py::arg("eps") = 1e-5, py::arg("out") = none, py::arg("scales") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "LayerNorm (no affine) -> MXFP8: e4m3 (rows, dim) + E8M0 (rows, dim // 32).");
    m.def("ada_layer_norm_quant_mxfp8_bf16",
          [](const Tensor& x, const Tensor& scale, const Tensor& shift, double eps, const OptT& out,
             const OptT& scales, const OptT& row_mean, const OptT& row_rstd) {
              return mxfp8(x, scale, shift, eps, out, scales, row_mean, row_rstd, 1);
          },
          py::arg("x"), py::arg("scale"), py::arg("shift"), py::arg("eps") = 1e-5,
          py::arg("out") = none, py::arg("scales") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none, "Broadcast AdaLN -> MXFP8; scale, shift (dim,) bf16.");
    m.def("ada_layer_norm_quant_mxfp8_ptok_bf16",
          [](const Tensor& x, const Tensor& scale, const Tensor& shift, double eps, const OptT& out,
             const OptT& scales, const OptT& row_mean, const OptT& row_rstd) {
              return mxfp8(x, scale, shift, eps, out, scales, row_mean, row_rstd, 2);
          },
          py::arg("x"), py::arg("scale"), py::arg("shift"), py::arg("eps") = 1e-5,
          py::arg("out") = none, py::arg("scales") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none, "Per-token AdaLN -> MXFP8; scale, shift (rows, dim) bf16.");
    m.def("ada_layer_norm_quant_mxfp8_ptok_table_bf16", &mxfp8_table, py::arg("x"),
          py::arg("temb"), py::arg("table"), py::arg("shift_idx"), py::arg("scale_idx"),
          py::arg("eps") = 1e-5, py::arg("out") = none, py::arg("scales") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Table-form AdaLN -> MXFP8: temb (rows, chunks, dim) bf16, table (chunks, dim) fp32; "
          "operands temb[:, idx] + table[idx].");
    m.def("layer_norm_no_affine_quant_mxfp4_bf16",
          [](const Tensor& x, double eps, const OptT& packed, const OptT& scales,
             const OptT& row_mean, const OptT& row_rstd) {
              return mxfp4(x, c10::nullopt, c10::nullopt, eps, packed, scales, row_mean, row_rstd);
          },
          py::arg("x"), py::arg("eps") = 1e-5, py::arg("packed") = none, py::arg("scales") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "LayerNorm (no affine) -> bf16 stage -> MXFP4: packed e2m1 (rows, dim // 2) + E8M0 "
          "(rows, dim // 32).");
    m.def("ada_layer_norm_quant_mxfp4_bf16",
          [](const Tensor& x, const Tensor& scale, const Tensor& shift, double eps,
             const OptT& packed, const OptT& scales, const OptT& row_mean, const OptT& row_rstd) {
              return mxfp4(x, scale, shift, eps, packed, scales, row_mean, row_rstd);
          },
          py::arg("x"), py::arg("scale"), py::arg("shift"), py::arg("eps") = 1e-5,
          py::arg("packed") = none, py::arg("scales") = none, py::arg("row_mean") = none,
          py::arg("row_rstd") = none, "Broadcast AdaLN -> bf16 stage -> MXFP4; scale, shift (dim,) bf16.");
    m.def("ada_layer_norm_quant_mxfp8_modfp8_bf16", &mxfp8_modfp8, py::arg("x"),
          py::arg("scale_fp8"), py::arg("shift_fp8"), py::arg("scale_deq"), py::arg("shift_deq"),
          py::arg("eps") = 1e-5, py::arg("out") = none, py::arg("scales") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars -> MXFP8.");
    m.def("awq_ada_layer_norm_quant_mxfp8_bf16", &awq_mxfp8, py::arg("x"), py::arg("scale"),
          py::arg("shift"), py::arg("inv_s"), py::arg("eps") = 1e-5, py::arg("out") = none,
          py::arg("scales") = none, py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "Broadcast AdaLN -> per-channel inv_s (dim,) bf16 -> MXFP8.");
    m.def("ada_layer_norm_quant_mxfp4_modfp8_bf16", &mxfp4_modfp8, py::arg("x"),
          py::arg("scale_fp8"), py::arg("shift_fp8"), py::arg("scale_deq"), py::arg("shift_deq"),
          py::arg("eps") = 1e-5, py::arg("packed") = none, py::arg("scales") = none,
          py::arg("row_mean") = none, py::arg("row_rstd") = none,
          "AdaLN with e4m3 (dim,) scale/shift and fp32 device dequantization scalars -> bf16 "
          "stage -> MXFP4.");
    m.def("adaln_modulation6_bf16", &modulation6, py::arg("adaln_params"),
          py::arg("layer_modulation"), py::arg("out") = none,
          "fp32 (batch, seq, 6, dim) + fp32 (6, dim) -> six bf16 (batch, seq, dim).");
    m.def("gated_residual_bf16", &gated_residual, py::arg("residual"), py::arg("gate"),
          py::arg("proj"), py::arg("out") = none,
          "out = bf16(residual + bf16(gate * proj)); gate (rows, dim) or (dim,).  Pass "
          "out=residual to update the residual stream in place.");
    m.def("rms_norm_modulate_seg_bf16", &rms_modulate, py::arg("x"), py::arg("weight"),
          py::arg("scale"), py::arg("shift"), py::arg("seg"), py::arg("eps") = 1e-5,
          py::arg("out") = none, py::arg("row_rstd") = none,
          "RMSNorm (weight (dim,) bf16 or None) then (n * (scale[seg] + 1)) + shift[seg] in bf16 "
          "operations.  scale, shift (segments, dim) bf16; seg (rows,) int32 table row per row "
          "(outside [0, segments): NaN row).  Returns out (rows, dim) bf16.");
}
