// gn_binding.cpp -- the compiled half of the torch binding (Python module _gnbind): the
// per-step calls gn_forward and gn_backward (both layouts) for torch tensors.
//
// Argument marshalling only: every tensor a caller passes is checked here (device, dtype,
// element count, layout), the current HIP stream of x's device is taken from torch, and the
// C ABI of libgn.so is called with plain pointers; its status is returned. The checks are
// those of the Python helpers in gn.py, done in C++ because at these calls' rate (a few us
// of GPU work at the small UNet sites) the interpreter's per-tensor attribute lookups had
// become the step's cost. Nothing here computes any part of GroupNorm.
#include <c10/hip/HIPStream.h>
#include <torch/extension.h>

#include <cstdint>
#include <string>
#include <utility>

#include "gn.h"

namespace {

namespace py = pybind11;

int dtype_code(const at::Tensor& t)
{
    switch (t.scalar_type()) {
        case at::kFloat: return GN_F32;
        case at::kBFloat16: return GN_BF16;
        case at::kHalf: return GN_F16;
        default: return -1;
    }
}

int code_of(const at::Tensor& t, const char* name)
{
    const int c = dtype_code(t);
    if (c < 0)
        throw py::type_error(std::string(name) + ": unsupported dtype " + std::string(c10::toString(t.scalar_type())) +
                             " (float32, bfloat16 or float16)");
    return c;
}

// Strides of a tensor of x's sizes laid out channels-last: (N, spatial..., C) contiguous.
bool is_channels_last(const at::Tensor& t)
{
    const int64_t d = t.dim();
    if (d < 3) return false;
    const auto sz = t.sizes();
    const auto st = t.strides();
    int64_t expect = 1;
    if (sz[1] != 1 && st[1] != expect) return false;
    expect *= sz[1];
    for (int64_t i = d - 1; i >= 2; --i) {
        if (sz[i] != 1 && st[i] != expect) return false;
        expect *= sz[i];
    }
    return sz[0] == 1 || st[0] == expect;
}

// 0: NCDHW, 1: NDHWC; want -1 picks from the strides (contiguous first).
int layout_of(const at::Tensor& x, int want)
{
    if (want < 0) {
        if (x.is_contiguous()) return 0;
        if (is_channels_last(x)) return 1;
        throw py::value_error("GroupNorm tensors must be contiguous NCDHW or contiguous channels-last");
    }
    if (want == 0 && x.is_contiguous()) return 0;
    if (want == 1 && is_channels_last(x)) return 1;
    throw py::value_error(std::string("tensor is not contiguous in layout ") + (want == 0 ? "'ncdhw'" : "'ndhwc'"));
}

struct Dims {
    int64_t N, C, S;
};

Dims dims_of(const at::Tensor& x)
{
    if (x.dim() < 2) throw py::value_error("GroupNorm input needs at least (N, C)");
    Dims d{x.size(0), x.size(1), 1};
    for (int64_t i = 2; i < x.dim(); ++i) d.S *= x.size(i);
    return d;
}

// A tensor with x's sizes and strides on x's device (its dtype is checked by the caller).
void* like(const char* name, const at::Tensor& t, const at::Tensor& x, int didx)
{
    if (t.sizes() != x.sizes() || t.strides() != x.strides())
        throw py::value_error(std::string(name) + " must have x's shape and layout");
    if (t.get_device() != didx) throw py::value_error(std::string(name) + " must be on x's device");
    return t.data_ptr();
}

// A contiguous tensor of `numel` elements of `type` on x's device (None passes as NULL).
void* buf(const char* name, const c10::optional<at::Tensor>& t, int64_t numel, int didx,
          at::ScalarType type = at::kFloat)
{
    if (!t.has_value()) return nullptr;
    const at::Tensor& v = *t;
    if (v.scalar_type() != type || v.numel() != numel || v.get_device() != didx || !v.is_contiguous())
        throw py::value_error(std::string(name) + " must be a contiguous " + std::string(c10::toString(type)) +
                              " tensor of " + std::to_string(numel) + " elements on x's device");
    return v.data_ptr();
}

void* stream_of(int didx)
{
    return didx < 0 ? nullptr : static_cast<void*>(c10::hip::getCurrentHIPStream(didx).stream());
}

at::ScalarType type_of_code(int code)
{
    return code == GN_F32 ? at::kFloat : code == GN_BF16 ? at::kBFloat16 : at::kHalf;
}

// Status, the name of the entry point that returned it, and the outputs.
py::tuple result(int status, const char* fn, py::object a, py::object b, py::object c)
{
    return py::make_tuple(std::move(a), std::move(b), std::move(c), status, fn);
}

py::object or_none(bool keep, const at::Tensor& t) { return keep ? py::cast(t) : py::none(); }

// The caller's workspace, or one of the size the plan of x's shape and layout asks for
// (*status set non-zero, and *fn to the size query, when the shape has no plan).
at::Tensor workspace_for(const c10::optional<at::Tensor>& ws, const at::Tensor& x, const Dims& d, int64_t G, int lay,
                         int* status, const char** fn)
{
    if (ws.has_value()) return *ws;
    const size_t nb = lay == 0 ? gn_workspace_bytes(d.N, d.C, d.S, G) : gn_workspace_bytes_cl(d.N, d.C, d.S, G);
    if (nb == 0) {  // a shape without a plan: the planner's status says why
        gn_plan_info info;
        gn_plan_info_cl info_cl;
        *status = lay == 0 ? gn_plan_query(d.N, d.C, d.S, G, &info) : gn_plan_query_cl(d.N, d.C, d.S, G, &info_cl);
        if (*status != GN_OK) *fn = lay == 0 ? "gn_workspace_bytes" : "gn_workspace_bytes_cl";
    }
    return at::empty({int64_t(nb)}, x.options().dtype(at::kByte));
}

std::pair<void*, size_t> ws_args(const at::Tensor& ws, int didx)
{
    if (ws.get_device() != didx || !ws.is_contiguous())
        throw py::value_error("workspace must be a contiguous tensor on x's device");
    return {ws.data_ptr(), size_t(ws.numel()) * ws.element_size()};
}

// gn_forward (NCDHW) or gn_forward_cl (channels-last). Outputs not given are allocated on
// x's device: y like x (out_code < 0: in x's dtype), mean and rstd [N, G] fp32.
py::tuple forward(const at::Tensor& x, const c10::optional<at::Tensor>& gamma,
                  const c10::optional<at::Tensor>& beta, int64_t G, double eps, int out_code, int activation,
                  const c10::optional<at::Tensor>& workspace, const c10::optional<at::Tensor>& out,
                  const c10::optional<at::Tensor>& mean, const c10::optional<at::Tensor>& rstd, int layout)
{
    const int lay = layout_of(x, layout);
    const Dims d = dims_of(x);
    const int didx = x.get_device();
    const int xc = code_of(x, "x");
    const at::Tensor y = out.has_value() ? *out : at::empty_like(x, x.options().dtype(
                                                      out_code < 0 ? x.scalar_type() : type_of_code(out_code)));
    void* yp = like("out", y, x, didx);
    const int yc = code_of(y, "out");
    void* mp = buf("mean", mean, d.N * G, didx);
    void* rp = buf("rstd", rstd, d.N * G, didx);
    void* gp = buf("gamma", gamma, d.C, didx);
    void* bp = buf("beta", beta, d.C, didx);
    const at::Tensor m = mean.has_value() ? *mean : at::empty({d.N, G}, x.options().dtype(at::kFloat));
    const at::Tensor r = rstd.has_value() ? *rstd : at::empty({d.N, G}, x.options().dtype(at::kFloat));
    int status = GN_OK;
    const char* fn = lay == 0 ? "gn_forward" : "gn_forward_cl";
    const at::Tensor ws = workspace_for(workspace, x, d, G, lay, &status, &fn);
    if (status != GN_OK) return result(status, fn, py::none(), py::none(), py::none());
    const auto [wsp, wsb] = ws_args(ws, didx);
    auto call = lay == 0 ? gn_forward : gn_forward_cl;
    status = call(x.data_ptr(), xc, static_cast<const float*>(gp), static_cast<const float*>(bp), d.N, d.C, d.S, G,
                  float(eps), activation, yp, yc, static_cast<float*>(mp ? mp : m.data_ptr()),
                  static_cast<float*>(rp ? rp : r.data_ptr()), wsp, wsb, stream_of(didx));
    return result(status, fn, py::cast(y), py::cast(m), py::cast(r));
}

// gn_backward (NCDHW) or gn_backward_cl (channels-last). dx (x's dtype and layout), dgamma
// and dbeta (C fp32) are allocated where asked for and not given; the others pass as NULL.
py::tuple backward(const at::Tensor& dy, const at::Tensor& x, const c10::optional<at::Tensor>& mean,
                   const c10::optional<at::Tensor>& rstd, const c10::optional<at::Tensor>& gamma,
                   const c10::optional<at::Tensor>& beta, int activation, int64_t G, bool need_dx,
                   bool need_dgamma, bool need_dbeta, const c10::optional<at::Tensor>& workspace,
                   const c10::optional<at::Tensor>& dx, const c10::optional<at::Tensor>& dgamma,
                   const c10::optional<at::Tensor>& dbeta, int layout)
{
    const int lay = layout_of(x, layout);
    const Dims d = dims_of(x);
    const int didx = x.get_device();
    const int xc = code_of(x, "x");
    void* dyp = like("dy", dy, x, didx);
    const int dyc = code_of(dy, "dy");
    at::Tensor dxt, dgt, dbt;
    void* dxp = nullptr;
    if (need_dx) {
        dxt = dx.has_value() ? *dx : at::empty_like(x);
        dxp = like("dx", dxt, x, didx);
        if (dxt.scalar_type() != x.scalar_type())
            throw py::type_error(std::string("dx must have x's dtype ") + std::string(c10::toString(x.scalar_type())));
    }
    if (need_dgamma) dgt = dgamma.has_value() ? *dgamma : at::empty({d.C}, x.options().dtype(at::kFloat));
    if (need_dbeta) dbt = dbeta.has_value() ? *dbeta : at::empty({d.C}, x.options().dtype(at::kFloat));
    void* mp = buf("mean", mean, d.N * G, didx);
    void* rp = buf("rstd", rstd, d.N * G, didx);
    void* gp = buf("gamma", gamma, d.C, didx);
    void* bp = buf("beta", beta, d.C, didx);
    void* dgp = need_dgamma ? buf("dgamma", dgt, d.C, didx) : nullptr;
    void* dbp = need_dbeta ? buf("dbeta", dbt, d.C, didx) : nullptr;
    int status = GN_OK;
    const char* fn = lay == 0 ? "gn_backward" : "gn_backward_cl";
    const at::Tensor ws = workspace_for(workspace, x, d, G, lay, &status, &fn);
    if (status != GN_OK) return result(status, fn, py::none(), py::none(), py::none());
    const auto [wsp, wsb] = ws_args(ws, didx);
    auto call = lay == 0 ? gn_backward : gn_backward_cl;
    status = call(dyp, dyc, x.data_ptr(), xc, static_cast<const float*>(mp), static_cast<const float*>(rp),
                  static_cast<const float*>(gp), static_cast<const float*>(bp), activation, d.N, d.C, d.S, G, dxp,
                  static_cast<float*>(dgp), static_cast<float*>(dbp), wsp, wsb, stream_of(didx));
    return result(status, fn, or_none(need_dx, dxt), or_none(need_dgamma, dgt), or_none(need_dbeta, dbt));
}

}  // namespace

PYBIND11_MODULE(TORCH_EXTENSION_NAME, m)
{
    m.doc() = "Compiled marshalling of gn_forward / gn_backward (libgn.so's C ABI) for torch tensors";
    m.def("forward", &forward, "gn_forward or gn_forward_cl: (y, mean, rstd, status, entry point)", py::arg("x"),
          py::arg("gamma"), py::arg("beta"), py::arg("G"), py::arg("eps"), py::arg("out_code"),
          py::arg("activation"), py::arg("workspace"), py::arg("out"), py::arg("mean"), py::arg("rstd"),
          py::arg("layout"));
    m.def("backward", &backward, "gn_backward or gn_backward_cl: (dx, dgamma, dbeta, status, entry point)",
          py::arg("dy"), py::arg("x"), py::arg("mean"), py::arg("rstd"), py::arg("gamma"), py::arg("beta"),
          py::arg("activation"), py::arg("G"), py::arg("need_dx"), py::arg("need_dgamma"), py::arg("need_dbeta"),
          py::arg("workspace"), py::arg("dx"), py::arg("dgamma"), py::arg("dbeta"), py::arg("layout"));
    m.def("abi_version", []() { return gn_abi_version(); });
}
