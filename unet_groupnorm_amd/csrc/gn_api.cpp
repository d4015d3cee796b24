// gn_api.cpp -- the C ABI declared in include/gn.h: validation, planning, launches.
//
// Every check runs before anything is enqueued. The library allocates nothing, never
// synchronizes and never reads device memory from the host. Its only state is, per
// device, the address of the static scratch array that gn_forward_noalloc uses.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "gn.h"
#include "gn_launch.hpp"
#include "gn_plan.hpp"

namespace {

// Volumes of x up to this many bytes are streamed with plain (cacheable) loads, others with
// nontemporal ones. A step reads x four times and dy twice; when x fits well inside MI355X's
// 256 MiB last-level cache the later reads find it there (measured: 128^3 x 32 channels of
// bf16, 128 MiB, 3-4% faster a step; 256 MiB and more, and 1 GiB by 7%, slower than
// nontemporal). Loads only: no result depends on it.
constexpr int64_t kCachedBytes = int64_t(160) << 20;

gn::KArgs kargs_for(const gn::Plan& p, int activation, int x_dtype)
{
    gn::KArgs a = gn::kargs_of(p, activation);
    const int64_t bytes = p.N * p.C * p.S * (x_dtype == GN_F32 ? 4 : 2);
    a.cached = bytes <= kCachedBytes ? 1 : 0;
    // The folded-job order pays where the inputs stay in the last-level cache; over
    // nontemporal streams it spreads each moment's accesses over every reduction job's span
    // (256^3: 1309 -> 1413 us a step), so they keep index order.
    if (!a.cached) a.fold_nest = a.step_nest = 1;
    return a;
}

gn::ClArgs clargs_for(const gn::PlanCL& p, int activation, int x_dtype)
{
    gn::ClArgs a = gn::clargs_of(p, activation);
    const int64_t bytes = p.N * p.C * p.S * (x_dtype == GN_F32 ? 4 : 2);
    a.cached = bytes <= kCachedBytes ? 1 : 0;
    if (!a.cached) a.fold_nest = 1;  // as for NCDHW: index order over nontemporal streams
    return a;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool dtype_ok(int d) { return d == GN_F32 || d == GN_BF16 || d == GN_F16; }
bool act_ok(int a) { return a == GN_ACT_NONE || a == GN_ACT_RELU; }

int plan_or_error(int64_t N, int64_t C, int64_t S, int64_t G, gn::Plan* p)
{
    const int rc = gn::make_plan(N, C, S, G, p);
    return rc == 0 ? GN_OK : (rc == 3 ? GN_ERR_GROUPS : GN_ERR_SHAPE);
}

int workspace_check(const void* ws, size_t bytes, const gn::Plan& p)
{
    if (!aligned(ws, 16)) return GN_ERR_ALIGN;
    if (bytes < p.ws_bytes) return GN_ERR_WORKSPACE;
    return GN_OK;
}

// The device that owns p, or -1 if p is not device memory (host, pinned or unknown).
int device_of(const void* p)
{
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return -1;
    return attr.device;
}

// Makes x's device current for the duration of a call ("Optimize GroupNorm", paragraph on
// the independent review: launching on the current device instead of the input's device
// faulted on a tensor living on another GPU). A stream of another device is rejected, and so
// is any other pointer argument that is not device memory of that device (a kernel would
// otherwise read or write host memory, or another GPU's).
class DeviceScope {
  public:
    int enter(const void* x, void* stream)
    {
        const int dev = device_of(x);
        if (dev < 0) return GN_ERR_DEVICE;
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GN_ERR_DEVICE;
        if (stream) {
            hipDevice_t sdev = -1;
            if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
                (void)hipGetLastError();
                return GN_ERR_DEVICE;
            }
            if (sdev != dev) return GN_ERR_DEVICE;
        }
        if (cur != dev) {
            if (hipSetDevice(dev) != hipSuccess) return GN_ERR_DEVICE;
            prev_ = cur;
        }
        dev_ = dev;
        return GN_OK;
    }
    // GN_OK if every non-NULL pointer lives on the call's device.
    int same_device(std::initializer_list<const void*> ptrs) const
    {
        for (const void* p : ptrs)
            if (p && device_of(p) != dev_) return GN_ERR_DEVICE;
        return GN_OK;
    }
    int device() const { return dev_; }
    ~DeviceScope()
    {
        if (prev_ >= 0) (void)hipSetDevice(prev_);
    }

  private:
    int prev_ = -1;
    int dev_ = -1;
};

// gn_forward's checks of everything but the workspace.
int fwd_args_check(const void* x, int x_dtype, const float* gamma, const float* beta, int64_t N,
                   int64_t C, int64_t S, int64_t G, float eps, int activation, const void* y, int y_dtype,
                   const float* mean, const float* rstd, gn::Plan* p)
{
    if (!x || !y || !mean || !rstd) return GN_ERR_NULL;
    int rc = plan_or_error(N, C, S, G, p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype) || !(y_dtype == x_dtype || y_dtype == GN_F32)) return GN_ERR_DTYPE;
    if (!std::isfinite(eps) || eps < 0.0f) return GN_ERR_EPS;
    if (!act_ok(activation)) return GN_ERR_ACTIVATION;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(mean, 4) || !aligned(rstd, 4) ||
        !aligned(gamma, 4) || !aligned(beta, 4))
        return GN_ERR_ALIGN;
    return GN_OK;
}

int fwd_check(const void* x, int x_dtype, const float* gamma, const float* beta, int64_t N,
              int64_t C, int64_t S, int64_t G, float eps, int activation, const void* y, int y_dtype,
              const float* mean, const float* rstd, const void* ws, size_t ws_bytes, gn::Plan* p)
{
    if (!ws) return GN_ERR_NULL;
    const int rc = fwd_args_check(x, x_dtype, gamma, beta, N, C, S, G, eps, activation, y, y_dtype, mean, rstd, p);
    if (rc) return rc;
    return workspace_check(ws, ws_bytes, *p);
}

int bwd_check(const void* dy, int dy_dtype, const void* x, int x_dtype, const float* mean,
              const float* rstd, const float* gamma, const float* beta, int activation, int64_t N,
              int64_t C, int64_t S, int64_t G, const void* dx, const float* dgamma,
              const float* dbeta, const void* ws, size_t ws_bytes, gn::Plan* p)
{
    if (!dy || !x || !mean || !rstd || !ws) return GN_ERR_NULL;
    int rc = plan_or_error(N, C, S, G, p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype) || !dtype_ok(dy_dtype)) return GN_ERR_DTYPE;
    if (!act_ok(activation)) return GN_ERR_ACTIVATION;
    if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(dx, 16) || !aligned(mean, 4) ||
        !aligned(rstd, 4) || !aligned(gamma, 4) || !aligned(beta, 4) || !aligned(dgamma, 4) ||
        !aligned(dbeta, 4))
        return GN_ERR_ALIGN;
    return workspace_check(ws, ws_bytes, *p);
}

int launch_status(hipError_t e) { return e == hipSuccess ? GN_OK : GN_ERR_LAUNCH; }

// ------------------------------------------------------------------ static scratch
//
// The workspace of gn_forward_noalloc: device memory of the library itself, one copy per
// device (each device the library runs on holds it until the process ends). In host code
// `scratch` names a host-side stand-in, not a device address; its address on a device is
// queried once per device, with that device current, and only that address is handed to
// kernels. Every call on a device shares that device's copy: calls that overlap on one
// device (two streams at once) race on it.
static __device__ __align__(256) unsigned char scratch[GN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on device dev, which must be current; nullptr if the
// runtime cannot give it.
void* scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

// The two halves of gn_forward. On the resident path the first does nothing and the
// second runs the whole forward; otherwise the second is the normalize with the finalize
// folded into each of its workgroups (the split-phase entry points run it alone).
int fwd_partials(const void* x, int x_dtype, const gn::Plan& p, const gn::KArgs& a, gn::Workspace w,
                 hipStream_t st)
{
    if (p.res_fwd) return GN_OK;
    return launch_status(gn::launch_stats_partials(x, x_dtype, a, w, st));
}

int fwd_finish(const void* x, int x_dtype, const float* gamma, const float* beta, float eps, void* y,
               int y_dtype, float* mean, float* rstd, const gn::Plan& p, const gn::KArgs& a,
               gn::Workspace w, hipStream_t st)
{
    if (p.res_fwd)
        return launch_status(gn::launch_res_fwd(x, x_dtype, gamma, beta, eps, mean, rstd, y, y_dtype, a, w,
                                                st, p.res_block_f, p.res_vecs_f));
    return launch_status(gn::launch_fwd_apply_fin(x, x_dtype, gamma, beta, eps, mean, rstd, y, y_dtype, a,
                                                  w, st));
}

// The two halves of gn_backward, likewise.
int bwd_partials(const void* dy, int dy_dtype, const void* x, int x_dtype, const float* mean,
                 const float* rstd, const float* gamma, const float* beta, const gn::Plan& p,
                 const gn::KArgs& a, gn::Workspace w, hipStream_t st)
{
    if (p.res_bwd) return GN_OK;
    return launch_status(gn::launch_bwd_partials(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, a, w, st));
}

int bwd_finish(const void* dy, int dy_dtype, const void* x, int x_dtype, const float* mean, const float* rstd,
               const float* gamma, const float* beta, void* dx, float* dgamma, float* dbeta,
               const gn::Plan& p, const gn::KArgs& a, gn::Workspace w, hipStream_t st)
{
    if (p.res_bwd)
        return launch_status(gn::launch_res_bwd(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dgamma,
                                                dbeta, dx, a, w, st, p.res_block_b, p.res_vecs_b,
                                                p.res_bwd_split));
    if (dx)
        return launch_status(gn::launch_bwd_apply_fin(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dgamma,
                                                      dbeta, dx, a, w, st));
    return launch_status(gn::launch_fin_bwd(mean, rstd, gamma, beta, dgamma, dbeta, a, w, st));
}

}  // namespace

extern "C" {

size_t gn_workspace_bytes(int64_t N, int64_t C, int64_t S, int64_t G)
{
    gn::Plan p;
    return gn::make_plan(N, C, S, G, &p) == 0 ? p.ws_bytes : 0;
}

int gn_plan_query(int64_t N, int64_t C, int64_t S, int64_t G, gn_plan_info* out)
{
    if (!out) return GN_ERR_NULL;
    gn::Plan p;
    const int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    out->rows = p.rows;
    out->chunk = p.chunk;
    out->chunks_per_row = p.K;
    out->jobs = p.jobs;
    out->partials_per_group = p.P;
    out->block = p.block;
    out->vectors_per_step = gn::kStepVecs;
    out->apply_chunk = p.chunk_a;
    out->apply_chunks_per_row = p.K_a;
    out->apply_jobs = p.jobs_a;
    out->apply_block = p.block_a;
    out->apply_vectors = gn::kApplyVecs;
    out->workspace_bytes = p.ws_bytes;
    out->resident_forward = p.res_fwd ? 1 : 0;
    out->resident_backward = p.res_bwd ? 1 : 0;
    out->resident_block_forward = p.res_block_f;
    out->resident_vectors_forward = p.res_vecs_f;
    out->resident_block_backward = p.res_block_b;
    out->resident_vectors_backward = p.res_vecs_b;
    out->fold_chunk = p.chunk_f;
    out->fold_chunks_per_row = p.K_f;
    out->fold_jobs = p.jobs_f;
    out->resident_backward_split = p.res_bwd_split ? 1 : 0;
    return GN_OK;
}

int gn_abi_version(void) { return GN_ABI_VERSION; }

const char* gn_status_string(int status)
{
    switch (status) {
        case GN_OK: return "ok";
        case GN_ERR_NULL: return "a required pointer is NULL";
        case GN_ERR_SHAPE: return "invalid shape (N, C, S, G must be positive; N*(C/G)*S must exceed 1)";
        case GN_ERR_GROUPS: return "C is not a multiple of G";
        case GN_ERR_DTYPE: return "unsupported dtype or dtype combination";
        case GN_ERR_EPS: return "eps must be finite and >= 0";
        case GN_ERR_WORKSPACE: return "workspace smaller than gn_workspace_bytes()";
        case GN_ERR_ALIGN: return "misaligned pointer (tensors and workspace need 16 bytes, fp32 vectors 4)";
        case GN_ERR_DEVICE: return "a pointer argument is not device memory of x's device, or the stream belongs to another device";
        case GN_ERR_LAUNCH: return "kernel launch failed";
        case GN_ERR_ACTIVATION: return "unknown activation (GN_ACT_NONE or GN_ACT_RELU)";
        case GN_ERR_LAYOUT: return "shape not supported channels-last (C a multiple of 8 with C/8 dividing 256; C/G dividing 8 or a multiple of 8)";
        case GN_ERR_SCRATCH: return "gn_forward_noalloc: the shape needs a larger workspace than its static scratch holds (gn_workspace_bytes > GN_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int gn_forward_stats(const void* x, int x_dtype, const float* gamma, const float* beta,
                     int64_t N, int64_t C, int64_t S, int64_t G, float eps,
                     float* mean, float* rstd,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    if (!x || !mean || !rstd || !workspace) return GN_ERR_NULL;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype)) return GN_ERR_DTYPE;
    if (!std::isfinite(eps) || eps < 0.0f) return GN_ERR_EPS;
    if (!aligned(x, 16) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(gamma, 4) ||
        !aligned(beta, 4))
        return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, mean, rstd, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, 0, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.res_fwd)
        return launch_status(gn::launch_res_fwd(x, x_dtype, gamma, beta, eps, mean, rstd, nullptr, x_dtype,
                                                a, w, st, p.res_block_f, p.res_vecs_f));
    return launch_status(gn::launch_fwd_stats(x, x_dtype, gamma, beta, eps, mean, rstd, a, w, st));
}

int gn_forward_apply(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                     int activation, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    if (!x || !y || !workspace) return GN_ERR_NULL;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype) || !(y_dtype == x_dtype || y_dtype == GN_F32)) return GN_ERR_DTYPE;
    if (!act_ok(activation)) return GN_ERR_ACTIVATION;
    if (!aligned(x, 16) || !aligned(y, 16)) return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({y, workspace}))) return rc;
    return launch_status(gn::launch_fwd_apply(x, x_dtype, y, y_dtype, kargs_for(p, activation, x_dtype),
                                              gn::workspace_of(workspace, p),
                                              static_cast<hipStream_t>(stream)));
}

int gn_forward(const void* x, int x_dtype, const float* gamma, const float* beta,
               int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
               void* y, int y_dtype, float* mean, float* rstd,
               void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = fwd_check(x, x_dtype, gamma, beta, N, C, S, G, eps, activation, y, y_dtype, mean, rstd,
                       workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, y, mean, rstd, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, activation, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = fwd_partials(x, x_dtype, p, a, w, st))) return rc;
    return fwd_finish(x, x_dtype, gamma, beta, eps, y, y_dtype, mean, rstd, p, a, w, st);
}

int gn_forward_noalloc(const void* x, int x_dtype, const float* gamma, const float* beta,
                       int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                       void* y, int y_dtype, float* mean, float* rstd, void* stream)
{
    gn::Plan p;
    int rc = fwd_args_check(x, x_dtype, gamma, beta, N, C, S, G, eps, activation, y, y_dtype, mean, rstd, &p);
    if (rc) return rc;
    if (p.ws_bytes > GN_NOALLOC_SCRATCH_BYTES) return GN_ERR_SCRATCH;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, y, mean, rstd}))) return rc;
    void* ws = scratch_on(ds.device());
    if (!ws) return GN_ERR_DEVICE;
    const gn::KArgs a = kargs_for(p, activation, x_dtype);
    const gn::Workspace w = gn::workspace_of(ws, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = fwd_partials(x, x_dtype, p, a, w, st))) return rc;
    return fwd_finish(x, x_dtype, gamma, beta, eps, y, y_dtype, mean, rstd, p, a, w, st);
}

int gn_forward_partials(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    if (!x || !workspace) return GN_ERR_NULL;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype)) return GN_ERR_DTYPE;
    if (!aligned(x, 16)) return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({workspace}))) return rc;
    return fwd_partials(x, x_dtype, p, kargs_for(p, 0, x_dtype), gn::workspace_of(workspace, p),
                        static_cast<hipStream_t>(stream));
}

int gn_forward_finish(const void* x, int x_dtype, const float* gamma, const float* beta,
                      int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                      void* y, int y_dtype, float* mean, float* rstd,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = fwd_check(x, x_dtype, gamma, beta, N, C, S, G, eps, activation, y, y_dtype, mean, rstd,
                       workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, y, mean, rstd, workspace}))) return rc;
    return fwd_finish(x, x_dtype, gamma, beta, eps, y, y_dtype, mean, rstd, p,
                      kargs_for(p, activation, x_dtype),
                      gn::workspace_of(workspace, p), static_cast<hipStream_t>(stream));
}

int gn_backward_reduce(const void* dy, int dy_dtype, const void* x, int x_dtype,
                       const float* mean, const float* rstd, const float* gamma,
                       const float* beta, int activation,
                       int64_t N, int64_t C, int64_t S, int64_t G,
                       float* dgamma, float* dbeta,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G,
                       nullptr, dgamma, dbeta, workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, dgamma, dbeta, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, activation, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.res_bwd)
        return launch_status(gn::launch_res_bwd(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dgamma,
                                                dbeta, nullptr, a, w, st, p.res_block_b, p.res_vecs_b,
                                                p.res_bwd_split));
    return launch_status(gn::launch_bwd_reduce(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta,
                                               dgamma, dbeta, a, w, st));
}

int gn_backward_apply(const void* dy, int dy_dtype, const void* x, int x_dtype,
                      int64_t N, int64_t C, int64_t S, int64_t G, int activation, void* dx,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    if (!dy || !x || !dx || !workspace) return GN_ERR_NULL;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (!dtype_ok(x_dtype) || !dtype_ok(dy_dtype)) return GN_ERR_DTYPE;
    if (!act_ok(activation)) return GN_ERR_ACTIVATION;
    if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(dx, 16)) return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, dx, workspace}))) return rc;
    return launch_status(gn::launch_bwd_apply(dy, dy_dtype, x, x_dtype, dx, kargs_for(p, activation, x_dtype),
                                              gn::workspace_of(workspace, p),
                                              static_cast<hipStream_t>(stream)));
}

int gn_backward(const void* dy, int dy_dtype, const void* x, int x_dtype,
                const float* mean, const float* rstd, const float* gamma,
                const float* beta, int activation,
                int64_t N, int64_t C, int64_t S, int64_t G,
                void* dx, float* dgamma, float* dbeta,
                void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G, dx,
                       dgamma, dbeta, workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, dx, dgamma, dbeta, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, activation, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = bwd_partials(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, p, a, w, st))) return rc;
    return bwd_finish(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dx, dgamma, dbeta, p, a, w, st);
}

int gn_backward_partials(const void* dy, int dy_dtype, const void* x, int x_dtype,
                         const float* mean, const float* rstd, const float* gamma,
                         const float* beta, int activation,
                         int64_t N, int64_t C, int64_t S, int64_t G,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G, nullptr,
                       nullptr, nullptr, workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, workspace}))) return rc;
    return bwd_partials(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, p,
                        kargs_for(p, activation, x_dtype),
                        gn::workspace_of(workspace, p), static_cast<hipStream_t>(stream));
}

int gn_backward_finish(const void* dy, int dy_dtype, const void* x, int x_dtype,
                       const float* mean, const float* rstd, const float* gamma,
                       const float* beta, int activation,
                       int64_t N, int64_t C, int64_t S, int64_t G,
                       void* dx, float* dgamma, float* dbeta,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G, dx,
                       dgamma, dbeta, workspace, workspace_bytes, &p);
    if (rc) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, dx, dgamma, dbeta, workspace}))) return rc;
    return bwd_finish(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dx, dgamma, dbeta, p,
                      kargs_for(p, activation, x_dtype), gn::workspace_of(workspace, p),
                      static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ spatial shards

static_assert(sizeof(gn_moments) == sizeof(gn::Moments16), "record layout");

int gn_forward_shard_stats(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                           gn_moments* moments, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!x || !moments || !workspace) return GN_ERR_NULL;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (p.M >= (int64_t(1) << 32)) return GN_ERR_SHAPE;
    if (!dtype_ok(x_dtype)) return GN_ERR_DTYPE;
    if (!aligned(x, 16) || !aligned(moments, 16)) return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({moments, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, 0, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = launch_status(gn::launch_stats_partials(x, x_dtype, a, w, st)))) return rc;
    return launch_status(gn::launch_shard_records(x, x_dtype, a, w, reinterpret_cast<gn::Moments16*>(moments), st));
}

int gn_forward_shard_merge(const gn_moments* moments, int64_t P, const float* gamma, const float* beta,
                           int64_t N, int64_t C, int64_t S, int64_t G, float eps,
                           float* mean, float* rstd, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!moments || !mean || !rstd || !workspace) return GN_ERR_NULL;
    if (P < 1) return GN_ERR_SHAPE;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (P > ((int64_t(1) << 62) / (N * G))) return GN_ERR_SHAPE;
    if (!std::isfinite(eps) || eps < 0.0f) return GN_ERR_EPS;
    if (!aligned(moments, 16) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(gamma, 4) ||
        !aligned(beta, 4))
        return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(moments, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, mean, rstd, workspace}))) return rc;
    return launch_status(gn::launch_shard_merge_fwd(reinterpret_cast<const gn::Moments16*>(moments), P, gamma,
                                                    beta, eps, mean, rstd, gn::kargs_of(p),
                                                    gn::workspace_of(workspace, p),
                                                    static_cast<hipStream_t>(stream)));
}

int gn_backward_shard_sums(const void* dy, int dy_dtype, const void* x, int x_dtype,
                           const float* mean, const float* rstd, const float* gamma,
                           const float* beta, int activation,
                           int64_t N, int64_t C, int64_t S, int64_t G,
                           float* sums, void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan p;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G, nullptr,
                       nullptr, nullptr, workspace, workspace_bytes, &p);
    if (rc) return rc;
    if (!sums) return GN_ERR_NULL;
    if (!aligned(sums, 8)) return GN_ERR_ALIGN;
    if (N > ((int64_t(1) << 31) - 1) / C) return GN_ERR_SHAPE;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, sums, workspace}))) return rc;
    const gn::KArgs a = kargs_for(p, activation, x_dtype);
    const gn::Workspace w = gn::workspace_of(workspace, p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = launch_status(gn::launch_bwd_partials(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, a, w, st))))
        return rc;
    return launch_status(gn::launch_shard_sums(a, w, reinterpret_cast<float2*>(sums), st));
}

int gn_backward_shard_merge(const float* sums, int64_t P, const float* mean, const float* rstd,
                            const float* gamma, const float* beta,
                            int64_t N, int64_t C, int64_t S, int64_t S_total, int64_t G,
                            float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!sums || !mean || !rstd || !workspace) return GN_ERR_NULL;
    if (P < 1 || S_total < S) return GN_ERR_SHAPE;
    gn::Plan p;
    int rc = plan_or_error(N, C, S, G, &p);
    if (rc) return rc;
    if (S_total > gn::kMaxNumel / (N * C) || P > ((int64_t(1) << 62) / (N * C))) return GN_ERR_SHAPE;
    if (!aligned(sums, 8) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(gamma, 4) ||
        !aligned(beta, 4) || !aligned(dgamma, 4) || !aligned(dbeta, 4))
        return GN_ERR_ALIGN;
    if ((rc = workspace_check(workspace, workspace_bytes, p))) return rc;
    DeviceScope ds;
    if ((rc = ds.enter(sums, stream))) return rc;
    if ((rc = ds.same_device({mean, rstd, gamma, beta, dgamma, dbeta, workspace}))) return rc;
    return launch_status(gn::launch_shard_merge_bwd(reinterpret_cast<const float2*>(sums), P, mean, rstd, gamma,
                                                    beta, p.Cg * S_total, dgamma, dbeta, gn::kargs_of(p),
                                                    gn::workspace_of(workspace, p),
                                                    static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ channels-last

static int plan_cl_or_error(int64_t N, int64_t C, int64_t S, int64_t G, gn::PlanCL* p)
{
    const int rc = gn::make_plan_cl(N, C, S, G, p);
    if (rc == 0) return GN_OK;
    return rc == 3 ? GN_ERR_GROUPS : (rc == 4 ? GN_ERR_LAYOUT : GN_ERR_SHAPE);
}

size_t gn_workspace_bytes_cl(int64_t N, int64_t C, int64_t S, int64_t G)
{
    gn::PlanCL p;
    return gn::make_plan_cl(N, C, S, G, &p) == 0 ? p.ws_bytes : 0;
}

int gn_plan_query_cl(int64_t N, int64_t C, int64_t S, int64_t G, gn_plan_info_cl* out)
{
    if (!out) return GN_ERR_NULL;
    gn::PlanCL p;
    const int rc = plan_cl_or_error(N, C, S, G, &p);
    if (rc) return rc;
    out->chunk = p.chunk;
    out->jobs_per_sample = p.K;
    out->jobs = p.jobs;
    out->voxels_per_round = p.vps;
    out->apply_chunk = p.chunk_a;
    out->apply_jobs_per_sample = p.K_a;
    out->apply_jobs = p.jobs_a;
    out->block = gn::kClBlock;
    out->rounds_per_step = gn::kClRounds;
    out->apply_rounds = gn::kClApplyRounds;
    out->groups_per_vector = p.ngl;
    out->workspace_bytes = p.ws_bytes;
    out->resident_forward = p.res_fwd ? 1 : 0;
    out->resident_backward = p.res_bwd ? 1 : 0;
    out->resident_block_forward = p.res_block_f;
    out->resident_vectors_forward = p.res_vecs_f;
    out->resident_block_backward = p.res_block_b;
    out->resident_vectors_backward = p.res_vecs_b;
    return GN_OK;
}

int gn_forward_cl(const void* x, int x_dtype, const float* gamma, const float* beta,
                  int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                  void* y, int y_dtype, float* mean, float* rstd,
                  void* workspace, size_t workspace_bytes, void* stream)
{
    // Same checks as gn_forward (which also rejects what no layout supports), then the
    // channels-last plan and its workspace size.
    gn::Plan base;
    int rc = fwd_check(x, x_dtype, gamma, beta, N, C, S, G, eps, activation, y, y_dtype, mean, rstd,
                       workspace, 0, &base);
    if (rc && rc != GN_ERR_WORKSPACE) return rc;
    gn::PlanCL p;
    if ((rc = plan_cl_or_error(N, C, S, G, &p))) return rc;
    if (workspace_bytes < p.ws_bytes) return GN_ERR_WORKSPACE;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({gamma, beta, y, mean, rstd, workspace}))) return rc;
    if (p.res_fwd)
        return launch_status(gn::launch_cl_res_forward(x, x_dtype, gamma, beta, eps, mean, rstd, y, y_dtype,
                                                       clargs_for(p, activation, x_dtype),
                                                       static_cast<hipStream_t>(stream), p.res_block_f,
                                                       p.res_vecs_f));
    return launch_status(gn::launch_cl_forward(x, x_dtype, gamma, beta, eps, mean, rstd, y, y_dtype,
                                               clargs_for(p, activation, x_dtype), gn::workspace_cl_of(workspace, p),
                                               static_cast<hipStream_t>(stream)));
}

int gn_backward_cl(const void* dy, int dy_dtype, const void* x, int x_dtype,
                   const float* mean, const float* rstd, const float* gamma,
                   const float* beta, int activation,
                   int64_t N, int64_t C, int64_t S, int64_t G,
                   void* dx, float* dgamma, float* dbeta,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    gn::Plan base;
    int rc = bwd_check(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, activation, N, C, S, G, dx,
                       dgamma, dbeta, workspace, 0, &base);
    if (rc && rc != GN_ERR_WORKSPACE) return rc;
    gn::PlanCL p;
    if ((rc = plan_cl_or_error(N, C, S, G, &p))) return rc;
    if (workspace_bytes < p.ws_bytes) return GN_ERR_WORKSPACE;
    DeviceScope ds;
    if ((rc = ds.enter(x, stream))) return rc;
    if ((rc = ds.same_device({dy, mean, rstd, gamma, beta, dx, dgamma, dbeta, workspace}))) return rc;
    if (p.res_bwd)
        return launch_status(gn::launch_cl_res_backward(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dx,
                                                        dgamma, dbeta, clargs_for(p, activation, x_dtype),
                                                        static_cast<hipStream_t>(stream), p.res_block_b,
                                                        p.res_vecs_b));
    return launch_status(gn::launch_cl_backward(dy, dy_dtype, x, x_dtype, mean, rstd, gamma, beta, dx, dgamma,
                                                dbeta, clargs_for(p, activation, x_dtype),
                                                gn::workspace_cl_of(workspace, p),
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
