// gn_launch.hpp -- kernel arguments and launchers shared by gn_api.cpp and gn_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gn_plan.hpp"

namespace gn {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
// Largest grid launched; kernels stride over any further jobs.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

// Plain-old-data view of a Plan, passed by value to every kernel.
struct KArgs {
    int64_t N, C, S, G;
    int64_t Cg, M;
    int64_t chunk, K, jobs, P;
    int32_t block;
};

inline KArgs kargs_of(const Plan& p)
{
    KArgs a;
    a.N = p.N; a.C = p.C; a.S = p.S; a.G = p.G;
    a.Cg = p.Cg; a.M = p.M;
    a.chunk = p.chunk; a.K = p.K; a.jobs = p.jobs; a.P = p.P;
    a.block = p.block;
    return a;
}

hipError_t launch_stats(const void* x, int xdt, const KArgs& a, float2* part, hipStream_t st);
hipError_t launch_apply(const void* x, int xdt, const float* gamma, const float* beta,
                        const float2* part, void* y, int ydt, float* mean, float* rstd,
                        const KArgs& a, float eps, hipStream_t st);
hipError_t launch_bwd_reduce(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                             const float* rstd, const KArgs& a, float2* part, hipStream_t st);
hipError_t launch_bwd_apply(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                            const float* rstd, const float* gamma, const float2* part,
                            const KArgs& a, void* dx, float* dgamma, float* dbeta, hipStream_t st);

}  // namespace gn
