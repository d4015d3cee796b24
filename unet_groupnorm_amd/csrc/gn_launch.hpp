// gn_launch.hpp -- kernel arguments and launchers shared by gn_api.cpp and gn_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gn_plan.hpp"

namespace gn {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kF16 = 2;
// Largest grid launched; kernels stride over any further jobs.
constexpr int64_t kMaxGrid = int64_t(1) << 30;

// Division by a divisor d fixed for a launch: floor(x / d) = (x * m) >> 32 with
// m = floor(2^32 / d) + 1, exact for x < 2^16 and d <= 2^16, because the product exceeds
// x / d by x * (m - 2^32 / d) / 2^32 < 2^-16 <= 1 / d, less than the distance from x / d
// to the next integer. The resident path's in-workgroup indices stay below 4096.
struct FastDiv {
    uint64_t m;
};

inline FastDiv fastdiv_of(int64_t d)
{
    return FastDiv{(d >= 1 && d <= 65536) ? (uint64_t(1) << 32) / uint64_t(d) + 1 : 0};
}

// The streaming jobs' order (job_in_order, gn_device.hpp): with F > 1 streaming jobs in
// each reduction job and fewer than 2^16 of them (fdiv's exact range), nest = F,
// R = jobs / F (the reduction jobs) and shift = log2(R) when R is a power of two, else -1;
// otherwise nest = 1 (index order).
inline void set_job_order(int64_t F, int64_t jobs, int32_t& nest, int32_t& R, int32_t& shift, FastDiv& divR)
{
    const bool permute = F > 1 && jobs < 65536;
    nest = permute ? int32_t(F) : 1;
    R = permute ? int32_t(jobs / F) : 1;
    shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((int64_t(1) << sh) == R) shift = sh;
    divR = fastdiv_of(R);
}

// Plain-old-data view of a Plan, passed by value to every kernel.
struct KArgs {
    int64_t N, C, S, G;
    int64_t Cg, M;
    int64_t chunk, K, jobs, P;        // reduction jobs
    int64_t chunk_a, K_a, jobs_a;     // streaming jobs
    int64_t chunk_f, K_f, jobs_f;     // streaming jobs with the finalize folded in
    int32_t block, block_a;
    int32_t act;                      // 0: none, 1: relu after the affine
    int32_t cached;                   // host's choice: plain loads, the volume fits the LLC
    FastDiv div_W, div_vg, div_Cg;    // resident path: S/8, M/8 and C/G as divisors
    // Folded-job order (job_in_order, set by set_job_order): folded jobs nested in the
    // reduction jobs.
    int32_t fold_nest, fold_R;
    FastDiv div_fold_R;
    int32_t fold_shift;
    // The same for the one-step streaming jobs (chunk_a) nested in the reduction jobs.
    int32_t step_nest, step_R;
    FastDiv div_step_R;
    int32_t step_shift;
};

inline KArgs kargs_of(const Plan& p, int act = 0)
{
    KArgs a;
    a.act = act;
    a.cached = 0;
    a.N = p.N; a.C = p.C; a.S = p.S; a.G = p.G;
    a.Cg = p.Cg; a.M = p.M;
    a.chunk = p.chunk; a.K = p.K; a.jobs = p.jobs; a.P = p.P;
    a.chunk_a = p.chunk_a; a.K_a = p.K_a; a.jobs_a = p.jobs_a;
    a.chunk_f = p.chunk_f; a.K_f = p.K_f; a.jobs_f = p.jobs_f;
    a.block = p.block; a.block_a = p.block_a;
    a.div_W = fastdiv_of(p.S % kVec == 0 ? p.S / kVec : 0);
    a.div_vg = fastdiv_of(p.S % kVec == 0 ? p.M / kVec : 0);
    a.div_Cg = fastdiv_of(p.Cg);
    const bool nest = p.chunk_f > 0 && p.chunk % p.chunk_f == 0 && p.K_f == p.K * (p.chunk / p.chunk_f);
    const int64_t F = nest ? p.chunk / p.chunk_f : 1;
    set_job_order(F, p.jobs_f, a.fold_nest, a.fold_R, a.fold_shift, a.div_fold_R);
    const bool nest_a = p.chunk_a > 0 && p.chunk % p.chunk_a == 0 && p.K_a == p.K * (p.chunk / p.chunk_a);
    set_job_order(nest_a ? p.chunk / p.chunk_a : 1, p.jobs_a, a.step_nest, a.step_R, a.step_shift, a.div_step_R);
    return a;
}

// Workspace views. The partials area holds one float2 per reduction job; the coefficient
// area two float4 per row, written by a finalize kernel and read by the streaming kernel.
struct Workspace {
    float2* part;
    float4* coef;
};

inline Workspace workspace_of(void* ws, const Plan& p)
{
    char* b = static_cast<char*>(ws);
    return Workspace{reinterpret_cast<float2*>(b), reinterpret_cast<float4*>(b + p.ws_coef_offset)};
}

// Forward, first half: statistics partials, then their fixed-order merge into mean/rstd
// and the per-row normalize coefficients.
hipError_t launch_fwd_stats(const void* x, int xdt, const float* gamma, const float* beta,
                            float eps, float* mean, float* rstd, const KArgs& a, Workspace ws,
                            hipStream_t st);
// Forward, second half: y from x and the per-row coefficients.
hipError_t launch_fwd_apply(const void* x, int xdt, void* y, int ydt, const KArgs& a,
                            Workspace ws, hipStream_t st);
// Backward, first half: per-job sums of dy and dy*xhat, then their fixed-order merge into
// dgamma/dbeta and the per-row dx coefficients.
hipError_t launch_bwd_reduce(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                             const float* rstd, const float* gamma, const float* beta, float* dgamma,
                             float* dbeta, const KArgs& a, Workspace ws, hipStream_t st);
// Backward, second half: dx from x, dy and the per-row coefficients.
hipError_t launch_bwd_apply(const void* dy, int dydt, const void* x, int xdt, void* dx,
                            const KArgs& a, Workspace ws, hipStream_t st);

// The finalize alone, after launch_stats_partials / launch_bwd_partials.
hipError_t launch_fin_fwd(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                          float* mean, float* rstd, const KArgs& a, Workspace ws, hipStream_t st);
hipError_t launch_fin_bwd(const float* mean, const float* rstd, const float* gamma, const float* beta,
                          float* dgamma, float* dbeta, const KArgs& a, Workspace ws, hipStream_t st);
// The finalize folded into the streaming pass (after launch_stats_partials /
// launch_bwd_partials): the same statistics, coefficients and parameter gradients as the
// split kernels, bitwise, with one launch fewer per direction.
hipError_t launch_fwd_apply_fin(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                                float* mean, float* rstd, void* y, int ydt, const KArgs& a, Workspace ws,
                                hipStream_t st);
hipError_t launch_bwd_apply_fin(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                                const float* rstd, const float* gamma, const float* beta, float* dgamma,
                                float* dbeta, void* dx, const KArgs& a, Workspace ws, hipStream_t st);

// Resident path, forward: statistics, the per-row coefficients, and y unless y is null.
hipError_t launch_res_fwd(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                          float* mean, float* rstd, void* y, int ydt, const KArgs& a, Workspace ws,
                          hipStream_t st, int block, int vecs);
// Resident path, backward: dgamma/dbeta (either may be null), the per-row dx coefficients,
// and dx unless dx is null; one workgroup per g over all samples, or with split one per
// (n, g) (the same bits).
hipError_t launch_res_bwd(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                          const float* rstd, const float* gamma, const float* beta, float* dgamma,
                          float* dbeta, void* dx, const KArgs& a, Workspace ws, hipStream_t st,
                          int block, int vecs, bool split);

// The partial reductions alone (one float2 per reduction job in ws.part).
hipError_t launch_stats_partials(const void* x, int xdt, const KArgs& a, Workspace ws, hipStream_t st);
hipError_t launch_bwd_partials(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                               const float* rstd, const float* gamma, const float* beta, const KArgs& a,
                               Workspace ws, hipStream_t st);

// ------------------------------------------------------------------ spatial shards
//
// One shard's statistics record per group: mean = mean_hi + mean_lo, m2 = sum of squared
// deviations from that mean, count = elements of the group in the shard. Same layout as
// gn_moments in gn.h.
struct Moments16 {
    float mean_hi, mean_lo, m2;
    uint32_t count;
};

// Forward: the shard's partials -> one record per group (after launch_stats_partials).
hipError_t launch_shard_records(const void* x, int xdt, const KArgs& a, Workspace ws, Moments16* rec,
                                hipStream_t st);
// Forward: P shards' records, merged in shard order -> mean, rstd, normalize coefficients.
hipError_t launch_shard_merge_fwd(const Moments16* rec, int64_t P, const float* gamma, const float* beta,
                                  float eps, float* mean, float* rstd, const KArgs& a, Workspace ws,
                                  hipStream_t st);
// Backward: the shard's partials -> per-row (sum g, rstd * sum g*(x - mean)).
hipError_t launch_shard_sums(const KArgs& a, Workspace ws, float2* sums, hipStream_t st);
// Backward: P shards' sums, merged in shard order -> dgamma, dbeta and dx coefficients.
hipError_t launch_shard_merge_bwd(const float2* sums, int64_t P, const float* mean, const float* rstd,
                                  const float* gamma, const float* beta, int64_t M_total, float* dgamma,
                                  float* dbeta, const KArgs& a, Workspace ws, hipStream_t st);

// ------------------------------------------------------------------ channels-last

struct ClArgs {
    int64_t N, C, S, G, Cg, M;
    int64_t Cv, vps;
    int64_t chunk, K, jobs;
    int64_t chunk_a, K_a, jobs_a;
    int32_t ngl, act;
    int32_t cached;                   // host's choice: plain loads, the volume fits the LLC
    int32_t lcvg;                     // resident path: log2 of a group's vectors per voxel
    FastDiv div_vg;                   // resident path: S * C/(8G), a group's vectors
    // Streaming-job order (job_in_order): as in KArgs, with the streaming jobs of chunk_a
    // voxels nested in the reduction jobs of chunk voxels.
    int32_t fold_nest, fold_R;
    FastDiv div_fold_R;
    int32_t fold_shift;
};

inline ClArgs clargs_of(const PlanCL& p, int act = 0)
{
    ClArgs a;
    a.N = p.N; a.C = p.C; a.S = p.S; a.G = p.G; a.Cg = p.Cg; a.M = p.M;
    a.Cv = p.Cv; a.vps = p.vps;
    a.chunk = p.chunk; a.K = p.K; a.jobs = p.jobs;
    a.chunk_a = p.chunk_a; a.K_a = p.K_a; a.jobs_a = p.jobs_a;
    a.ngl = p.ngl; a.act = act;
    a.cached = 0;
    a.lcvg = p.lcvg;
    a.div_vg = fastdiv_of(p.res_bwd ? p.S << p.lcvg : 0);
    const bool nest = p.chunk_a > 0 && p.chunk % p.chunk_a == 0 && p.K_a == p.K * (p.chunk / p.chunk_a);
    set_job_order(nest ? p.chunk / p.chunk_a : 1, p.jobs_a, a.fold_nest, a.fold_R, a.fold_shift, a.div_fold_R);
    return a;
}

// Channels-last workspace: partials (forward: one float2 per job and group; backward: one
// per job and channel), per-channel float2 coefficients (forward: gamma_c*rstd, beta_c;
// backward: rstd*gamma_c, beta_c) and per-group float4 coefficients (forward: mean head,
// mean tail; backward: mean, -rstd*c1, -rstd^2*c2).
struct WorkspaceCL {
    float2* part;
    float2* partg;   // backward: per job and group, sum over the group's channels of gamma_c * partial_c
    float2* coefc;
    float4* coefg;
};

inline WorkspaceCL workspace_cl_of(void* ws, const PlanCL& p)
{
    char* b = static_cast<char*>(ws);
    return WorkspaceCL{reinterpret_cast<float2*>(b), reinterpret_cast<float2*>(b + p.ws_partg_offset),
                       reinterpret_cast<float2*>(b + p.ws_coefc_offset),
                       reinterpret_cast<float4*>(b + p.ws_coefg_offset)};
}

// Forward, channels-last: statistics, finalize, normalize (three kernels).
hipError_t launch_cl_forward(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                             float* mean, float* rstd, void* y, int ydt, const ClArgs& a,
                             WorkspaceCL ws, hipStream_t st);
// Backward, channels-last: per-channel sums, finalize (dgamma/dbeta, dx coefficients), dx
// unless dx is null.
hipError_t launch_cl_backward(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                              const float* rstd, const float* gamma, const float* beta, void* dx,
                              float* dgamma, float* dbeta, const ClArgs& a, WorkspaceCL ws,
                              hipStream_t st);
// Channels-last resident path, one kernel per direction (block threads, vecs vectors a lane).
hipError_t launch_cl_res_forward(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                                 float* mean, float* rstd, void* y, int ydt, const ClArgs& a, hipStream_t st,
                                 int block, int vecs);
hipError_t launch_cl_res_backward(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                                  const float* rstd, const float* gamma, const float* beta, void* dx,
                                  float* dgamma, float* dbeta, const ClArgs& a, hipStream_t st, int block,
                                  int vecs);

}  // namespace gn
