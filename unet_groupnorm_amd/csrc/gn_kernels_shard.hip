// gn_kernels_shard.hip -- GroupNorm statistics of a volume split into spatial shards.
//
// "Optimize GroupNorm" (LBANN/ScaFFold pull 93), paragraphs on DistConv: the UNet's
// activations are split over GPUs along D/H/W, and GroupNorm normalizes each shard with
// its own statistics; global statistics are left open there. These kernels are the
// per-GPU half of global statistics: a shard's moments per group as one 16-byte record;
// the merge of P shards' records in shard order, the same computation on every rank, so
// that every rank normalizes with bitwise identical statistics; and the backward's per-row
// sums with their merge. Moving the records between GPUs is the caller's (one all-gather:
// N*G records forward, N*C float2 backward); the shard itself is then normalized by the
// streaming kernels of gn_kernels.hip (gn_forward_apply, gn_backward_apply).
#include "gn_device.hpp"

namespace gn {

namespace {

// Records or sums a merge workgroup stages in LDS before its thread 0 merges them in order.
constexpr int64_t kShardStage = 256;

// The shift of group (n, g) within the shard: its first element, 0 if not finite.
template <typename T>
__device__ __forceinline__ float shard_shift(const T* __restrict__ x, const KArgs& a, int64_t n, int64_t g)
{
    const float k = Io<T>::load1(x + (n * a.C + g * a.Cg) * a.S);
    return __builtin_isfinite(k) ? k : 0.0f;
}

__device__ __forceinline__ int64_t shard_job_count(const KArgs& a, int64_t k)
{
    const int64_t end = (k + 1) * a.chunk;
    return (end < a.S ? end : a.S) - k * a.chunk;
}

// One workgroup per group (n, g): the group's C/G * K partials of this shard merged in the
// order of the forward finalize (lane t takes partials t, t + B, ..., then the shuffle
// tree, then the waves in order), written as the shard's record: mean = head + tail
// (head alone when it is infinite), M2 and the element count.
template <typename TX>
__global__ void __launch_bounds__(256)
shard_record_kernel(const TX* __restrict__ x, const float2* __restrict__ part, KArgs a,
                    Moments16* __restrict__ rec)
{
    __shared__ uint64_t s_n[kMaxWaves];
    __shared__ float s_m[kMaxWaves], s_M[kMaxWaves];
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / a.G, g = ng - n * a.G;
    const int64_t pbase = (n * a.C + g * a.Cg) * a.K;
    const float K = shard_shift(x, a, n, g);
    Moments<uint64_t> acc = {0ull, 0.0f, 0.0f};
    for (int64_t j = threadIdx.x; j < a.P; j += blockDim.x) {
        const float2 pm = part[pbase + j];
        chan_merge(acc, uint64_t(shard_job_count(a, j % a.K)), pm.x, pm.y);
    }
    const Moments<uint64_t> r = block_merge(acc, s_n, s_m, s_M);
    if (threadIdx.x == 0) {
        const float hi = K + r.m;
        const float lo = __builtin_isinf(hi) ? 0.0f : (K - hi) + r.m;
        rec[ng] = Moments16{hi, lo, r.M2, uint32_t(r.n)};
    }
}

// One workgroup per group (n, g): thread 0 merges the group's records of shards 0, 1, ...,
// P-1 in that order with Chan's formula, each shard's mean taken relative to shard 0's
// mean head (0 if that is not finite) as (head - shift) + tail; then var = M2 / count,
// rstd, the global mean as head + tail, and the group's rows' normalize coefficients
// (head, tail, gamma_c * rstd, beta_c) for gn_forward_apply.
__global__ void __launch_bounds__(64)
shard_merge_fwd_kernel(const Moments16* __restrict__ rec, int64_t P, const float* __restrict__ gamma,
                       const float* __restrict__ beta, float eps, float* __restrict__ mean_out,
                       float* __restrict__ rstd_out, KArgs a, float4* __restrict__ coef)
{
    __shared__ float s_stat[3];
    __shared__ Moments16 s_rec[kShardStage];
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / a.G, g = ng - n * a.G;
    const int64_t NG = a.N * a.G;
    // The group's records staged in LDS by all threads at once (thread 0's merge then reads
    // them in order without waiting on one global load at a time).
    const bool staged = P <= kShardStage;
    if (staged) {
        for (int64_t p = threadIdx.x; p < P; p += blockDim.x) s_rec[p] = rec[p * NG + ng];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const float k0 = staged ? s_rec[0].mean_hi : rec[ng].mean_hi;
        const float K = __builtin_isfinite(k0) ? k0 : 0.0f;
        Moments<uint64_t> acc = {0ull, 0.0f, 0.0f};
        for (int64_t p = 0; p < P; ++p) {
            const Moments16 r = staged ? s_rec[p] : rec[p * NG + ng];
            chan_merge(acc, uint64_t(r.count), (r.mean_hi - K) + r.mean_lo, r.m2);
        }
        float var = float(double(acc.M2) / double(acc.n));
        var = (var < 0.0f) ? 0.0f : var;  // NaN passes through
        const float rstd = 1.0f / __fsqrt_rn(var + eps);
        const float hi = K + acc.m;
        const float lo = (K - hi) + acc.m;
        mean_out[ng] = hi;
        rstd_out[ng] = rstd;
        s_stat[0] = hi; s_stat[1] = lo; s_stat[2] = rstd;
    }
    __syncthreads();
    const float hi = s_stat[0], lo = s_stat[1], rstd = s_stat[2];
    for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) {
        const int64_t c = g * a.Cg + i;
        coef[2 * (n * a.C + c)] = make_float4(hi, lo, (gamma ? gamma[c] : 1.0f) * rstd, beta ? beta[c] : 0.0f);
    }
}

// One workgroup per row (n, c): the row's K backward partials of this shard summed in a
// fixed order (lane t takes partials t, t + B, ..., then the shuffle tree, then the waves
// in order): (sum g, rstd * sum g*(x - mean)) with the global mean and rstd.
__global__ void __launch_bounds__(256)
shard_sums_kernel(const float2* __restrict__ part, KArgs a, float2* __restrict__ sums)
{
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    const int64_t row = blockIdx.x;
    float t1 = 0.0f, t2 = 0.0f;
    for (int64_t j = threadIdx.x; j < a.K; j += blockDim.x) {
        const float2 pp = part[row * a.K + j];
        t1 = t1 + pp.x;
        t2 = t2 + pp.y;
    }
    const float2 r = block_sum2(t1, t2, s_a, s_b);
    if (threadIdx.x == 0) sums[row] = r;
}

// Workgroups [0, ngroups): group (n, g). Thread 0 sums each channel's (s1, s2) over shards
// 0..P-1 in order, then c1 = (1/M) sum gamma_c s1 and c2 = (1/M) sum gamma_c s2 over the
// group's channels in order, M the group's element count over all shards; the group's rows
// get the dx coefficients (mean, rstd*gamma_c, -rstd*c1, -rstd^2*c2) and (beta_c, 1 if M is
// 1 else 0) for gn_backward_apply. Workgroups [ngroups, ngroups + nchan): channel c, whose dgamma and
// dbeta are the sums over samples (outer) and shards (inner), in order.
__global__ void __launch_bounds__(64)
shard_merge_bwd_kernel(const float2* __restrict__ sums, int64_t P, const float* __restrict__ mean,
                       const float* __restrict__ rstd, const float* __restrict__ gamma,
                       const float* __restrict__ beta, int64_t M_total, KArgs a, int64_t ngroups,
                       int64_t nchan, float4* __restrict__ coef, float* __restrict__ dgamma,
                       float* __restrict__ dbeta)
{
    __shared__ float s_coef[2];
    __shared__ float2 s_sum[kShardStage];
    __shared__ float s_gm[kShardStage];
    const int64_t w = blockIdx.x;
    const int64_t NC = a.N * a.C;
    if (w < ngroups) {
        const int64_t n = w / a.G, g = w - n * a.G;
        const float mu = mean[w], rs = rstd[w];
        // The group's (shard, channel) sums and gammas staged in LDS, [i][p], by all threads.
        const bool staged = a.Cg * P <= kShardStage;
        if (staged) {
            for (int64_t q = threadIdx.x; q < a.Cg * P; q += blockDim.x) {
                const int64_t i = q / P, p = q - i * P;
                s_sum[q] = sums[p * NC + n * a.C + g * a.Cg + i];
            }
            for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) s_gm[i] = gamma ? gamma[g * a.Cg + i] : 1.0f;
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            float t1 = 0.0f, t2 = 0.0f;
            for (int64_t i = 0; i < a.Cg; ++i) {
                const int64_t c = g * a.Cg + i;
                float s1 = 0.0f, s2 = 0.0f;
                for (int64_t p = 0; p < P; ++p) {
                    const float2 v = staged ? s_sum[i * P + p] : sums[p * NC + n * a.C + c];
                    s1 = s1 + v.x;
                    s2 = s2 + v.y;
                }
                const float gm = staged ? s_gm[i] : (gamma ? gamma[c] : 1.0f);
                t1 = t1 + gm * s1;
                t2 = t2 + gm * s2;
            }
            s_coef[0] = float(double(t1) / double(M_total));
            s_coef[1] = float(double(t2) / double(M_total));
        }
        __syncthreads();
        const float B = -(rs * s_coef[0]);
        const float E = -((rs * rs) * s_coef[1]);
        for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) {
            const int64_t c = g * a.Cg + i;
            const float gm = gamma ? gamma[c] : 1.0f;
            coef[2 * (n * a.C + c)] = make_float4(mu, rs * gm, B, E);
            coef[2 * (n * a.C + c) + 1] = make_float4(beta ? beta[c] : 0.0f, M_total == 1 ? 1.0f : 0.0f, 0.0f, 0.0f);
        }
    } else if (w < ngroups + nchan) {
        const int64_t c = w - ngroups;
        // The channel's (sample, shard) sums staged in LDS, [n][p], by all threads.
        const bool staged = a.N * P <= kShardStage;
        if (staged) {
            for (int64_t q = threadIdx.x; q < a.N * P; q += blockDim.x) {
                const int64_t n = q / P, p = q - n * P;
                s_sum[q] = sums[p * NC + n * a.C + c];
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            float q1 = 0.0f, q2 = 0.0f;
            for (int64_t n = 0; n < a.N; ++n) {
                for (int64_t p = 0; p < P; ++p) {
                    const float2 v = staged ? s_sum[n * P + p] : sums[p * NC + n * a.C + c];
                    q1 = q1 + v.y;
                    q2 = q2 + v.x;
                }
            }
            if (dgamma) dgamma[c] = q1;
            if (dbeta) dbeta[c] = q2;
        }
    }
}

}  // namespace

hipError_t launch_shard_records(const void* x, int xdt, const KArgs& a, Workspace ws, Moments16* rec,
                                hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
        using TX = decltype(tx);
        return launch(shard_record_kernel<TX>, dim3(unsigned(a.N * a.G)), dim3(256), st, cp<TX>(x),
                      static_cast<const float2*>(ws.part), a, rec);
    });
}

hipError_t launch_shard_merge_fwd(const Moments16* rec, int64_t P, const float* gamma, const float* beta,
                                  float eps, float* mean, float* rstd, const KArgs& a, Workspace ws,
                                  hipStream_t st)
{
    return launch(shard_merge_fwd_kernel, dim3(unsigned(a.N * a.G)), dim3(64), st, rec, P, gamma, beta, eps,
                  mean, rstd, a, ws.coef);
}

hipError_t launch_shard_sums(const KArgs& a, Workspace ws, float2* sums, hipStream_t st)
{
    return launch(shard_sums_kernel, dim3(unsigned(a.N * a.C)), dim3(256), st,
                  static_cast<const float2*>(ws.part), a, sums);
}

hipError_t launch_shard_merge_bwd(const float2* sums, int64_t P, const float* mean, const float* rstd,
                                  const float* gamma, const float* beta, int64_t M_total, float* dgamma,
                                  float* dbeta, const KArgs& a, Workspace ws, hipStream_t st)
{
    const int64_t ngroups = a.N * a.G;
    const int64_t nchan = (dgamma || dbeta) ? a.C : 0;
    return launch(shard_merge_bwd_kernel, dim3(unsigned(ngroups + nchan)), dim3(64), st, sums, P, mean, rstd,
                  gamma, beta, M_total, a, ngroups, nchan, ws.coef, dgamma, dbeta);
}

}  // namespace gn
