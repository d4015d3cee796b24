// gn_kernels_cl.hip -- GroupNorm over channels-last (NDHWC) activations on gfx950.
//
// "Optimize GroupNorm" (LBANN/ScaFFold pull 93), paragraph introducing the NDHWC kernel:
// reading a contiguous span of voxels with every channel of each gives all groups'
// statistics in one coalesced sweep; visiting channels-last memory channel by channel
// instead would read with a stride of C.
//
// x[n][s][c] sits at (n*S + s)*C + c with C a multiple of 8, so a voxel is C/8 whole
// vectors. Lane t of a workgroup owns channel vector cv = t mod (C/8) (channels 8cv ..
// 8cv+7) for a whole job, and voxel t / (C/8) + r*vps of each round r (vps = B / (C/8)
// voxels per round). Its 8 channels lie in NGL = max(1, 8 / (C/G)) groups, the lane's
// "slots". Numerics follow the NCDHW kernels: fp32 throughout, every statistic relative to
// the group's first element, corrected two-pass tiles merged with Chan's formula, lanes
// and waves merged in a fixed order, no atomics. The mapping is defined on elements, so
// fp32, bf16 and fp16 data reduce in the same order.
//
// Five kernels: statistics per (job, group), their finalize per group, normalize; per
// (job, channel) backward sums, their finalize (dx coefficients per group and channel,
// dgamma/dbeta per channel), dx.
#include "gn_device.hpp"

namespace gn {

namespace {

constexpr int kClWaves = kClBlock / 64;
// Partials a finalize thread requests at once.
constexpr int kBatch = 8;

// The shift of group (n, g): its first element (channel g*C/G of voxel 0), 0 if not finite.
template <typename T>
__device__ __forceinline__ float cl_group_shift(const T* __restrict__ x, const ClArgs& a, int64_t n, int64_t g)
{
    const float k = Io<T>::load1(x + n * a.S * a.C + g * a.Cg);
    return __builtin_isfinite(k) ? k : 0.0f;
}

// Voxels of reduction job k of a sample (the plan fixes it; it is never stored).
__device__ __forceinline__ int64_t cl_job_voxels(const ClArgs& a, int64_t k)
{
    const int64_t end = (k + 1) * a.chunk;
    return (end < a.S ? end : a.S) - k * a.chunk;
}

// Lanes of a wave that own the same channel vector are Cv apart (Cv a power of two). Lane
// i takes lane i + off for off = 32, 16, ..., Cv; lanes 0 .. min(Cv, 64) - 1 then hold the
// merge over their channel vector's lanes of the wave. At each level only lanes i < off
// feed those lanes, which is what lane_down guarantees. Cv is the same for every lane, so
// the level tests are scalar branches and every lane stays active.
template <typename CT>
__device__ __forceinline__ void wave_merge_stride(Moments<CT>& a, int Cv)
{
    if (Cv <= 32) wave_merge_level<32>(a);
    if (Cv <= 16) wave_merge_level<16>(a);
    if (Cv <= 8) wave_merge_level<8>(a);
    if (Cv <= 4) wave_merge_level<4>(a);
    if (Cv <= 2) wave_merge_level<2>(a);
    if (Cv <= 1) wave_merge_level<1>(a);
}

__device__ __forceinline__ float wave_sum_stride(float v, int Cv)
{
    if (Cv <= 32) v = v + lane_down<32>(v);
    if (Cv <= 16) v = v + lane_down<16>(v);
    if (Cv <= 8) v = v + lane_down<8>(v);
    if (Cv <= 4) v = v + lane_down<4>(v);
    if (Cv <= 2) v = v + lane_down<2>(v);
    if (Cv <= 1) v = v + lane_down<1>(v);
    return v;
}

// The lane of wave w that holds channel vector c after the strided merge (or -1): with
// Cv <= 64 every wave holds every vector in lane c; with Cv > 64 wave w's lane l holds
// vector (64w + l) mod Cv.
__device__ __forceinline__ int cl_holder(int c, int w, int Cv)
{
    const int l = ((c - 64 * w) % Cv + Cv) % Cv;
    return l < 64 ? l : -1;
}

// The channel vectors [lo, hi) and slot that make up group g.
__device__ __forceinline__ void cl_group_vectors(const ClArgs& a, int64_t g, int& lo, int& hi, int& slot)
{
    if (a.Cg < kVec) {
        lo = int((g * a.Cg) / kVec);
        hi = lo + 1;
        slot = int(((g * a.Cg) % kVec) / a.Cg);
    } else {
        lo = int((g * a.Cg) / kVec);
        hi = int(((g + 1) * a.Cg) / kVec);
        slot = 0;
    }
}

// Corrected two-pass over an N-element tile of shifted values t (all valid): m = mean,
// M2 = sum d^2 - (sum d)^2 / N with d = t - m. N is a power of two.
template <int N>
__device__ __forceinline__ void cl_tile_full(float (&t)[N], float& m, float& M2)
{
    m = tree_sum(t) * (1.0f / N);
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = t[i] - m;
    const float sd = tree_sum(t);
    const float sq = tree_sumsq(t);
    M2 = sq - (sd * sd) * (1.0f / N);
}

// Same with a validity mask (invalid entries hold 0 and contribute nothing).
template <int N>
__device__ __forceinline__ void cl_tile_masked(float (&t)[N], uint32_t valid, float cnt, float& m, float& M2)
{
    m = tree_sum(t) / cnt;
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = ((valid >> i) & 1u) ? t[i] - m : 0.0f;
    const float sd = tree_sum(t);
    const float sq = tree_sumsq(t);
    M2 = sq - (sd * sd) / cnt;
}

// ------------------------------------------------------------------ forward

// One step's raw vectors: round r of the lane at voxel s0 + r*vps (all inside the job).
template <bool NT, typename T>
__device__ __forceinline__ void cl_load_step(const T* __restrict__ p, int64_t s0, int vps, int64_t C,
                                             typename Io<T>::Raw (&R)[kClRounds])
{
#pragma unroll
    for (int r = 0; r < kClRounds; ++r) R[r] = Io<T>::template load_raw<NT>(p + (s0 + int64_t(r) * vps) * C);
}

// Tiles of one step (rounds that are in the job: bit r of `valid`) merged into the lane's
// slot accumulators.
template <int NGL>
__device__ __forceinline__ void cl_stats_step(const float (&e)[kClRounds][kVec], uint32_t valid, bool full,
                                              const float (&Ks)[NGL], Moments<uint32_t> (&acc)[NGL])
{
    constexpr int W = kVec / NGL;
    constexpr int T = kClRounds * W;
#pragma unroll
    for (int q = 0; q < NGL; ++q) {
        float t[T];
        uint32_t tv = 0;
#pragma unroll
        for (int r = 0; r < kClRounds; ++r) {
            const bool ok = (valid >> r) & 1u;
#pragma unroll
            for (int i = 0; i < W; ++i) t[r * W + i] = ok ? e[r][q * W + i] - Ks[q] : 0.0f;
            if (ok) tv |= ((1u << W) - 1u) << (r * W);
        }
        float m, M2;
        if (full) {
            cl_tile_full(t, m, M2);
            chan_merge(acc[q], uint32_t(T), m, M2);
        } else if (tv) {
            const uint32_t cnt = __builtin_popcount(tv);
            cl_tile_masked(t, tv, float(cnt), m, M2);
            chan_merge(acc[q], cnt, m, M2);
        }
    }
}

template <int NGL, typename TX>
__device__ __forceinline__ void cl_stats_full(const typename Io<TX>::Raw (&R)[kClRounds], const float (&Ks)[NGL],
                                              Moments<uint32_t> (&acc)[NGL])
{
    float e[kClRounds][kVec];
#pragma unroll
    for (int r = 0; r < kClRounds; ++r) Io<TX>::widen(R[r], e[r]);
    cl_stats_step<NGL>(e, (1u << kClRounds) - 1u, true, Ks, acc);
}

// Per reduction job (n, voxels [v0, v1)): (mean relative to the shift, M2) of every group,
// stored group-major: part[(g*N + n)*K + k]. The full steps are software-pipelined (the
// next step's vectors are requested before the current one is reduced, alternating two
// register sets); a last partial step is masked by voxel.
template <int NGL, typename TX, bool NT>
__global__ void __launch_bounds__(kClBlock)
cl_stats_kernel(const TX* __restrict__ x, ClArgs a, float2* __restrict__ part)
{
    using Raw = typename Io<TX>::Raw;
    __shared__ uint32_t s_n[kClBlock * NGL];
    __shared__ float s_m[kClBlock * NGL], s_M[kClBlock * NGL];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Cv = int(a.Cv), cv = tid % Cv, vo = tid / Cv, vps = int(a.vps);
    const int reps = Cv < 64 ? Cv : 64;
    const int64_t g0 = (int64_t(cv) * kVec) / a.Cg;
    const int64_t step = int64_t(kClRounds) * vps;
    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const int64_t n = j / a.K, k = j - n * a.K;
        const int64_t v0 = k * a.chunk, v1 = (v0 + a.chunk < a.S) ? v0 + a.chunk : a.S;
        const TX* xs = x + n * a.S * a.C + int64_t(cv) * kVec + int64_t(vo) * a.C;
        float Ks[NGL];
#pragma unroll
        for (int q = 0; q < NGL; ++q) Ks[q] = cl_group_shift(x, a, n, g0 + q);
        Moments<uint32_t> acc[NGL];
#pragma unroll
        for (int q = 0; q < NGL; ++q) acc[q] = {0u, 0.0f, 0.0f};
        const int64_t nfull = (v1 - v0) / step;
        if (nfull > 0) {
            Raw A[kClRounds], B[kClRounds];
            cl_load_step<NT>(xs, v0, vps, a.C, A);
            int64_t s = 0;
            for (; s + 2 < nfull; s += 2) {
                cl_load_step<NT>(xs, v0 + (s + 1) * step, vps, a.C, B);
                cl_stats_full<NGL, TX>(A, Ks, acc);
                cl_load_step<NT>(xs, v0 + (s + 2) * step, vps, a.C, A);
                cl_stats_full<NGL, TX>(B, Ks, acc);
            }
            if (s + 1 < nfull) {
                cl_load_step<NT>(xs, v0 + (s + 1) * step, vps, a.C, B);
                cl_stats_full<NGL, TX>(A, Ks, acc);
                cl_stats_full<NGL, TX>(B, Ks, acc);
            } else {
                cl_stats_full<NGL, TX>(A, Ks, acc);
            }
        }
        const int64_t st = v0 + nfull * step;
        if (st < v1) {
            float e[kClRounds][kVec];
            uint32_t valid = 0;
#pragma unroll
            for (int r = 0; r < kClRounds; ++r) {
                const int64_t vox = st + int64_t(r) * vps + vo;
                if (vox < v1) {
                    Io<TX>::template load8<NT>(xs + (st + int64_t(r) * vps) * a.C, e[r]);
                    valid |= 1u << r;
                } else {
#pragma unroll
                    for (int i = 0; i < kVec; ++i) e[r][i] = 0.0f;
                }
            }
            cl_stats_step<NGL>(e, valid, false, Ks, acc);
        }
#pragma unroll
        for (int q = 0; q < NGL; ++q) wave_merge_stride(acc[q], Cv);
        if (lane < reps) {
#pragma unroll
            for (int q = 0; q < NGL; ++q) {
                const int idx = (wave * 64 + lane) * NGL + q;
                s_n[idx] = acc[q].n; s_m[idx] = acc[q].m; s_M[idx] = acc[q].M2;
            }
        }
        __syncthreads();
        for (int64_t g = tid; g < a.G; g += blockDim.x) {
            int lo, hi, q;
            cl_group_vectors(a, g, lo, hi, q);
            Moments<uint32_t> r = {0u, 0.0f, 0.0f};
            for (int w = 0; w < kClWaves; ++w) {
                for (int c = lo; c < hi; ++c) {
                    const int l = cl_holder(c, w, Cv);
                    if (l >= 0) {
                        const int idx = (w * 64 + l) * NGL + q;
                        chan_merge(r, s_n[idx], s_m[idx], s_M[idx]);
                    }
                }
            }
            part[(g * a.N + n) * a.K + k] = make_float2(r.m, r.M2);
        }
        __syncthreads();
    }
}

// One workgroup per group (n, g): the group's K partials (contiguous) merged in a fixed order (lane t
// takes partials t, t + B, ..., then the shuffle tree, then the waves in order); mean,
// rstd; the group's (mean head, mean tail) and each channel's (gamma_c * rstd, beta_c).
template <typename TX>
__global__ void __launch_bounds__(256)
cl_fin_fwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                  float eps, const float2* __restrict__ part, float* __restrict__ mean_out,
                  float* __restrict__ rstd_out, ClArgs a, float2* __restrict__ coefc, float4* __restrict__ coefg)
{
    __shared__ uint64_t s_n[kMaxWaves];
    __shared__ float s_m[kMaxWaves], s_M[kMaxWaves];
    __shared__ float s_stat[3];
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / a.G, g = ng - n * a.G;
    const float K = cl_group_shift(x, a, n, g);
    Moments<uint64_t> acc = {0ull, 0.0f, 0.0f};
    const float2* pg = part + (g * a.N + n) * a.K;
    // Partials t, t + B, ... in index order; requested kBatch at a time so that their
    // latencies overlap.
    for (int64_t k0 = threadIdx.x; k0 < a.K; k0 += kBatch * blockDim.x) {
        float2 pm[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t kk = k0 + int64_t(u) * blockDim.x;
            pm[u] = kk < a.K ? pg[kk] : make_float2(0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t kk = k0 + int64_t(u) * blockDim.x;
            if (kk < a.K) chan_merge(acc, uint64_t(cl_job_voxels(a, kk) * a.Cg), pm[u].x, pm[u].y);
        }
    }
    const Moments<uint64_t> r = block_merge(acc, s_n, s_m, s_M);
    if (threadIdx.x == 0) {
        float var = float(double(r.M2) / double(a.M));
        var = (var < 0.0f) ? 0.0f : var;  // NaN passes through
        const float rstd = 1.0f / __fsqrt_rn(var + eps);
        const float hi = K + r.m;
        const float lo = (K - hi) + r.m;
        mean_out[ng] = hi;
        rstd_out[ng] = rstd;
        coefg[ng] = make_float4(hi, lo, 0.0f, 0.0f);
        s_stat[0] = rstd;
    }
    __syncthreads();
    const float rstd = s_stat[0];
    for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) {
        const int64_t c = g * a.Cg + i;
        coefc[n * a.C + c] = make_float2((gamma ? gamma[c] : 1.0f) * rstd, beta ? beta[c] : 0.0f);
    }
}

// The lane's 8 per-channel coefficient pairs (64 bytes, 16-byte aligned).
__device__ __forceinline__ void cl_load_coefc(const float2* __restrict__ p, float (&u)[kVec], float (&v)[kVec])
{
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int h = 0; h < kVec / 2; ++h) {
        const float4 c = q[h];
        u[2 * h] = c.x; v[2 * h] = c.y;
        u[2 * h + 1] = c.z; v[2 * h + 1] = c.w;
    }
}

// y = ((x - head) - tail) * gamma_c*rstd + beta_c, optional relu, one narrowing store; a
// streaming job is kClApplyRounds rounds of a workgroup over one sample's voxels.
template <int NGL, typename TX, typename TY, bool NT, bool ACT>
__global__ void __launch_bounds__(kClBlock)
cl_apply_kernel(const TX* __restrict__ x, TY* __restrict__ y, ClArgs a, const float2* __restrict__ coefc,
                const float4* __restrict__ coefg)
{
    constexpr int W = kVec / NGL;
    const int tid = threadIdx.x;
    const int Cv = int(a.Cv), cv = tid % Cv, vo = tid / Cv, vps = int(a.vps);
    const int64_t g0 = (int64_t(cv) * kVec) / a.Cg;
    constexpr bool act = ACT;  // a template parameter, as in the NCDHW streaming kernels
    for (int64_t jj = blockIdx.x; jj < a.jobs_a; jj += gridDim.x) {
        const int64_t j = job_in_order(jj, a);
        const int64_t n = j / a.K_a, k = j - n * a.K_a;
        const int64_t v0 = k * a.chunk_a, v1 = (v0 + a.chunk_a < a.S) ? v0 + a.chunk_a : a.S;
        float sc[kVec], sh[kVec], hi[NGL], lo[NGL];
        cl_load_coefc(coefc + n * a.C + int64_t(cv) * kVec, sc, sh);
#pragma unroll
        for (int q = 0; q < NGL; ++q) {
            const float4 cg = coefg[n * a.G + g0 + q];
            hi[q] = cg.x; lo[q] = cg.y;
        }
#pragma unroll
        for (int r = 0; r < kClApplyRounds; ++r) {
            const int64_t vox = v0 + int64_t(r) * vps + vo;
            if (vox < v1) {
                const int64_t off = (n * a.S + vox) * a.C + int64_t(cv) * kVec;
                float e[kVec], o[kVec];
                Io<TX>::template load8<NT>(x + off, e);
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const float v = fmaf((e[i] - hi[i / W]) - lo[i / W], sc[i], sh[i]);
                    o[i] = act ? relu_f(v) : v;
                }
                // y goes out with nontemporal stores, so the backward sums that follow do
                // not find it as dirty lines to write back (MI355X, bf16, C=32, G=8 step:
                // 128^3 187.3 -> 186.1 us, 256^3 1400.7 -> 1382.8 us); dx keeps plain stores
                // (nontemporal in both kernels: 128^3 189 -> 198 us).
                Io<TY>::template store8<true>(y + off, o);
            }
        }
    }
}

// ------------------------------------------------------------------ backward

// One round of the backward sums: per channel, g and g*(x - mean) added to the step's sums
// (rounds in order within a step, steps in order within the job).
template <int NGL, bool ACT>
__device__ __forceinline__ void cl_bwd_round(const float (&e)[kVec], const float (&f)[kVec], const float (&mu)[NGL],
                                             const float (&A)[kVec], const float (&bt)[kVec],
                                             float (&p1)[kVec], float (&p2)[kVec])
{
    constexpr int W = kVec / NGL;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
        const float d = e[i] - mu[i / W];
        const float gv = ACT ? relu_gate(fmaf(d, A[i], bt[i]), f[i]) : f[i];
        p1[i] = p1[i] + gv;
        p2[i] = p2[i] + gv * d;
    }
}

template <int NGL, bool ACT, typename TX, typename TD>
__device__ __forceinline__ void cl_bwd_full(const typename Io<TX>::Raw (&RX)[kClRounds],
                                            const typename Io<TD>::Raw (&RD)[kClRounds], const float (&mu)[NGL],
                                            const float (&A)[kVec], const float (&bt)[kVec],
                                            float (&s1)[kVec], float (&s2)[kVec])
{
    float p1[kVec], p2[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) { p1[i] = 0.0f; p2[i] = 0.0f; }
#pragma unroll
    for (int r = 0; r < kClRounds; ++r) {
        float e[kVec], f[kVec];
        Io<TX>::widen(RX[r], e);
        Io<TD>::widen(RD[r], f);
        cl_bwd_round<NGL, ACT>(e, f, mu, A, bt, p1, p2);
    }
#pragma unroll
    for (int i = 0; i < kVec; ++i) { s1[i] = s1[i] + p1[i]; s2[i] = s2[i] + p2[i]; }
}

// Per reduction job: s1 = sum g and s2 = rstd * sum g*(x - mean) for every channel, g = dy
// or dy gated by the relu on pre = (x - mean) * rstd*gamma_c + beta_c, stored channel-major:
// part[(c*N + n)*K + k]. A lane sums its rounds in order within a step and the steps in
// order (full steps software-pipelined as in cl_stats_kernel); lanes sharing a channel
// vector in the shuffle tree; waves in order.
template <int NGL, bool ACT, typename TX, typename TD, bool NT>
__global__ void __launch_bounds__(kClBlock)
cl_bwd_reduce_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ mean,
                     const float* __restrict__ rstd, const float* __restrict__ gamma,
                     const float* __restrict__ beta, ClArgs a, float2* __restrict__ part,
                     float2* __restrict__ partg)
{
    using RawX = typename Io<TX>::Raw;
    using RawD = typename Io<TD>::Raw;
    constexpr int W = kVec / NGL;
    __shared__ float s_1[kClBlock * kVec], s_2[kClBlock * kVec];
    __shared__ float s_c1[kClBlock * kVec], s_c2[kClBlock * kVec];  // per channel, gamma-weighted
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Cv = int(a.Cv), cv = tid % Cv, vo = tid / Cv, vps = int(a.vps);
    const int reps = Cv < 64 ? Cv : 64;
    const int64_t g0 = (int64_t(cv) * kVec) / a.Cg;
    const int64_t step = int64_t(kClRounds) * vps;
    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const int64_t n = j / a.K, k = j - n * a.K;
        const int64_t v0 = k * a.chunk, v1 = (v0 + a.chunk < a.S) ? v0 + a.chunk : a.S;
        const int64_t base = n * a.S * a.C + int64_t(cv) * kVec + int64_t(vo) * a.C;
        const TX* xs = x + base;
        const TD* ds = dy + base;
        float mu[NGL], A[kVec], bt[kVec];
#pragma unroll
        for (int q = 0; q < NGL; ++q) mu[q] = mean[n * a.G + g0 + q];
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            const int64_t c = int64_t(cv) * kVec + i;
            A[i] = ACT ? rstd[n * a.G + g0 + i / W] * (gamma ? gamma[c] : 1.0f) : 0.0f;
            bt[i] = ACT ? (beta ? beta[c] : 0.0f) : 0.0f;
        }
        float s1[kVec], s2[kVec];
#pragma unroll
        for (int i = 0; i < kVec; ++i) { s1[i] = 0.0f; s2[i] = 0.0f; }
        const int64_t nfull = (v1 - v0) / step;
        if (nfull > 0) {
            RawX AX[kClRounds], BX[kClRounds];
            RawD AD[kClRounds], BD[kClRounds];
            cl_load_step<NT>(xs, v0, vps, a.C, AX);
            cl_load_step<NT>(ds, v0, vps, a.C, AD);
            int64_t s = 0;
            for (; s + 2 < nfull; s += 2) {
                cl_load_step<NT>(xs, v0 + (s + 1) * step, vps, a.C, BX);
                cl_load_step<NT>(ds, v0 + (s + 1) * step, vps, a.C, BD);
                cl_bwd_full<NGL, ACT, TX, TD>(AX, AD, mu, A, bt, s1, s2);
                cl_load_step<NT>(xs, v0 + (s + 2) * step, vps, a.C, AX);
                cl_load_step<NT>(ds, v0 + (s + 2) * step, vps, a.C, AD);
                cl_bwd_full<NGL, ACT, TX, TD>(BX, BD, mu, A, bt, s1, s2);
            }
            if (s + 1 < nfull) {
                cl_load_step<NT>(xs, v0 + (s + 1) * step, vps, a.C, BX);
                cl_load_step<NT>(ds, v0 + (s + 1) * step, vps, a.C, BD);
                cl_bwd_full<NGL, ACT, TX, TD>(AX, AD, mu, A, bt, s1, s2);
                cl_bwd_full<NGL, ACT, TX, TD>(BX, BD, mu, A, bt, s1, s2);
            } else {
                cl_bwd_full<NGL, ACT, TX, TD>(AX, AD, mu, A, bt, s1, s2);
            }
        }
        const int64_t st = v0 + nfull * step;
        if (st < v1) {
            float p1[kVec], p2[kVec];
#pragma unroll
            for (int i = 0; i < kVec; ++i) { p1[i] = 0.0f; p2[i] = 0.0f; }
#pragma unroll
            for (int r = 0; r < kClRounds; ++r) {
                const int64_t vox = st + int64_t(r) * vps + vo;
                if (vox < v1) {
                    float e[kVec], f[kVec];
                    Io<TX>::template load8<NT>(xs + (st + int64_t(r) * vps) * a.C, e);
                    Io<TD>::template load8<NT>(ds + (st + int64_t(r) * vps) * a.C, f);
                    cl_bwd_round<NGL, ACT>(e, f, mu, A, bt, p1, p2);
                }
            }
#pragma unroll
            for (int i = 0; i < kVec; ++i) { s1[i] = s1[i] + p1[i]; s2[i] = s2[i] + p2[i]; }
        }
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            s1[i] = wave_sum_stride(s1[i], Cv);
            s2[i] = wave_sum_stride(s2[i], Cv);
        }
        if (lane < reps) {
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                s_1[(wave * 64 + lane) * kVec + i] = s1[i];
                s_2[(wave * 64 + lane) * kVec + i] = s2[i];
            }
        }
        __syncthreads();
        for (int64_t c = tid; c < a.C; c += blockDim.x) {
            const int cvq = int(c / kVec), i = int(c % kVec);
            float t1 = 0.0f, t2 = 0.0f;
            for (int w = 0; w < kClWaves; ++w) {
                const int l = cl_holder(cvq, w, Cv);
                if (l >= 0) {
                    t1 = t1 + s_1[(w * 64 + l) * kVec + i];
                    t2 = t2 + s_2[(w * 64 + l) * kVec + i];
                }
            }
            const float s2c = t2 * rstd[n * a.G + c / a.Cg];
            part[(c * a.N + n) * a.K + k] = make_float2(t1, s2c);
            const float gm = gamma ? gamma[c] : 1.0f;
            s_c1[c] = gm * t1;
            s_c2[c] = gm * s2c;
        }
        __syncthreads();
        // per group: the gamma-weighted channel sums in channel order
        for (int64_t g = tid; g < a.G; g += blockDim.x) {
            float u1 = 0.0f, u2 = 0.0f;
            for (int64_t i = 0; i < a.Cg; ++i) {
                u1 = u1 + s_c1[g * a.Cg + i];
                u2 = u2 + s_c2[g * a.Cg + i];
            }
            partg[(g * a.N + n) * a.K + k] = make_float2(u1, u2);
        }
        __syncthreads();
    }
}

// Workgroups [0, ngroups) each take one group (n, g): c1 = (1/M) sum gamma_c s1 and
// c2 = (1/M) sum gamma_c s2 over the group's K per-job gamma-weighted partials in a fixed
// order (lane t takes jobs t, t + B, ..., then the shuffle tree, then the waves), then (mean, B = -rstd*c1, E = -rstd^2*c2) per group and (A = rstd*gamma_c,
// beta_c) per channel, so that dx = A*g + (B + E*(x - mean)). Workgroups [ngroups,
// ngroups + nchan) each take one channel: dgamma_c and dbeta_c over its N*K partials.
__global__ void __launch_bounds__(256)
cl_fin_bwd_kernel(const float* __restrict__ mean, const float* __restrict__ rstd,
                  const float* __restrict__ gamma, const float* __restrict__ beta,
                  const float2* __restrict__ part, const float2* __restrict__ partg, ClArgs a,
                  int64_t ngroups, int64_t nchan,
                  float2* __restrict__ coefc, float4* __restrict__ coefg, float* __restrict__ dgamma,
                  float* __restrict__ dbeta)
{
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    __shared__ float s_coef[2];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t w = blockIdx.x;
    if (w < ngroups) {
        const int64_t n = w / a.G, g = w - n * a.G;
        const float mu = mean[w], rs = rstd[w];
        float t1 = 0.0f, t2 = 0.0f;
        const float2* pg = partg + (g * a.N + n) * a.K;
        for (int64_t k0 = tid; k0 < a.K; k0 += kBatch * blk) {
            float2 pp[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t kk = k0 + int64_t(u) * blk;
                pp[u] = kk < a.K ? pg[kk] : make_float2(0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (k0 + int64_t(u) * blk < a.K) {
                    t1 = t1 + pp[u].x;
                    t2 = t2 + pp[u].y;
                }
            }
        }
        const float2 r = block_sum2(t1, t2, s_a, s_b);
        if (tid == 0) {
            s_coef[0] = float(double(r.x) / double(a.M));
            s_coef[1] = float(double(r.y) / double(a.M));
        }
        __syncthreads();
        const float B = -(rs * s_coef[0]);
        const float E = -((rs * rs) * s_coef[1]);
        if (tid == 0) coefg[w] = make_float4(mu, B, E, 0.0f);
        for (int64_t i = tid; i < a.Cg; i += blk) {
            const int64_t c = g * a.Cg + i;
            coefc[n * a.C + c] = make_float2(rs * (gamma ? gamma[c] : 1.0f), beta ? beta[c] : 0.0f);
        }
    } else if (w < ngroups + nchan) {
        const int64_t c = w - ngroups;
        float sa = 0.0f, sb = 0.0f;
        const int64_t cnt = a.N * a.K;
        const float2* pc = part + c * cnt;
        for (int64_t i0 = tid; i0 < cnt; i0 += kBatch * blk) {
            float2 pp[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t i = i0 + int64_t(u) * blk;
                pp[u] = i < cnt ? pc[i] : make_float2(0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (i0 + int64_t(u) * blk < cnt) {
                    sa = sa + pp[u].y;
                    sb = sb + pp[u].x;
                }
            }
        }
        const float2 r = block_sum2(sa, sb, s_a, s_b);
        if (tid == 0) {
            if (dgamma) dgamma[c] = r.x;
            if (dbeta) dbeta[c] = r.y;
        }
    }
}

// dx = A*g + (B + E*(x - mean)), g = dy or the relu-gated dy, narrowed once to x's dtype.
template <int NGL, typename TX, typename TD, bool NT>
__global__ void __launch_bounds__(kClBlock)
cl_bwd_apply_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, ClArgs a,
                    const float2* __restrict__ coefc, const float4* __restrict__ coefg, TX* __restrict__ dx)
{
    constexpr int W = kVec / NGL;
    const int tid = threadIdx.x;
    const int Cv = int(a.Cv), cv = tid % Cv, vo = tid / Cv, vps = int(a.vps);
    const int64_t g0 = (int64_t(cv) * kVec) / a.Cg;
    const bool act = a.act != 0;
    // A single-element group is answered as t - t: +0 for finite t, NaN otherwise.
    const bool single = (a.M == 1);
    for (int64_t jj = blockIdx.x; jj < a.jobs_a; jj += gridDim.x) {
        const int64_t j = job_in_order(jj, a);
        const int64_t n = j / a.K_a, k = j - n * a.K_a;
        const int64_t v0 = k * a.chunk_a, v1 = (v0 + a.chunk_a < a.S) ? v0 + a.chunk_a : a.S;
        float A[kVec], bt[kVec], mu[NGL], B[NGL], E[NGL];
        cl_load_coefc(coefc + n * a.C + int64_t(cv) * kVec, A, bt);
#pragma unroll
        for (int q = 0; q < NGL; ++q) {
            const float4 cg = coefg[n * a.G + g0 + q];
            mu[q] = cg.x; B[q] = cg.y; E[q] = cg.z;
        }
#pragma unroll
        for (int r = 0; r < kClApplyRounds; ++r) {
            const int64_t vox = v0 + int64_t(r) * vps + vo;
            if (vox < v1) {
                const int64_t off = (n * a.S + vox) * a.C + int64_t(cv) * kVec;
                float xv[kVec], gv[kVec], o[kVec];
                Io<TX>::template load8<NT>(x + off, xv);
                Io<TD>::template load8<NT>(dy + off, gv);
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const int q = i / W;
                    const float d = xv[i] - mu[q];
                    const float g = act ? relu_gate(fmaf(d, A[i], bt[i]), gv[i]) : gv[i];
                    float t = fmaf(A[i], g, fmaf(E[q], d, B[q]));
                    if (single) t = t - t;
                    o[i] = t;
                }
                // dx goes out with nontemporal stores, like y (MI355X, bf16, C=32, G=8, step with
                // plain loads at 128^3: 181.9 -> 176.3 us; nontemporal loads at 256^3: 1388 ->
                // 1354 us)
                Io<TX>::template store8<true>(dx + off, o);
            }
        }
    }
}

// ------------------------------------------------------------------ resident path
//
// Groups of whole vectors (C/G a multiple of 8, cvg = C/(8G) vectors per voxel, a power of
// two up to 8) that fit one workgroup are held in registers from the single read to the
// write, as in the NCDHW resident kernels: one launch per direction instead of three. Vector
// w of a group is channel vector w mod cvg of voxel w / cvg; lane t holds vectors t, t + B,
// ... (B a multiple of 64, hence of cvg), so all of a lane's vectors carry the same 8
// channels. The statistics are an exact two-pass over the registers relative to the
// group's first element.

// Element offset of vector w (< S * cvg) of group (n, g).
__device__ __forceinline__ int64_t cl_res_off(const ClArgs& a, int64_t n, int64_t g, int w)
{
    const int64_t s = w >> a.lcvg;
    const int k = w & ((1 << a.lcvg) - 1);
    return (n * a.S + s) * a.C + g * a.Cg + k * kVec;
}

// Forward, one workgroup per group: blockIdx.x = g, blockIdx.y = n. Writes mean, rstd and y.
template <int V, typename TX, typename TY>
__global__ void __launch_bounds__(kResMaxBlock)
cl_res_fwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                  float eps, float* __restrict__ mean_out, float* __restrict__ rstd_out, ClArgs a,
                  TY* __restrict__ y)
{
    __shared__ float s_red[2 * kResMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int vg = int(a.S << a.lcvg);  // vectors per group (<= kResMaxVecs)
    const float fM = float(a.M);        // exact: M <= 8 * kResMaxVecs
    const bool act = a.act != 0;
    const int64_t g = blockIdx.x, n = blockIdx.y, ng = n * a.G + g;
    const float K = cl_group_shift(x, a, n, g);
    float e[V * kVec];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int w = u * blk + tid;
        float v[kVec];
        if (w < vg) {
            Io<TX>::template load8<kNtApply>(x + cl_res_off(a, n, g, w), v);
        } else {
#pragma unroll
            for (int i = 0; i < kVec; ++i) v[i] = K;  // contributes exact zeros below
        }
#pragma unroll
        for (int i = 0; i < kVec; ++i) e[u * kVec + i] = v[i];
    }
    float t[V * kVec];
#pragma unroll
    for (int i = 0; i < V * kVec; ++i) t[i] = e[i] - K;
    const float m = block_allsum2(tree_sum(t), 0.0f, s_red).x / fM;
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const bool ok = u * blk + tid < vg;
#pragma unroll
        for (int i = 0; i < kVec; ++i) t[u * kVec + i] = ok ? (e[u * kVec + i] - K) - m : 0.0f;
    }
    const float2 r = block_allsum2(tree_sum(t), tree_sumsq(t), s_red);
    float var = (r.y - (r.x * r.x) / fM) / fM;
    var = (var < 0.0f) ? 0.0f : var;  // NaN passes through
    const float rstd = 1.0f / __fsqrt_rn(var + eps);
    const float hi = K + m;
    const float lo = (K - hi) + m;
    if (tid == 0) {
        mean_out[ng] = hi;
        rstd_out[ng] = rstd;
    }
    const int64_t c0 = g * a.Cg + (tid & ((1 << a.lcvg) - 1)) * kVec;  // the lane's first channel
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int w = u * blk + tid;
        if (w < vg) {
            float o[kVec];
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                const float scale = (gamma ? gamma[c0 + i] : 1.0f) * rstd;
                const float v = fmaf((e[u * kVec + i] - hi) - lo, scale, beta ? beta[c0 + i] : 0.0f);
                o[i] = act ? relu_f(v) : v;
            }
            Io<TY>::store8(y + cl_res_off(a, n, g, w), o);
        }
    }
}

// Backward, one workgroup per g covering the groups (n, g) of all N samples: vector w of
// the workgroup is vector w mod vg of sample w / vg (vg = S * cvg, a multiple of 64, so
// every wave lies in one sample). Per vector and channel: g (dy, or dy gated by the relu)
// and g*(x - mean); lanes of a wave that share a channel vector add them in the strided
// lane tree (lane i takes lane i + off, off = 32 down to cvg); per (sample, channel) row
// the waves' sums in (vector set, wave) order, then s2 times rstd; per sample c1, c2 over
// the group's channels in order; per channel dgamma, dbeta over the samples in order; then
// dx from the registers as bwd_apply computes it (dx = A*g + (B + E*(x - mean))).
template <int V, typename TX, typename TD>
__global__ void __launch_bounds__(kResMaxBlock)
cl_res_bwd_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ mean,
                  const float* __restrict__ rstd, const float* __restrict__ gamma,
                  const float* __restrict__ beta, ClArgs a, float* __restrict__ dgamma,
                  float* __restrict__ dbeta, TX* __restrict__ dx)
{
    constexpr int kSlot = 2 * kVec;  // per channel vector: 8 sums of g, 8 of g*(x - mean)
    __shared__ float s_part[kResMaxLaneVecs * kResMaxWaves * kClResMaxGroupVecs * kSlot];
    __shared__ float s_r1[kClResMaxRows], s_r2[kClResMaxRows];
    __shared__ float s_b[kResMaxVecs / 64], s_e[kResMaxVecs / 64];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = blk >> 6;
    const int cvg = 1 << a.lcvg, Cg = int(a.Cg), N = int(a.N);
    const int vg = int(a.S << a.lcvg), nvt = N * vg;
    const bool act = a.act != 0;
    const int64_t g = blockIdx.x;
    const int64_t c0 = g * Cg + (tid & (cvg - 1)) * kVec;  // the lane's first channel
    float xs[V * kVec], gs[V * kVec];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int wb = u * blk + wave * 64;  // the wave's first vector
        if (wb < nvt) {                      // whole waves are in or out
            const int nn = int(fdiv(uint32_t(wb), a.div_vg));
            const int64_t off = cl_res_off(a, nn, g, u * blk + tid - nn * vg);
            const int64_t ng = int64_t(nn) * a.G + g;
            float e[kVec], f[kVec], p[kSlot];
            Io<TX>::template load8<kNtBwdApply>(x + off, e);
            Io<TD>::template load8<kNtBwdApply>(dy + off, f);
            const float mu = mean[ng], rs = rstd[ng];
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                const float d = e[i] - mu;
                const float A = rs * (gamma ? gamma[c0 + i] : 1.0f);
                const float q = act ? relu_gate(fmaf(d, A, beta ? beta[c0 + i] : 0.0f), f[i]) : f[i];
                xs[u * kVec + i] = e[i];
                gs[u * kVec + i] = q;
                p[i] = q;
                p[kVec + i] = q * d;
            }
#pragma unroll
            for (int j = 0; j < kSlot; ++j) p[j] = wave_sum_stride(p[j], cvg);
            if (lane < cvg) {
                float* dst = s_part + ((u * kResMaxWaves + wave) * kClResMaxGroupVecs + lane) * kSlot;
#pragma unroll
                for (int j = 0; j < kSlot; ++j) dst[j] = p[j];
            }
        }
    }
    __syncthreads();
    for (int r = tid; r < N * Cg; r += blk) {
        const int nn = r / Cg, ci = r - nn * Cg;
        const int kk = ci / kVec, j = ci - kk * kVec;
        float t1 = 0.0f, t2 = 0.0f;
        for (int u = 0; u < V; ++u) {
            for (int wv = 0; wv < nw; ++wv) {
                const int wb = u * blk + wv * 64;
                if (wb < nvt && int(fdiv(uint32_t(wb), a.div_vg)) == nn) {
                    const float* src = s_part + ((u * kResMaxWaves + wv) * kClResMaxGroupVecs + kk) * kSlot;
                    t1 = t1 + src[j];
                    t2 = t2 + src[kVec + j];
                }
            }
        }
        s_r1[r] = t1;
        s_r2[r] = t2 * rstd[int64_t(nn) * a.G + g];
    }
    __syncthreads();
    for (int nn = tid; nn < N; nn += blk) {
        float t1 = 0.0f, t2 = 0.0f;
        for (int ci = 0; ci < Cg; ++ci) {
            const float gm = gamma ? gamma[g * Cg + ci] : 1.0f;
            t1 = t1 + gm * s_r1[nn * Cg + ci];
            t2 = t2 + gm * s_r2[nn * Cg + ci];
        }
        const float rs = rstd[int64_t(nn) * a.G + g];
        s_b[nn] = -(rs * float(double(t1) / double(a.M)));
        s_e[nn] = -((rs * rs) * float(double(t2) / double(a.M)));
    }
    if (dgamma || dbeta) {
        for (int ci = tid; ci < Cg; ci += blk) {
            float q1 = 0.0f, q2 = 0.0f;
            for (int nn = 0; nn < N; ++nn) {
                q1 = q1 + s_r2[nn * Cg + ci];
                q2 = q2 + s_r1[nn * Cg + ci];
            }
            if (dgamma) dgamma[g * Cg + ci] = q1;
            if (dbeta) dbeta[g * Cg + ci] = q2;
        }
    }
    __syncthreads();
    if (!dx) return;
    const bool single = (a.M == 1);
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int wb = u * blk + wave * 64;
        if (wb < nvt) {
            const int nn = int(fdiv(uint32_t(wb), a.div_vg));
            const int64_t off = cl_res_off(a, nn, g, u * blk + tid - nn * vg);
            const int64_t ng = int64_t(nn) * a.G + g;
            const float mu = mean[ng], rs = rstd[ng], B = s_b[nn], E = s_e[nn];
            float o[kVec];
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                const float d = xs[u * kVec + i] - mu;
                float t = fmaf(rs * (gamma ? gamma[c0 + i] : 1.0f), gs[u * kVec + i], fmaf(E, d, B));
                if (single) t = t - t;
                o[i] = t;
            }
            Io<TX>::store8(dx + off, o);
        }
    }
}

// Calls f with std::integral_constant<int, NGL> for the lane's slot count.
// Calls f with std::bool_constant<NT> for the streamed loads: plain loads (false) when the
// host found that x fits the last-level cache, so that the step's later kernels find x there,
// else nontemporal ones (measured on MI355X, bf16, C=32, G=8, fwd+bwd: 128^3 185.2 -> 181.9 us
// with plain loads, 176.3 with nontemporal dx stores as well; 256^3 1354 -> 1477 us with plain
// loads). The policy moves no bit of any result.
template <typename F>
hipError_t with_cl_policy(const ClArgs& a, F&& f)
{
    if (a.cached) return f(std::bool_constant<false>{});
    return f(std::bool_constant<true>{});
}

template <typename F>
hipError_t with_ngl(int ngl, F&& f)
{
    if (ngl == 1) return f(std::integral_constant<int, 1>{});
    if (ngl == 2) return f(std::integral_constant<int, 2>{});
    if (ngl == 4) return f(std::integral_constant<int, 4>{});
    return f(std::integral_constant<int, 8>{});
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_cl_forward(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                             float* mean, float* rstd, void* y, int ydt, const ClArgs& a,
                             WorkspaceCL ws, hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
      return with_cl_policy(a, [&](auto nt) {
        return with_ngl(a.ngl, [&](auto ng) {
            using TX = decltype(tx);
            constexpr int NGL = decltype(ng)::value;
            constexpr bool NT = decltype(nt)::value;
            hipError_t e = launch(cl_stats_kernel<NGL, TX, NT>, grid_of(a.jobs), dim3(kClBlock), st, cp<TX>(x), a,
                                  ws.part);
            if (e != hipSuccess) return e;
            e = launch(cl_fin_fwd_kernel<TX>, dim3(unsigned(a.N * a.G)), dim3(256), st, cp<TX>(x), gamma, beta,
                       eps, static_cast<const float2*>(ws.part), mean, rstd, a, ws.coefc, ws.coefg);
            if (e != hipSuccess) return e;
            const float2* cc = ws.coefc;
            const float4* cg = ws.coefg;
            if (ydt == kF32)
                return a.act ? launch(cl_apply_kernel<NGL, TX, float, NT, true>, grid_of(a.jobs_a), dim3(kClBlock),
                                      st, cp<TX>(x), mp<float>(y), a, cc, cg)
                             : launch(cl_apply_kernel<NGL, TX, float, NT, false>, grid_of(a.jobs_a), dim3(kClBlock),
                                      st, cp<TX>(x), mp<float>(y), a, cc, cg);
            return a.act ? launch(cl_apply_kernel<NGL, TX, TX, NT, true>, grid_of(a.jobs_a), dim3(kClBlock), st,
                                  cp<TX>(x), mp<TX>(y), a, cc, cg)
                         : launch(cl_apply_kernel<NGL, TX, TX, NT, false>, grid_of(a.jobs_a), dim3(kClBlock), st,
                                  cp<TX>(x), mp<TX>(y), a, cc, cg);
        });
      });
    });
}

hipError_t launch_cl_backward(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                              const float* rstd, const float* gamma, const float* beta, void* dx,
                              float* dgamma, float* dbeta, const ClArgs& a, WorkspaceCL ws,
                              hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
      return with_type(dydt, [&](auto td) {
        return with_cl_policy(a, [&](auto nt) {
            return with_ngl(a.ngl, [&](auto ng) {
                using TX = decltype(tx);
                using TD = decltype(td);
                constexpr int NGL = decltype(ng)::value;
                constexpr bool NT = decltype(nt)::value;
                hipError_t e = a.act
                    ? launch(cl_bwd_reduce_kernel<NGL, true, TX, TD, NT>, grid_of(a.jobs), dim3(kClBlock), st,
                             cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a, ws.part, ws.partg)
                    : launch(cl_bwd_reduce_kernel<NGL, false, TX, TD, NT>, grid_of(a.jobs), dim3(kClBlock), st,
                             cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a, ws.part, ws.partg);
                if (e != hipSuccess) return e;
                const int64_t ngroups = a.N * a.G;
                const int64_t nchan = (dgamma || dbeta) ? a.C : 0;
                e = launch(cl_fin_bwd_kernel, dim3(unsigned(ngroups + nchan)), dim3(256), st, mean, rstd, gamma,
                           beta, static_cast<const float2*>(ws.part), static_cast<const float2*>(ws.partg), a,
                           ngroups, nchan, ws.coefc, ws.coefg, dgamma, dbeta);
                if (e != hipSuccess || !dx) return e;
                return launch(cl_bwd_apply_kernel<NGL, TX, TD, NT>, grid_of(a.jobs_a), dim3(kClBlock), st,
                              cp<TD>(dy), cp<TX>(x), a, static_cast<const float2*>(ws.coefc),
                              static_cast<const float4*>(ws.coefg), mp<TX>(dx));
            });
        });
      });
    });
}

// The plan keeps a resident workgroup within 1024 vectors, one a lane (vecs == 1).
hipError_t launch_cl_res_forward(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                                 float* mean, float* rstd, void* y, int ydt, const ClArgs& a, hipStream_t st,
                                 int block, int vecs)
{
    if (vecs != 1) return hipErrorInvalidValue;
    const dim3 grid(unsigned(a.G), unsigned(a.N)), blk{unsigned(block)};
    return with_type(xdt, [&](auto tx) {
        using TX = decltype(tx);
        if (ydt == kF32)
            return launch(cl_res_fwd_kernel<1, TX, float>, grid, blk, st, cp<TX>(x), gamma, beta, eps, mean, rstd,
                          a, mp<float>(y));
        return launch(cl_res_fwd_kernel<1, TX, TX>, grid, blk, st, cp<TX>(x), gamma, beta, eps, mean, rstd, a,
                      mp<TX>(y));
    });
}

hipError_t launch_cl_res_backward(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                                  const float* rstd, const float* gamma, const float* beta, void* dx,
                                  float* dgamma, float* dbeta, const ClArgs& a, hipStream_t st, int block,
                                  int vecs)
{
    if (vecs != 1) return hipErrorInvalidValue;
    return with_type(xdt, [&](auto tx) {
        return with_type(dydt, [&](auto td) {
            using TX = decltype(tx);
            using TD = decltype(td);
            return launch(cl_res_bwd_kernel<1, TX, TD>, dim3(unsigned(a.G)), dim3(unsigned(block)), st,
                          cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a, dgamma, dbeta, mp<TX>(dx));
        });
    });
}

}  // namespace gn
