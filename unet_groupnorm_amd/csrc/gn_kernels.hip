// gn_kernels.hip -- GroupNorm forward/backward kernels for gfx950 (MI355X, CDNA4).
//
// Four kernels, two per direction ("Optimize GroupNorm", LBANN/ScaFFold pull 93,
// paragraph folding seven launches into four):
//   stats_kernel       per-job (mean, M2) of x                       [read x]
//   apply_kernel       fixed-order merge -> mean/rstd, y = affine    [read x, write y]
//   bwd_reduce_kernel  per-job (sum dy, sum dy*xhat)                  [read x, dy]
//   bwd_apply_kernel   fixed-order merge -> c1, c2, dgamma, dbeta; dx [read x, dy, write dx]
//
// A job is a contiguous run of one row (row = n*C + c) given by the plan. Lane t of a
// workgroup owns the 8-element vectors t, t + B, t + 2B, ... of its job (B = block
// size, vectors counted on the global 8-element grid), holding kStepVecs of them per
// step. The mapping is defined on elements, never on bytes, so the reduction order is
// the same for fp32 and bf16 data.
//
// Statistics are fp32 throughout. Each lane takes a corrected two-pass over its
// register tile (tile mean, then sum of squared deviations minus the squared sum of
// deviations over n), merges tiles with Chan's parallel formula, then lanes merge in a
// fixed shuffle tree and waves in a fixed order through LDS ("Optimize GroupNorm",
// paragraph introducing the NDHWC kernel: corrected two-pass per tile combined by Chan's
// formula, register-only reductions, fixed order, no float atomics). No atomics are
// used anywhere, so every result is bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "gn_launch.hpp"

namespace gn {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element access

// bf16 is stored as the upper 16 bits of an fp32: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Narrowing fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

template <typename T> struct Io;

template <> struct Io<uint16_t> {  // bf16 storage
    static __device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8])
    {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
        v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
        v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    }
    static __device__ __forceinline__ float load1(const uint16_t* p)
    {
        return __uint_as_float(uint32_t(*p) << 16);
    }
    static __device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8])
    {
        uint4 u;
        u.x = pack_bf16(v[0], v[1]);
        u.y = pack_bf16(v[2], v[3]);
        u.z = pack_bf16(v[4], v[5]);
        u.w = pack_bf16(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = u;
    }
    static __device__ __forceinline__ void store1(uint16_t* p, float v)
    {
        *p = uint16_t(pack_bf16(v, 0.0f) & 0xffffu);
    }
};

template <> struct Io<float> {
    static __device__ __forceinline__ void load8(const float* p, float (&v)[8])
    {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
    static __device__ __forceinline__ void store8(float* p, const float (&v)[8])
    {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};

// ------------------------------------------------------------------ job geometry

struct Job {
    int64_t row, k;   // row = n*C + c, chunk index within the row
    int64_t lo, hi;   // global element range [lo, hi)
    int64_t v0;       // first vector (floor(lo / 8))
    int64_t vf0, vf1; // full vectors are [vf0, vf1)
    int64_t nvec;     // vectors touched: [v0, v0 + nvec)
};

__device__ __forceinline__ Job job_at(const KArgs& a, int64_t j)
{
    Job b;
    b.row = j / a.K;
    b.k = j - b.row * a.K;
    const int64_t base = b.row * a.S;
    const int64_t end = (b.k + 1) * a.chunk;
    b.lo = base + b.k * a.chunk;
    b.hi = base + (end < a.S ? end : a.S);
    b.v0 = b.lo / kVec;
    b.vf0 = (b.lo + kVec - 1) / kVec;
    b.vf1 = b.hi / kVec;
    b.nvec = (b.hi + kVec - 1) / kVec - b.v0;
    return b;
}

// Element count of job j (the plan fixes it; it is never stored).
__device__ __forceinline__ int64_t job_count(const KArgs& a, int64_t k)
{
    const int64_t end = (k + 1) * a.chunk;
    return (end < a.S ? end : a.S) - k * a.chunk;
}

// ------------------------------------------------------------------ Chan merge

template <typename CT>
struct Moments {
    CT n;
    float m, M2;
};

// a <- a (+) b with Chan's parallel formula. Empty operands are skipped, so a merge
// never mixes a zero count into the mean. With equal means (a constant group) the mean
// is untouched and M2 stays exactly zero. An infinite mean (a part holding +-Inf) stays
// what the sum of the parts makes it (+-Inf, or NaN for opposite signs) instead of the
// NaN that Inf - Inf would give; its M2 is already NaN.
template <typename CT>
__device__ __forceinline__ void chan_merge(Moments<CT>& a, CT nb, float mb, float M2b)
{
    if (nb == 0) return;
    if (a.n == 0) {
        a.n = nb; a.m = mb; a.M2 = M2b;
        return;
    }
    const CT n = a.n + nb;
    const float w = float(nb) / float(n);
    const float d = mb - a.m;
    const bool inf = __builtin_isinf(a.m) || __builtin_isinf(mb);
    a.m = inf ? a.m + mb : fmaf(d, w, a.m);
    a.M2 = (a.M2 + M2b) + (d * d) * (float(a.n) * w);
    a.n = n;
}

// Lane 0 ends up with the merge of all 64 lanes, combined in a fixed tree: lane i takes
// lane i + off for off = 32, 16, ..., 1 (left operand always the lower lane).
template <typename CT>
__device__ __forceinline__ void wave_merge(Moments<CT>& a)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const CT nb = __shfl_down(a.n, off);
        const float mb = __shfl_down(a.m, off);
        const float Mb = __shfl_down(a.M2, off);
        chan_merge(a, nb, mb, Mb);
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_down(v, off);
    return v;
}

// Balanced pairwise sum of 2^k values (pairs i, i + half). A constant input is summed
// exactly: every addition doubles a value.
template <int N>
__device__ __forceinline__ float tree_sum(float (&t)[N])
{
#pragma unroll
    for (int h = N / 2; h >= 1; h >>= 1) {
#pragma unroll
        for (int i = 0; i < h; ++i) t[i] = t[i] + t[i + h];
    }
    return t[0];
}

constexpr int kTile = kVec * kStepVecs;  // elements per lane per step (32)

// Corrected two-pass over a full register tile of values shifted by the group's shift K:
// t = v - K, m = mean(t), M2 = sum d^2 - (sum d)^2 / n with d = t - m. The balanced sum
// makes m exactly 0 for a constant tile equal to K.
__device__ __forceinline__ void tile_moments_full(const float (&v)[kTile], float K, float& m, float& M2)
{
    float t[kTile], u[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        t[i] = v[i] - K;
        u[i] = t[i];
    }
    m = tree_sum(u) * (1.0f / kTile);
    float d[kTile], q[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        d[i] = t[i] - m;
        q[i] = d[i] * d[i];
    }
    const float sd = tree_sum(d);
    const float sq = tree_sum(q);
    M2 = sq - (sd * sd) * (1.0f / kTile);
}

// Same over a tile with a validity mask (job edges); invalid elements contribute nothing.
__device__ __forceinline__ void tile_moments_masked(const float (&v)[kTile], float K, uint32_t valid,
                                                    uint32_t cnt, float& m, float& M2)
{
    float t[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) t[i] = ((valid >> i) & 1u) ? v[i] - K : 0.0f;
    const float fc = float(cnt);
    float u[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) u[i] = t[i];
    m = tree_sum(u) / fc;
    float d[kTile], q[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        d[i] = ((valid >> i) & 1u) ? t[i] - m : 0.0f;
        q[i] = d[i] * d[i];
    }
    const float sd = tree_sum(d);
    const float sq = tree_sum(q);
    M2 = sq - (sd * sd) / fc;
}

// The shift of group (n, g): its first element, or 0 if that is not finite. Every
// statistic of the group is accumulated relative to it, so that means stay small next to
// the spread even when |mean| >> sigma (fp32 resolution of a mean near 1e5 would
// otherwise be 1e-2 of a unit sigma), and a constant group has exactly zero deviations.
template <typename T>
__device__ __forceinline__ float group_shift(const T* __restrict__ x, const KArgs& a, int64_t n, int64_t g)
{
    const float k = Io<T>::load1(x + (n * a.C + g * a.Cg) * a.S);
    return __builtin_isfinite(k) ? k : 0.0f;
}

// Loads the lane's kStepVecs vectors of one step with per-element validity. Vectors that
// are wholly inside the job use one vector load; edge vectors are loaded element-wise.
template <typename T>
__device__ __forceinline__ uint32_t load_step_masked(const T* __restrict__ p, const Job& jb,
                                                     int64_t sv0, int blk, int tid,
                                                     float (&v)[kTile])
{
    uint32_t valid = 0;
#pragma unroll
    for (int u = 0; u < kStepVecs; ++u) {
        const int64_t vi = sv0 + int64_t(u) * blk + tid;
        float e[kVec];
        if (vi >= jb.vf0 && vi < jb.vf1) {
            Io<T>::load8(p + vi * kVec, e);
            valid |= 0xffu << (u * kVec);
        } else {
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                const int64_t gi = vi * kVec + i;
                const bool ok = gi >= jb.lo && gi < jb.hi;
                e[i] = ok ? Io<T>::load1(p + gi) : 0.0f;
                valid |= uint32_t(ok) << (u * kVec + i);
            }
        }
#pragma unroll
        for (int i = 0; i < kVec; ++i) v[u * kVec + i] = e[i];
    }
    return valid;
}

template <typename T>
__device__ __forceinline__ void load_step_full(const T* __restrict__ p, int64_t sv0, int blk,
                                               int tid, float (&v)[kTile])
{
#pragma unroll
    for (int u = 0; u < kStepVecs; ++u) {
        float e[kVec];
        Io<T>::load8(p + (sv0 + int64_t(u) * blk + tid) * kVec, e);
#pragma unroll
        for (int i = 0; i < kVec; ++i) v[u * kVec + i] = e[i];
    }
}

// Whole workgroup step inside the full-vector range (uniform across the workgroup).
__device__ __forceinline__ bool step_is_full(const Job& jb, int64_t sv0, int64_t stepv)
{
    return sv0 >= jb.vf0 && sv0 + stepv <= jb.vf1;
}

constexpr int kMaxWaves = 4;

// Merges the per-wave moments (lane 0 of each wave) in wave order; result valid in thread 0.
template <typename CT>
__device__ __forceinline__ Moments<CT> block_merge(Moments<CT> a, CT* s_n, float* s_m, float* s_M)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    wave_merge(a);
    if (lane == 0) { s_n[wave] = a.n; s_m[wave] = a.m; s_M[wave] = a.M2; }
    __syncthreads();
    Moments<CT> r = {0, 0.0f, 0.0f};
    if (threadIdx.x == 0) {
        r.n = s_n[0]; r.m = s_m[0]; r.M2 = s_M[0];
        for (int w = 1; w < nw; ++w) chan_merge(r, s_n[w], s_m[w], s_M[w]);
    }
    __syncthreads();
    return r;
}

// Sums (lane 0 of each wave) in wave order; result valid in thread 0.
__device__ __forceinline__ float2 block_sum2(float a, float b, float* s_a, float* s_b)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) { s_a[wave] = a; s_b[wave] = b; }
    __syncthreads();
    float2 r = make_float2(0.0f, 0.0f);
    if (threadIdx.x == 0) {
        r.x = s_a[0]; r.y = s_b[0];
        for (int w = 1; w < nw; ++w) { r.x = r.x + s_a[w]; r.y = r.y + s_b[w]; }
    }
    __syncthreads();
    return r;
}

// ------------------------------------------------------------------ forward

template <typename TX>
__global__ void __launch_bounds__(256)
stats_kernel(const TX* __restrict__ x, KArgs a, float2* __restrict__ part)
{
    __shared__ uint32_t s_n[kMaxWaves];
    __shared__ float s_m[kMaxWaves], s_M[kMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;

    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const Job jb = job_at(a, j);
        const int64_t n = jb.row / a.C, g = (jb.row - n * a.C) / a.Cg;
        const float K = group_shift(x, a, n, g);
        Moments<uint32_t> acc = {0u, 0.0f, 0.0f};
        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
            float v[kTile];
            float m, M2;
            if (step_is_full(jb, sv0, stepv)) {
                load_step_full(x, sv0, blk, tid, v);
                tile_moments_full(v, K, m, M2);
                chan_merge(acc, uint32_t(kTile), m, M2);
            } else {
                const uint32_t valid = load_step_masked(x, jb, sv0, blk, tid, v);
                if (valid) {
                    const uint32_t cnt = __builtin_popcount(valid);
                    tile_moments_masked(v, K, valid, cnt, m, M2);
                    chan_merge(acc, cnt, m, M2);
                }
            }
        }
        const Moments<uint32_t> r = block_merge(acc, s_n, s_m, s_M);
        if (tid == 0) part[j] = make_float2(r.m, r.M2);
    }
}

// Fixed-order merge of the P partials of group (n, g) into mean and rstd, broadcast
// through LDS to the whole workgroup. Every workgroup that needs the group runs the same
// merge on the same data and so obtains bitwise the same values.
__device__ __forceinline__ void finalize_stats(const float2* __restrict__ part, const KArgs& a,
                                               int64_t n, int64_t g, float eps,
                                               float* s_stat, uint64_t* s_n, float* s_m, float* s_M)
{
    const int64_t pbase = (n * a.C + g * a.Cg) * a.K;
    Moments<uint64_t> acc = {0ull, 0.0f, 0.0f};
    for (int64_t j = threadIdx.x; j < a.P; j += blockDim.x) {
        const float2 pm = part[pbase + j];
        chan_merge(acc, uint64_t(job_count(a, j % a.K)), pm.x, pm.y);
    }
    const Moments<uint64_t> r = block_merge(acc, s_n, s_m, s_M);
    if (threadIdx.x == 0) {
        float var = float(double(r.M2) / double(a.M));
        var = (var < 0.0f) ? 0.0f : var;  // rounding can leave a tiny negative; NaN passes through
        s_stat[0] = r.m;                  // mean relative to the group's shift
        s_stat[1] = 1.0f / __fsqrt_rn(var + eps);
    }
    __syncthreads();
}

template <typename TX, typename TY>
__global__ void __launch_bounds__(256)
apply_kernel(const TX* __restrict__ x, const float* __restrict__ gamma,
             const float* __restrict__ beta, const float2* __restrict__ part,
             TY* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out,
             KArgs a, float eps)
{
    __shared__ uint64_t s_n[kMaxWaves];
    __shared__ float s_m[kMaxWaves], s_M[kMaxWaves];
    __shared__ float s_stat[2];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;
    int64_t cached = -1;

    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const Job jb = job_at(a, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, g = c / a.Cg, ng = n * a.G + g;
        if (ng != cached) {
            finalize_stats(part, a, n, g, eps, s_stat, s_n, s_m, s_M);
            cached = ng;
        }
        // The mean as an unevaluated sum hi + lo: hi is the fp32 mean that is published,
        // lo what rounding it left out. x - mean is taken as (x - hi) - lo, which is exact
        // in its first step whenever x is close to the mean.
        const float K = group_shift(x, a, n, g);
        const float rel = s_stat[0], rstd = s_stat[1];  // mean relative to K
        const float mu = K + rel;
        const float mu_lo = (K - mu) + rel;
        // The group's first job publishes the statistics.
        if (tid == 0 && jb.k == 0 && c == g * a.Cg) {
            mean_out[ng] = mu;
            rstd_out[ng] = rstd;
        }
        const float scale = (gamma ? gamma[c] : 1.0f) * rstd;
        const float shift = beta ? beta[c] : 0.0f;

        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
            if (step_is_full(jb, sv0, stepv)) {
                float v[kTile];
                load_step_full(x, sv0, blk, tid, v);
#pragma unroll
                for (int u = 0; u < kStepVecs; ++u) {
                    float o[kVec];
#pragma unroll
                    for (int i = 0; i < kVec; ++i) o[i] = fmaf((v[u * kVec + i] - mu) - mu_lo, scale, shift);
                    Io<TY>::store8(y + (sv0 + int64_t(u) * blk + tid) * kVec, o);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kStepVecs; ++u) {
                    const int64_t vi = sv0 + int64_t(u) * blk + tid;
                    if (vi >= jb.vf0 && vi < jb.vf1) {
                        float e[kVec], o[kVec];
                        Io<TX>::load8(x + vi * kVec, e);
#pragma unroll
                        for (int i = 0; i < kVec; ++i) o[i] = fmaf((e[i] - mu) - mu_lo, scale, shift);
                        Io<TY>::store8(y + vi * kVec, o);
                    } else {
                        for (int i = 0; i < kVec; ++i) {
                            const int64_t gi = vi * kVec + i;
                            if (gi >= jb.lo && gi < jb.hi)
                                Io<TY>::store1(y + gi, fmaf((Io<TX>::load1(x + gi) - mu) - mu_lo, scale, shift));
                        }
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ backward

template <typename TX, typename TD>
__global__ void __launch_bounds__(256)
bwd_reduce_kernel(const TD* __restrict__ dy, const TX* __restrict__ x,
                  const float* __restrict__ mean, const float* __restrict__ rstd,
                  KArgs a, float2* __restrict__ part)
{
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;

    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const Job jb = job_at(a, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, ng = n * a.G + c / a.Cg;
        const float mu = mean[ng];
        float s1 = 0.0f, s2 = 0.0f;  // sum dy, sum dy * (x - mu)
        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
            float xv[kTile], gv[kTile];
            if (step_is_full(jb, sv0, stepv)) {
                load_step_full(x, sv0, blk, tid, xv);
                load_step_full(dy, sv0, blk, tid, gv);
            } else {
                const uint32_t valid = load_step_masked(x, jb, sv0, blk, tid, xv);
                load_step_masked(dy, jb, sv0, blk, tid, gv);  // same mask: zeros outside
#pragma unroll
                for (int i = 0; i < kTile; ++i) xv[i] = ((valid >> i) & 1u) ? xv[i] : mu;
            }
            float p[kTile];
#pragma unroll
            for (int i = 0; i < kTile; ++i) p[i] = gv[i] * (xv[i] - mu);
            s1 = s1 + tree_sum(gv);
            s2 = s2 + tree_sum(p);
        }
        const float2 r = block_sum2(s1, s2, s_a, s_b);
        if (tid == 0) part[j] = make_float2(r.x, r.y * rstd[ng]);
    }
}

template <typename TX, typename TD>
__global__ void __launch_bounds__(256)
bwd_apply_kernel(const TD* __restrict__ dy, const TX* __restrict__ x,
                 const float* __restrict__ mean, const float* __restrict__ rstd,
                 const float* __restrict__ gamma, const float2* __restrict__ part, KArgs a,
                 TX* __restrict__ dx, float* __restrict__ dgamma, float* __restrict__ dbeta)
{
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    __shared__ float s_coef[2];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;
    int64_t cached = -1;

    for (int64_t j = blockIdx.x; j < a.jobs; j += gridDim.x) {
        const Job jb = job_at(a, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, g = c / a.Cg, ng = n * a.G + g;

        // dgamma_c, dbeta_c: the job (n = 0, k = 0) of channel c sums the N*K partials of
        // the channel, n-major then k, in a fixed tree.
        if ((dgamma || dbeta) && n == 0 && jb.k == 0) {
            float sa = 0.0f, sb = 0.0f;
            for (int64_t i = tid; i < a.N * a.K; i += blk) {
                const int64_t nn = i / a.K, kk = i - nn * a.K;
                const float2 pp = part[(nn * a.C + c) * a.K + kk];
                sa = sa + pp.y;
                sb = sb + pp.x;
            }
            const float2 r = block_sum2(sa, sb, s_a, s_b);
            if (tid == 0) {
                if (dgamma) dgamma[c] = r.x;
                if (dbeta) dbeta[c] = r.y;
            }
        }
        if (!dx) continue;

        if (ng != cached) {
            // c1 = (1/M) sum_{c in g} gamma_c s1[n,c], c2 likewise with s2, over the
            // group's P partials in a fixed order.
            const int64_t pbase = (n * a.C + g * a.Cg) * a.K;
            float t1 = 0.0f, t2 = 0.0f;
            for (int64_t i = tid; i < a.P; i += blk) {
                const float2 pp = part[pbase + i];
                const float gm = gamma ? gamma[g * a.Cg + i / a.K] : 1.0f;
                t1 = t1 + gm * pp.x;
                t2 = t2 + gm * pp.y;
            }
            const float2 r = block_sum2(t1, t2, s_a, s_b);
            if (tid == 0) {
                s_coef[0] = float(double(r.x) / double(a.M));
                s_coef[1] = float(double(r.y) / double(a.M));
            }
            __syncthreads();
            cached = ng;
        }
        const float mu = mean[ng], rs = rstd[ng];
        const float gm = gamma ? gamma[c] : 1.0f;
        // dx = rstd * (gamma*dy - c1 - xhat*c2) = A*dy + (B + E*(x - mu))
        const float A = rs * gm;
        const float B = -(rs * s_coef[0]);
        const float E = -((rs * rs) * s_coef[1]);
        // A single-element group is answered as t - t: +0 for finite t, NaN otherwise.
        const bool single = (a.M == 1);

        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
            if (step_is_full(jb, sv0, stepv)) {
                float xv[kTile], gv[kTile];
                load_step_full(x, sv0, blk, tid, xv);
                load_step_full(dy, sv0, blk, tid, gv);
#pragma unroll
                for (int u = 0; u < kStepVecs; ++u) {
                    float o[kVec];
#pragma unroll
                    for (int i = 0; i < kVec; ++i) {
                        const int e = u * kVec + i;
                        float t = fmaf(A, gv[e], fmaf(E, xv[e] - mu, B));
                        if (single) t = t - t;
                        o[i] = t;
                    }
                    Io<TX>::store8(dx + (sv0 + int64_t(u) * blk + tid) * kVec, o);
                }
            } else {
                for (int u = 0; u < kStepVecs; ++u) {
                    const int64_t vi = sv0 + int64_t(u) * blk + tid;
                    for (int i = 0; i < kVec; ++i) {
                        const int64_t gi = vi * kVec + i;
                        if (gi >= jb.lo && gi < jb.hi) {
                            float t = fmaf(A, Io<TD>::load1(dy + gi),
                                           fmaf(E, Io<TX>::load1(x + gi) - mu, B));
                            if (single) t = t - t;
                            Io<TX>::store1(dx + gi, t);
                        }
                    }
                }
            }
        }
    }
}

// Launches kernel k and returns the runtime's status for this launch alone.
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A... args)
{
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    std::tuple<P...> t(args...);
    void* ptrs[sizeof...(P)];
    std::apply([&](auto&... e) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&e)), ...);
    }, t);
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, st);
}

template <typename T> const T* cp(const void* p) { return static_cast<const T*>(p); }
template <typename T> T* mp(void* p) { return static_cast<T*>(p); }

int64_t grid_for(const KArgs& a) { return a.jobs < kMaxGrid ? a.jobs : kMaxGrid; }

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_stats(const void* x, int xdt, const KArgs& a, float2* part, hipStream_t st)
{
    const dim3 grid(unsigned(grid_for(a))), block(unsigned(a.block));
    if (xdt == kBF16)
        return launch(stats_kernel<uint16_t>, grid, block, st, cp<uint16_t>(x), a, part);
    else
        return launch(stats_kernel<float>, grid, block, st, cp<float>(x), a, part);
}

hipError_t launch_apply(const void* x, int xdt, const float* gamma, const float* beta,
                        const float2* part, void* y, int ydt, float* mean, float* rstd,
                        const KArgs& a, float eps, hipStream_t st)
{
    const dim3 grid(unsigned(grid_for(a))), block(unsigned(a.block));
    if (xdt == kBF16 && ydt == kBF16)
        return launch(apply_kernel<uint16_t, uint16_t>, grid, block, st,
                           cp<uint16_t>(x), gamma, beta, part, mp<uint16_t>(y), mean, rstd, a, eps);
    else if (xdt == kBF16)
        return launch(apply_kernel<uint16_t, float>, grid, block, st,
                           cp<uint16_t>(x), gamma, beta, part, mp<float>(y), mean, rstd, a, eps);
    else
        return launch(apply_kernel<float, float>, grid, block, st,
                           cp<float>(x), gamma, beta, part, mp<float>(y), mean, rstd, a, eps);
}

hipError_t launch_bwd_reduce(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                             const float* rstd, const KArgs& a, float2* part, hipStream_t st)
{
    const dim3 grid(unsigned(grid_for(a))), block(unsigned(a.block));
    if (xdt == kBF16 && dydt == kBF16)
        return launch(bwd_reduce_kernel<uint16_t, uint16_t>, grid, block, st,
                           cp<uint16_t>(dy), cp<uint16_t>(x), mean, rstd, a, part);
    else if (xdt == kBF16)
        return launch(bwd_reduce_kernel<uint16_t, float>, grid, block, st,
                           cp<float>(dy), cp<uint16_t>(x), mean, rstd, a, part);
    else if (dydt == kBF16)
        return launch(bwd_reduce_kernel<float, uint16_t>, grid, block, st,
                           cp<uint16_t>(dy), cp<float>(x), mean, rstd, a, part);
    else
        return launch(bwd_reduce_kernel<float, float>, grid, block, st,
                           cp<float>(dy), cp<float>(x), mean, rstd, a, part);
}

hipError_t launch_bwd_apply(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                            const float* rstd, const float* gamma, const float2* part,
                            const KArgs& a, void* dx, float* dgamma, float* dbeta, hipStream_t st)
{
    const dim3 grid(unsigned(grid_for(a))), block(unsigned(a.block));
    if (xdt == kBF16 && dydt == kBF16)
        return launch(bwd_apply_kernel<uint16_t, uint16_t>, grid, block, st,
                           cp<uint16_t>(dy), cp<uint16_t>(x), mean, rstd, gamma, part, a,
                           mp<uint16_t>(dx), dgamma, dbeta);
    else if (xdt == kBF16)
        return launch(bwd_apply_kernel<uint16_t, float>, grid, block, st,
                           cp<float>(dy), cp<uint16_t>(x), mean, rstd, gamma, part, a,
                           mp<uint16_t>(dx), dgamma, dbeta);
    else if (dydt == kBF16)
        return launch(bwd_apply_kernel<float, uint16_t>, grid, block, st,
                           cp<uint16_t>(dy), cp<float>(x), mean, rstd, gamma, part, a,
                           mp<float>(dx), dgamma, dbeta);
    else
        return launch(bwd_apply_kernel<float, float>, grid, block, st,
                           cp<float>(dy), cp<float>(x), mean, rstd, gamma, part, a,
                           mp<float>(dx), dgamma, dbeta);
}

}  // namespace gn
