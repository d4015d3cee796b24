// gn_kernels.hip -- GroupNorm forward/backward kernels for gfx950 (MI355X, CDNA4).
//
// Three kernel sets. The two-pass set, two kernels per direction, used by gn_forward and
// gn_backward:
//   stats_kernel          per reduction job: (mean, M2) of x                  [read x]
//   apply_fin_kernel      per folded job: the group's finalize, then
//                         y = (x - mean) * gamma*rstd + beta                 [read x, write y]
//   bwd_reduce_kernel     per reduction job: sum dy, sum dy*xhat              [read x, dy]
//   bwd_apply_fin_kernel  per folded job: the group's c1, c2, then dx; per
//                         channel (one job each): dgamma, dbeta              [read x, dy, write dx]
// The split-phase entry points run the finalize as a kernel of its own, so that the
// statistics exist between the two calls, and stream with one-step jobs:
//   fin_fwd_kernel        per group: fixed-order merge -> mean, rstd, and per-row
//                         normalize coefficients                             [tiny]
//   apply_kernel          per streaming job: y from the coefficients          [read x, write y]
//   fin_bwd_kernel        per group: c1, c2 -> per-row dx coefficients; per
//                         channel: dgamma, dbeta                             [tiny]
//   bwd_apply_kernel      per streaming job: dx                              [read x, dy, write dx]
// Both run the same merge code in the same order, so their results agree bitwise. The
// resident set for small groups, one kernel per direction (see "resident path"):
//   res_fwd_kernel        per group: statistics and y from registers          [read x, write y]
//   res_bwd_kernel        per g over all samples: sums, dgamma/dbeta, dx      [read x, dy, write dx]
//
// The pages fold the finalize into the elementwise kernels ("Optimize GroupNorm",
// LBANN/ScaFFold pull 93, paragraph folding seven launches into four) and cap the
// elementwise grid so that the redundant partial reads stay small. Here the folded jobs
// are kFoldChunk elements (16 KiB of bf16 in, 16 KiB out), so a group's P partials (2 KiB
// at 128^3, C=32, G=8) are re-read from L2 by a few hundred workgroups instead of a few
// thousand one-step ones; on MI355X that removes the finalize launch (about 5 us each
// way) for about 1 us of merge latency per workgroup, most of it behind the workgroup's
// first loads.
//
// A reduction job is a contiguous run of one row (row = n*C + c). Lane t of a workgroup
// owns the 8-element vectors t, t + B, t + 2B, ... of its job (B = block size, vectors
// counted on the global 8-element grid), holding kStepVecs of them per step. The mapping
// is defined on elements, never on bytes, so the reduction order is the same for fp32
// and bf16 data.
//
// Statistics are fp32 throughout. Each lane takes a corrected two-pass over its register
// tile (tile mean, then sum of squared deviations minus the squared sum of deviations over
// n), merges tiles with Chan's parallel formula, then lanes merge in a fixed shuffle tree
// and waves in a fixed order through LDS ("Optimize GroupNorm", paragraph introducing the
// NDHWC kernel, which takes the same route: per-tile two-pass moments, Chan merges, sums
// kept in registers and combined in one order, no floating-point atomics). No atomics are
// used anywhere, so every result is bitwise reproducible run to run.
#include "gn_device.hpp"

namespace gn {

namespace {

// ------------------------------------------------------------------ job geometry

struct Job {
    int64_t row, k;   // row = n*C + c, job index within the row
    int64_t lo, hi;   // global element range [lo, hi)
    int64_t v0;       // first vector (floor(lo / 8))
    int64_t vf0, vf1; // full vectors are [vf0, vf1)
    int64_t nvec;     // vectors touched: [v0, v0 + nvec)
};

__device__ __forceinline__ Job job_at(int64_t S, int64_t chunk, int64_t K, int64_t j)
{
    Job b;
    b.row = j / K;
    b.k = j - b.row * K;
    const int64_t base = b.row * S;
    const int64_t end = (b.k + 1) * chunk;
    b.lo = base + b.k * chunk;
    b.hi = base + (end < S ? end : S);
    b.v0 = b.lo / kVec;
    b.vf0 = (b.lo + kVec - 1) / kVec;
    b.vf1 = b.hi / kVec;
    b.nvec = (b.hi + kVec - 1) / kVec - b.v0;
    return b;
}

// Element count of reduction job k of a row (the plan fixes it; it is never stored).
__device__ __forceinline__ int64_t job_count(const KArgs& a, int64_t k)
{
    const int64_t end = (k + 1) * a.chunk;
    return (end < a.S ? end : a.S) - k * a.chunk;
}

constexpr int kTile = kVec * kStepVecs;  // elements per lane per step (32)

// Corrected two-pass over a full register tile of values shifted by the group's shift K:
// t = v - K, m = mean(t), M2 = sum d^2 - (sum d)^2 / n with d = t - m. The balanced sum
// makes m exactly 0 for a constant tile equal to K.
__device__ __forceinline__ void tile_moments_full(float (&t)[kTile], float& m, float& M2)
{
    m = tree_sum(t) * (1.0f / kTile);
#pragma unroll
    for (int i = 0; i < kTile; ++i) t[i] = t[i] - m;
    const float sd = tree_sum(t);
    const float sq = tree_sumsq(t);
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
    m = tree_sum(t) / fc;
#pragma unroll
    for (int i = 0; i < kTile; ++i) t[i] = ((valid >> i) & 1u) ? t[i] - m : 0.0f;
    const float sd = tree_sum(t);
    const float sq = tree_sumsq(t);
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
template <bool NT, typename T>
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
            Io<T>::template load8<NT>(p + vi * kVec, e);
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


// ------------------------------------------------------------------ forward

// Dword 3 of a raw buffer resource (gfx9 layout): data format 32 bits, no swizzle, no
// index stride. Raw loads ignore the format, but a zero format would make them return 0.
constexpr int kBufWord3 = 0x00020000;

// The lane's V raw vectors of one full step, plain global loads. Under the nontemporal
// policy (inputs that outgrow the last-level cache) the wave raises its issue priority while
// it requests the step, so that a step's loads leave together ahead of other waves' arithmetic
// on the SIMD. Measured on MI355X (256^3, C=32, G=8, bf16, interleaved A/B, same bits): 1318.6
// -> 1311.9 us a step (backward sums 312.1 -> 308.9 us); given to the cached loads of
// smaller inputs as well, the same hint cost the 128^3 step 2.7 us, so they go without it.
template <bool NT, int V, typename T>
__device__ __forceinline__ void load_raw_step_global(const T* __restrict__ p, int64_t sv0, int blk, int tid,
                                                     typename Io<T>::Raw (&r)[V])
{
    if constexpr (NT) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < V; ++u) r[u] = Io<T>::template load_raw<NT>(p + (sv0 + int64_t(u) * blk + tid) * kVec);
    if constexpr (NT) __builtin_amdgcn_s_setprio(0);
}

// The same vectors. Plain 16-byte vectors (bf16, fp16) are read through a buffer resource
// that spans just this step: the step's start is the same for every lane, so it goes into
// the resource's scalar base and each load carries a 32-bit lane offset instead of a 64-bit
// vector address (fewer VALU operations a vector), and the resource's range check keeps
// every load inside the step. Same addresses, same bits. Measured on MI355X (bf16, C=32,
// G=8, interleaved A/B): 128^3 168.2 -> 167.1 us a step (normalize 45.2 -> 44.5, dx 64.5 ->
// 63.8), 64^3 56.0 -> 54.8, 32^3 23.4 -> 24.1. The backward sums read x this way and dy with
// load_raw_step_global: with both through resources they lost 2.3 us at 128^3; with x alone
// the resident-input step is unchanged (166.8 against 167.0 us) and the sums gain 3-5 us
// when x and dy come from HBM (after a 512 MiB read 49.6 -> 44.6 us, with x and dy just
// rewritten 58.8 -> 55.8).
template <bool NT, int V, typename T>
__device__ __forceinline__ void load_raw_step(const T* __restrict__ p, int64_t sv0, int blk, int tid,
                                              typename Io<T>::Raw (&r)[V])
{
    if constexpr (!NT && sizeof(typename Io<T>::Raw) == 16) {
        // readfirstlane returns a signed int: both words are kept unsigned, so that a low word
        // with bit 31 set is not sign-extended over the high word.
        const uint64_t a = reinterpret_cast<uint64_t>(p + sv0 * kVec);
        const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a)));
        const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32)));
        const uint64_t base = (uint64_t(hi) << 32) | uint64_t(lo);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, V * blk * 16, kBufWord3);
#pragma unroll
        for (int u = 0; u < V; ++u) r[u].u = __builtin_amdgcn_raw_buffer_load_b128(rs, (u * blk + tid) * 16, 0, 0);
    } else {
        load_raw_step_global<NT>(p, sv0, blk, tid, r);
    }
}

// Steps [fs, fe) of a job are full; step 0 when fs = 1 and step fe when fe < nsteps hold
// the job's partial edge vectors (there is at most one partial step on each side).
__device__ __forceinline__ void full_step_range(const Job& jb, int64_t stepv, int64_t& fs, int64_t& fe,
                                                int64_t& nsteps)
{
    nsteps = (jb.nvec + stepv - 1) / stepv;
    fs = (jb.v0 < jb.vf0) ? 1 : 0;
    fe = (jb.vf1 - jb.v0) / stepv;
    if (fe < fs) fe = fs;
}

template <typename TX>
__device__ __forceinline__ void stats_full_step(const typename Io<TX>::Raw (&r)[kStepVecs], float K,
                                                Moments<uint32_t>& acc)
{
    float t[kTile];
#pragma unroll
    for (int u = 0; u < kStepVecs; ++u) {
        float e[kVec];
        Io<TX>::widen(r[u], e);
#pragma unroll
        for (int i = 0; i < kVec; ++i) t[u * kVec + i] = e[i] - K;
    }
    float m, M2;
    tile_moments_full(t, m, M2);
    chan_merge(acc, uint32_t(kTile), m, M2);
}

template <bool NT, typename TX>
__device__ __forceinline__ void stats_masked_step(const TX* __restrict__ x, const Job& jb, int64_t sv0,
                                                  int blk, int tid, float K, Moments<uint32_t>& acc)
{
    float v[kTile];
    const uint32_t valid = load_step_masked<NT>(x, jb, sv0, blk, tid, v);
    if (valid) {
        const uint32_t cnt = __builtin_popcount(valid);
        float m, M2;
        tile_moments_masked(v, K, valid, cnt, m, M2);
        chan_merge(acc, cnt, m, M2);
    }
}

// The full steps are software-pipelined: the next step's vectors are requested before
// the current step is reduced, alternating between two register sets so that waiting for
// one set leaves the other in flight.
template <typename TX, bool NT>
__global__ void __launch_bounds__(kRedBlock)
stats_kernel(const TX* __restrict__ x, KArgs a, float2* __restrict__ part)
{
    using Raw = typename Io<TX>::Raw;
    __shared__ uint32_t s_n[kMaxWaves];
    __shared__ float s_m[kMaxWaves], s_M[kMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;

    for (int64_t wb = blockIdx.x; wb < a.jobs; wb += gridDim.x) {
        const int64_t j = wb;
        const Job jb = job_at(a.S, a.chunk, a.K, j);
        const int64_t n = jb.row / a.C, g = (jb.row - n * a.C) / a.Cg;
        const float K = group_shift(x, a, n, g);
        Moments<uint32_t> acc = {0u, 0.0f, 0.0f};
        int64_t fs, fe, nsteps;
        full_step_range(jb, stepv, fs, fe, nsteps);
        // At most one partial step before and one after the full steps. They are written as
        // conditionals: a one-trip loop over them was merged twice when built by hipcc
        // (ROCm 7.2) for gfx950.
        if (fs > 0) stats_masked_step<NT>(x, jb, jb.v0, blk, tid, K, acc);
        if (fe > fs) {
            Raw A[kStepVecs], B[kStepVecs];
            load_raw_step<NT>(x, jb.v0 + fs * stepv, blk, tid, A);
            int64_t s = fs;
            for (; s + 2 < fe; s += 2) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, B);
                stats_full_step<TX>(A, K, acc);
                load_raw_step<NT>(x, jb.v0 + (s + 2) * stepv, blk, tid, A);
                stats_full_step<TX>(B, K, acc);
            }
            if (s + 1 < fe) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, B);
                stats_full_step<TX>(A, K, acc);
                stats_full_step<TX>(B, K, acc);
            } else {
                stats_full_step<TX>(A, K, acc);
            }
        }
        if (fe < nsteps) stats_masked_step<NT>(x, jb, jb.v0 + fe * stepv, blk, tid, K, acc);
        const Moments<uint32_t> r = block_merge(acc, s_n, s_m, s_M);
        if (tid == 0) part[j] = make_float2(r.m, r.M2);
    }
}

// Shared memory of the forward finalize.
struct FinFwdLds {
    uint64_t n[kMaxWaves];
    float m[kMaxWaves], M[kMaxWaves];
    float stat[3];
};

struct GroupStat {
    float hi, lo, rstd;
};

// The forward finalize of group (n, g), called by every thread of a 256-thread workgroup:
// the group's P partials merged in a fixed order (lane t takes partials t, t + 256, ... in
// index order, then the shuffle tree, then the waves in order), var = M2 / M, rstd, and
// the mean as an unevaluated sum hi + lo: hi is the fp32 mean that is published, lo what
// rounding it left out. The normalize takes x - mean as (x - hi) - lo, which is exact in
// its first step whenever x is close to the mean. Every thread receives the result.
template <typename TX>
__device__ __forceinline__ GroupStat group_stat(const TX* __restrict__ x, const float2* __restrict__ part,
                                                const KArgs& a, float eps, int64_t n, int64_t g,
                                                FinFwdLds& l)
{
    const int64_t pbase = (n * a.C + g * a.Cg) * a.K;
    // Requested before the merge so that its latency overlaps the partials' loads.
    const float K = group_shift(x, a, n, g);
    Moments<uint64_t> acc = {0ull, 0.0f, 0.0f};
    for (int64_t j = threadIdx.x; j < a.P; j += blockDim.x) {
        const float2 pm = part[pbase + j];
        chan_merge(acc, uint64_t(job_count(a, j % a.K)), pm.x, pm.y);
    }
    const Moments<uint64_t> r = block_merge(acc, l.n, l.m, l.M);
    if (threadIdx.x == 0) {
        float var = float(double(r.M2) / double(a.M));
        var = (var < 0.0f) ? 0.0f : var;  // rounding can leave a tiny negative; NaN passes through
        const float hi = K + r.m;
        l.stat[0] = hi;
        l.stat[1] = (K - hi) + r.m;
        l.stat[2] = 1.0f / __fsqrt_rn(var + eps);
    }
    __syncthreads();
    // The next writer of l.stat is thread 0 after two barriers of the next merge.
    return GroupStat{l.stat[0], l.stat[1], l.stat[2]};
}

// Publishes group (n, g)'s mean and rstd and writes each of its rows' normalize
// coefficients (mean head, mean tail, gamma_c * rstd, beta_c).
__device__ __forceinline__ void publish_group_stat(const GroupStat& st, const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, const KArgs& a,
                                                   int64_t n, int64_t g, float* __restrict__ mean_out,
                                                   float* __restrict__ rstd_out, float4* __restrict__ coef)
{
    if (threadIdx.x == 0) {
        mean_out[n * a.G + g] = st.hi;
        rstd_out[n * a.G + g] = st.rstd;
    }
    for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) {
        const int64_t c = g * a.Cg + i;
        const float gm = gamma ? gamma[c] : 1.0f;
        const float bt = beta ? beta[c] : 0.0f;
        coef[2 * (n * a.C + c)] = make_float4(st.hi, st.lo, gm * st.rstd, bt);
    }
}

// One workgroup per group (n, g): the forward finalize, mean and rstd, and the rows'
// normalize coefficients for apply_kernel.
template <typename TX>
__global__ void __launch_bounds__(256)
fin_fwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma,
               const float* __restrict__ beta, float eps, const float2* __restrict__ part,
               float* __restrict__ mean_out, float* __restrict__ rstd_out, KArgs a,
               float4* __restrict__ coef)
{
    __shared__ FinFwdLds l;
    const int64_t ng = blockIdx.x;
    const int64_t n = ng / a.G, g = ng - n * a.G;
    const GroupStat st = group_stat(x, part, a, eps, n, g, l);
    publish_group_stat(st, gamma, beta, a, n, g, mean_out, rstd_out, coef);
}

// Vectors per lane per step of the folded streaming kernels, and the waves per SIMD they
// are compiled for (their register cap): forward 4, backward 3.
constexpr int kFinVecs = 2;

// The normalize of one element: ((x - hi) - lo) * gamma*rstd + beta, then the relu.
template <bool ACT>
struct Affine {
    float hi, lo, scale, shift;
    __device__ __forceinline__ float operator()(float e) const
    {
        const float v = fmaf((e - hi) - lo, scale, shift);
        return ACT ? relu_f(v) : v;
    }
};

// y for vector vi of job jb: one vector load and store when the vector lies wholly inside
// the job, element-wise at its edges.
template <bool NT, typename TX, typename TY, typename F>
__device__ __forceinline__ void apply_vec(const TX* __restrict__ x, TY* __restrict__ y, const Job& jb,
                                          int64_t vi, const F& f)
{
    if (vi >= jb.vf0 && vi < jb.vf1) {
        float e[kVec], o[kVec];
        Io<TX>::template load8<NT>(x + vi * kVec, e);
#pragma unroll
        for (int i = 0; i < kVec; ++i) o[i] = f(e[i]);
        Io<TY>::template store8<kNtStoreStream>(y + vi * kVec, o);
    } else {
        for (int i = 0; i < kVec; ++i) {
            const int64_t gi = vi * kVec + i;
            if (gi >= jb.lo && gi < jb.hi) Io<TY>::store1(y + gi, f(Io<TX>::load1(x + gi)));
        }
    }
}

template <typename TX, typename TY, bool NT, bool ACT>
__global__ void __launch_bounds__(256)
apply_kernel(const TX* __restrict__ x, TY* __restrict__ y, KArgs a,
             const float4* __restrict__ coef)
{
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kApplyVecs;
    for (int64_t jj = blockIdx.x; jj < a.jobs_a; jj += gridDim.x) {
        const int64_t j = step_job_in_order(jj, a);
        const Job jb = job_at(a.S, a.chunk_a, a.K_a, j);
        const float4 cf = coef[2 * jb.row];
        const Affine<ACT> f = {cf.x, cf.y, cf.z, cf.w};
        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
#pragma unroll
            for (int u = 0; u < kApplyVecs; ++u) apply_vec<NT>(x, y, jb, sv0 + int64_t(u) * blk + tid, f);
        }
    }
}

// y for the lane's V vectors of one full step, from raw loads.
template <typename TX, typename TY, int V, typename F>
__device__ __forceinline__ void apply_full_step(const typename Io<TX>::Raw (&r)[V], TY* __restrict__ y,
                                                int64_t sv0, int blk, int tid, const F& f)
{
#pragma unroll
    for (int u = 0; u < V; ++u) {
        float e[kVec], o[kVec];
        Io<TX>::widen(r[u], e);
#pragma unroll
        for (int i = 0; i < kVec; ++i) o[i] = f(e[i]);
        Io<TY>::template store8<kNtStoreStream>(y + (sv0 + int64_t(u) * blk + tid) * kVec, o);
    }
}

// The normalize with the forward finalize folded in ("Optimize GroupNorm", the paragraph
// folding the finalize into the elementwise kernels with a capped grid), over the folded
// streaming jobs: each 256-thread workgroup takes one job (a contiguous run of one row of
// at most kFoldChunk elements), merges its group's P partials exactly as fin_fwd_kernel does (so the
// statistics are bitwise those of the split-phase path), and streams the job. The
// partials it re-reads are a few percent of the bytes it moves, and the separate
// finalize launch is gone. The group's first job publishes mean, rstd and the rows'
// coefficients. The job's first full step is requested before the merge so that its
// latency overlaps it; the full steps are software-pipelined as in stats_kernel.
template <typename TX, typename TY, bool NT, bool ACT>
__global__ void __launch_bounds__(256, 4)
apply_fin_kernel(const TX* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
                 float eps, const float2* __restrict__ part, float* __restrict__ mean_out,
                 float* __restrict__ rstd_out, KArgs a, float4* __restrict__ coef, TY* __restrict__ y)
{
    using Raw = typename Io<TX>::Raw;
    __shared__ FinFwdLds l;
    const int tid = threadIdx.x, blk = blockDim.x;
    constexpr int V = kFinVecs;
    const int64_t stepv = int64_t(blk) * V;
    for (int64_t jj = blockIdx.x; jj < a.jobs_f; jj += gridDim.x) {
        const int64_t j = job_in_order(jj, a);
        const Job jb = job_at(a.S, a.chunk_f, a.K_f, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, g = c / a.Cg;
        int64_t fs, fe, nsteps;
        full_step_range(jb, stepv, fs, fe, nsteps);
        Raw A[V], B[V];
        if (fe > fs) load_raw_step<NT>(x, jb.v0 + fs * stepv, blk, tid, A);
        const GroupStat st = group_stat(x, part, a, eps, n, g, l);
        if (jb.k == 0 && c == g * a.Cg) publish_group_stat(st, gamma, beta, a, n, g, mean_out, rstd_out, coef);
        const Affine<ACT> f = {st.hi, st.lo, (gamma ? gamma[c] : 1.0f) * st.rstd, beta ? beta[c] : 0.0f};
        // The edge steps stay rolled: unrolled, their element-wise loads would set the
        // kernel's register count.
        if (fs > 0) {
#pragma unroll 1
            for (int u = 0; u < V; ++u) apply_vec<NT>(x, y, jb, jb.v0 + int64_t(u) * blk + tid, f);
        }
        if (fe > fs) {
            int64_t s = fs;
            for (; s + 2 < fe; s += 2) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, B);
                apply_full_step<TX, TY, V>(A, y, jb.v0 + s * stepv, blk, tid, f);
                load_raw_step<NT>(x, jb.v0 + (s + 2) * stepv, blk, tid, A);
                apply_full_step<TX, TY, V>(B, y, jb.v0 + (s + 1) * stepv, blk, tid, f);
            }
            if (s + 1 < fe) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, B);
                apply_full_step<TX, TY, V>(A, y, jb.v0 + s * stepv, blk, tid, f);
                apply_full_step<TX, TY, V>(B, y, jb.v0 + (s + 1) * stepv, blk, tid, f);
            } else {
                apply_full_step<TX, TY, V>(A, y, jb.v0 + s * stepv, blk, tid, f);
            }
        }
        if (fe < nsteps) {
#pragma unroll 1
            for (int u = 0; u < V; ++u) apply_vec<NT>(x, y, jb, jb.v0 + fe * stepv + int64_t(u) * blk + tid, f);
        }
    }
}

// ------------------------------------------------------------------ backward

// One full step of the backward sums. With the relu, dy is gated on the recomputed
// pre-activation pre = (x - mean) * gamma*rstd + beta.
template <typename TX, typename TD>
__device__ __forceinline__ void bwd_full_step(const typename Io<TX>::Raw (&rx)[kStepVecs],
                                              const typename Io<TD>::Raw (&rd)[kStepVecs], float mu,
                                              bool act, float scale, float shift, float& s1, float& s2)
{
    float d[kTile], gv[kTile];
#pragma unroll
    for (int u = 0; u < kStepVecs; ++u) {
        float e[kVec], f[kVec];
        Io<TX>::widen(rx[u], e);
        Io<TD>::widen(rd[u], f);
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            d[u * kVec + i] = e[i] - mu;
            gv[u * kVec + i] = act ? relu_gate(fmaf(d[u * kVec + i], scale, shift), f[i]) : f[i];
        }
    }
    s1 = s1 + tree_sum(gv);
    s2 = s2 + tree_sumprod(gv, d);
}

template <bool NT, typename TX, typename TD>
__device__ __forceinline__ void bwd_masked_step(const TD* __restrict__ dy, const TX* __restrict__ x,
                                                const Job& jb, int64_t sv0, int blk, int tid, float mu,
                                                bool act, float scale, float shift, float& s1, float& s2)
{
    float xv[kTile], gv[kTile];
    const uint32_t valid = load_step_masked<NT>(x, jb, sv0, blk, tid, xv);
    load_step_masked<NT>(dy, jb, sv0, blk, tid, gv);  // same mask: zeros outside
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        xv[i] = ((valid >> i) & 1u) ? xv[i] - mu : 0.0f;
        if (act) gv[i] = relu_gate(fmaf(xv[i], scale, shift), gv[i]);
    }
    s1 = s1 + tree_sum(gv);
    s2 = s2 + tree_sumprod(gv, xv);
}

// Per job: s1 = sum dy and s2 = rstd * sum dy * (x - mean) over the job's elements, lanes
// summing their tiles in step order, then the shuffle tree, then the waves in order. The
// full steps are software-pipelined as in stats_kernel. The relu gate is a template
// parameter (with_act): read from the launch arguments at run time, it was evaluated on
// every element and then discarded when off (an fma, two compares and two selects an
// element).
template <typename TX, typename TD, bool NT, bool ACT>
__global__ void __launch_bounds__(kRedBlock)
bwd_reduce_kernel(const TD* __restrict__ dy, const TX* __restrict__ x,
                  const float* __restrict__ mean, const float* __restrict__ rstd,
                  const float* __restrict__ gamma, const float* __restrict__ beta,
                  KArgs a, float2* __restrict__ part)
{
    using RawX = typename Io<TX>::Raw;
    using RawD = typename Io<TD>::Raw;
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kStepVecs;

    for (int64_t wb = blockIdx.x; wb < a.jobs; wb += gridDim.x) {
        const int64_t j = wb;
        const Job jb = job_at(a.S, a.chunk, a.K, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, ng = n * a.G + c / a.Cg;
        const float mu = mean[ng];
        constexpr bool act = ACT;
        const float scale = act ? rstd[ng] * (gamma ? gamma[c] : 1.0f) : 0.0f;
        const float shift = act ? (beta ? beta[c] : 0.0f) : 0.0f;
        float s1 = 0.0f, s2 = 0.0f;  // sum dy, sum dy * (x - mu)
        int64_t fs, fe, nsteps;
        full_step_range(jb, stepv, fs, fe, nsteps);
        if (fs > 0) bwd_masked_step<NT>(dy, x, jb, jb.v0, blk, tid, mu, act, scale, shift, s1, s2);
        if (fe > fs) {
            RawX AX[kStepVecs], BX[kStepVecs];
            RawD AD[kStepVecs], BD[kStepVecs];
            load_raw_step<NT>(x, jb.v0 + fs * stepv, blk, tid, AX);
            load_raw_step_global<NT>(dy, jb.v0 + fs * stepv, blk, tid, AD);
            int64_t s = fs;
            for (; s + 2 < fe; s += 2) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, BX);
                load_raw_step_global<NT>(dy, jb.v0 + (s + 1) * stepv, blk, tid, BD);
                bwd_full_step<TX, TD>(AX, AD, mu, act, scale, shift, s1, s2);
                load_raw_step<NT>(x, jb.v0 + (s + 2) * stepv, blk, tid, AX);
                load_raw_step_global<NT>(dy, jb.v0 + (s + 2) * stepv, blk, tid, AD);
                bwd_full_step<TX, TD>(BX, BD, mu, act, scale, shift, s1, s2);
            }
            if (s + 1 < fe) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, BX);
                load_raw_step_global<NT>(dy, jb.v0 + (s + 1) * stepv, blk, tid, BD);
                bwd_full_step<TX, TD>(AX, AD, mu, act, scale, shift, s1, s2);
                bwd_full_step<TX, TD>(BX, BD, mu, act, scale, shift, s1, s2);
            } else {
                bwd_full_step<TX, TD>(AX, AD, mu, act, scale, shift, s1, s2);
            }
        }
        if (fe < nsteps) bwd_masked_step<NT>(dy, x, jb, jb.v0 + fe * stepv, blk, tid, mu, act, scale, shift, s1, s2);
        const float2 r = block_sum2(s1, s2, s_a, s_b);
        if (tid == 0) part[j] = make_float2(r.x, r.y * rstd[ng]);
    }
}

// c1 = (1/M) sum gamma_c s1 and c2 = (1/M) sum gamma_c s2 of group (n, g), called by every
// thread of a 256-thread workgroup: the group's P partials in a fixed order (lane t takes
// partials t, t + 256, ... in index order, then the shuffle tree, then the waves in order).
// Every thread receives the result.
__device__ __forceinline__ float2 group_c12(const float2* __restrict__ part, const float* __restrict__ gamma,
                                            const KArgs& a, int64_t n, int64_t g, float* s_a, float* s_b,
                                            float* s_coef)
{
    const int64_t pbase = (n * a.C + g * a.Cg) * a.K;
    float t1 = 0.0f, t2 = 0.0f;
    for (int64_t i = threadIdx.x; i < a.P; i += blockDim.x) {
        const float2 pp = part[pbase + i];
        const float gm = gamma ? gamma[g * a.Cg + i / a.K] : 1.0f;
        t1 = t1 + gm * pp.x;
        t2 = t2 + gm * pp.y;
    }
    const float2 r = block_sum2(t1, t2, s_a, s_b);
    if (threadIdx.x == 0) {
        s_coef[0] = float(double(r.x) / double(a.M));
        s_coef[1] = float(double(r.y) / double(a.M));
    }
    __syncthreads();
    // The next writer of s_coef is thread 0 after two barriers of the next sum.
    return make_float2(s_coef[0], s_coef[1]);
}

// The dx coefficients of row (n, c): mean, A = rstd*gamma_c, B = -rstd*c1, E = -rstd^2*c2, so
// that dx = rstd*(gamma_c*g - c1 - xhat*c2) = A*g + (B + E*(x - mean)), where g is dy, or with
// the relu dy gated on pre = (x - mean)*A + beta_c.
template <bool ACT>
struct DxCoef {
    float mu, A, B, E, bt;
    bool single;
    // A single-element group is answered as t - t: +0 for finite t, NaN otherwise.
    __device__ __forceinline__ float operator()(float xv, float gv) const
    {
        float t = full(xv, gv);
        if (single) t = t - t;
        return t;
    }
    // The same without the single-element rule, for full steps: a single-element group's
    // rows are one element long, so no full step ever holds one.
    __device__ __forceinline__ float full(float xv, float gv) const
    {
        const float d = xv - mu;
        const float g = ACT ? relu_gate(fmaf(d, A, bt), gv) : gv;
        return fmaf(A, g, fmaf(E, d, B));
    }
};

template <bool ACT>
__device__ __forceinline__ DxCoef<ACT> dx_coef(float mu, float rs, float gm, float2 c12, float bt, const KArgs& a)
{
    return DxCoef<ACT>{mu, rs * gm, -(rs * c12.x), -((rs * rs) * c12.y), bt, a.M == 1};
}

// Writes the dx coefficient records of group (n, g)'s rows for bwd_apply_kernel.
__device__ __forceinline__ void publish_dx_coef(float mu, float rs, float2 c12, const float* __restrict__ gamma,
                                                const float* __restrict__ beta, const KArgs& a, int64_t n,
                                                int64_t g, float4* __restrict__ coef)
{
    for (int64_t i = threadIdx.x; i < a.Cg; i += blockDim.x) {
        const int64_t c = g * a.Cg + i;
        const DxCoef<false> k = dx_coef<false>(mu, rs, gamma ? gamma[c] : 1.0f, c12, 0.0f, a);
        coef[2 * (n * a.C + c)] = make_float4(mu, k.A, k.B, k.E);
        coef[2 * (n * a.C + c) + 1] = make_float4(beta ? beta[c] : 0.0f, a.M == 1 ? 1.0f : 0.0f, 0.0f, 0.0f);
    }
}

// dgamma_c and dbeta_c as the sums of channel c's N*K partials, n-major then k, in a fixed
// order (lane t takes t, t + 256, ..., then the shuffle tree, then the waves in order);
// called by every thread, written by thread 0.
__device__ __forceinline__ void channel_param_sums(const float2* __restrict__ part, const KArgs& a, int64_t c,
                                                   float* s_a, float* s_b, float* __restrict__ dgamma,
                                                   float* __restrict__ dbeta)
{
    float sa = 0.0f, sb = 0.0f;
    for (int64_t i = threadIdx.x; i < a.N * a.K; i += blockDim.x) {
        const int64_t nn = i / a.K, kk = i - nn * a.K;
        const float2 pp = part[(nn * a.C + c) * a.K + kk];
        sa = sa + pp.y;
        sb = sb + pp.x;
    }
    const float2 r = block_sum2(sa, sb, s_a, s_b);
    if (threadIdx.x == 0) {
        if (dgamma) dgamma[c] = r.x;
        if (dbeta) dbeta[c] = r.y;
    }
}

// Workgroups [0, ngroups) each take one group (n, g): c1 and c2, then each row's dx
// coefficients and beta_c. Workgroups [ngroups, ngroups + nchan) each take one channel c:
// dgamma_c and dbeta_c.
__global__ void __launch_bounds__(256)
fin_bwd_kernel(const float* __restrict__ mean, const float* __restrict__ rstd,
               const float* __restrict__ gamma, const float* __restrict__ beta,
               const float2* __restrict__ part, KArgs a,
               int64_t ngroups, int64_t nchan, float4* __restrict__ coef,
               float* __restrict__ dgamma, float* __restrict__ dbeta)
{
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    __shared__ float s_coef[2];
    const int64_t w = blockIdx.x;
    if (w < ngroups) {
        const int64_t n = w / a.G, g = w - n * a.G;
        const float mu = mean[w], rs = rstd[w];  // requested before the merge
        const float2 c12 = group_c12(part, gamma, a, n, g, s_a, s_b, s_coef);
        publish_dx_coef(mu, rs, c12, gamma, beta, a, n, g, coef);
    } else if (w < ngroups + nchan) {
        channel_param_sums(part, a, w - ngroups, s_a, s_b, dgamma, dbeta);
    }
}

// dx for vector vi of job jb: vector loads and store when the vector lies wholly inside the
// job, element-wise at its edges.
template <bool NT, typename TX, typename TD, typename F>
__device__ __forceinline__ void dx_vec(const TD* __restrict__ dy, const TX* __restrict__ x, TX* __restrict__ dx,
                                       const Job& jb, int64_t vi, const F& k)
{
    if (vi >= jb.vf0 && vi < jb.vf1) {
        float xv[kVec], gv[kVec], o[kVec];
        Io<TX>::template load8<NT>(x + vi * kVec, xv);
        Io<TD>::template load8<NT>(dy + vi * kVec, gv);
#pragma unroll
        for (int i = 0; i < kVec; ++i) o[i] = k(xv[i], gv[i]);
        Io<TX>::template store8<kNtStoreStream>(dx + vi * kVec, o);
    } else {
        for (int i = 0; i < kVec; ++i) {
            const int64_t gi = vi * kVec + i;
            if (gi >= jb.lo && gi < jb.hi) Io<TX>::store1(dx + gi, k(Io<TX>::load1(x + gi), Io<TD>::load1(dy + gi)));
        }
    }
}

template <typename TX, typename TD, bool NT, bool ACT>
__global__ void __launch_bounds__(256)
bwd_apply_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, KArgs a,
                 const float4* __restrict__ coef, TX* __restrict__ dx)
{
    const int tid = threadIdx.x, blk = blockDim.x;
    const int64_t stepv = int64_t(blk) * kApplyVecs;
    for (int64_t jj = blockIdx.x; jj < a.jobs_a; jj += gridDim.x) {
        const int64_t j = step_job_in_order(jj, a);
        const Job jb = job_at(a.S, a.chunk_a, a.K_a, j);
        const float4 cf = coef[2 * jb.row], cg = coef[2 * jb.row + 1];
        // Whether the whole group is one element comes from the record: a spatial shard's
        // piece of a group can be one element when the group is not.
        const DxCoef<ACT> k = {cf.x, cf.y, cf.z, cf.w, ACT ? cg.x : 0.0f, cg.y != 0.0f};
        for (int64_t sv0 = jb.v0; sv0 < jb.v0 + jb.nvec; sv0 += stepv) {
#pragma unroll
            for (int u = 0; u < kApplyVecs; ++u) dx_vec<NT>(dy, x, dx, jb, sv0 + int64_t(u) * blk + tid, k);
        }
    }
}

// dx for the lane's V vectors of one full step, from raw loads.
template <typename TX, typename TD, int V, typename F>
__device__ __forceinline__ void dx_full_step(const typename Io<TX>::Raw (&rx)[V],
                                             const typename Io<TD>::Raw (&rd)[V], TX* __restrict__ dx,
                                             int64_t sv0, int blk, int tid, const F& k)
{
#pragma unroll
    for (int u = 0; u < V; ++u) {
        float xv[kVec], gv[kVec], o[kVec];
        Io<TX>::widen(rx[u], xv);
        Io<TD>::widen(rd[u], gv);
#pragma unroll
        for (int i = 0; i < kVec; ++i) o[i] = k.full(xv[i], gv[i]);
        Io<TX>::template store8<kNtStoreStream>(dx + (sv0 + int64_t(u) * blk + tid) * kVec, o);
    }
}

// dx with the backward finalize folded in, over the folded streaming jobs, as apply_fin_kernel
// does for the forward: each 256-thread workgroup takes one job, forms its group's c1, c2
// exactly as fin_bwd_kernel does, and streams the job. The group's first job writes the
// rows' coefficient records; the first job of channel c in sample 0 writes dgamma_c and
// dbeta_c, summed exactly as fin_bwd_kernel sums them.
// Workgroups a CU the folded dx kernel is compiled for, which sets its register budget:
// 3 in general; 6 (at most 80 VGPRs, six waves a SIMD) for the cached relu build with
// bf16 x and 16-bit dy, which otherwise took 95 VGPRs and ran five waves a SIMD. With the
// cap it takes 78, spills none and moves SGPRs to VGPR lanes instead: relu step at 128^3
// 163.2 -> 162.1 us, 64^3 x 64 49.5 -> 48.4 (interleaved A/B, same bits). The other input
// types spill to memory under that cap, so they keep 3.
template <typename TX, typename TD, bool NT, bool ACT>
constexpr int bwd_apply_fin_blocks()
{
    return (ACT && !NT && std::is_same<TX, uint16_t>::value && sizeof(TD) == 2) ? 6 : 3;
}

template <typename TX, typename TD, bool NT, bool ACT>
__global__ void __launch_bounds__(256, (bwd_apply_fin_blocks<TX, TD, NT, ACT>()))
bwd_apply_fin_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ mean,
                     const float* __restrict__ rstd, const float* __restrict__ gamma,
                     const float* __restrict__ beta, const float2* __restrict__ part, KArgs a,
                     float4* __restrict__ coef, float* __restrict__ dgamma, float* __restrict__ dbeta,
                     TX* __restrict__ dx)
{
    using RawX = typename Io<TX>::Raw;
    using RawD = typename Io<TD>::Raw;
    __shared__ float s_a[kMaxWaves], s_b[kMaxWaves];
    __shared__ float s_coef[2];
    const int tid = threadIdx.x, blk = blockDim.x;
    constexpr int V = kFinVecs;
    const int64_t stepv = int64_t(blk) * V;
    for (int64_t jj = blockIdx.x; jj < a.jobs_f; jj += gridDim.x) {
        const int64_t j = job_in_order(jj, a);
        const Job jb = job_at(a.S, a.chunk_f, a.K_f, j);
        const int64_t n = jb.row / a.C, c = jb.row - n * a.C, g = c / a.Cg, ng = n * a.G + g;
        int64_t fs, fe, nsteps;
        full_step_range(jb, stepv, fs, fe, nsteps);
        RawX AX[V], BX[V];
        RawD AD[V], BD[V];
        if (fe > fs) {
            load_raw_step<NT>(x, jb.v0 + fs * stepv, blk, tid, AX);
            load_raw_step<NT>(dy, jb.v0 + fs * stepv, blk, tid, AD);
        }
        const float mu = mean[ng], rs = rstd[ng];
        const float2 c12 = group_c12(part, gamma, a, n, g, s_a, s_b, s_coef);
        if (jb.k == 0 && c == g * a.Cg) publish_dx_coef(mu, rs, c12, gamma, beta, a, n, g, coef);
        if ((dgamma || dbeta) && jb.k == 0 && n == 0) channel_param_sums(part, a, c, s_a, s_b, dgamma, dbeta);
        constexpr bool act = ACT;
        const DxCoef<ACT> k = dx_coef<ACT>(mu, rs, gamma ? gamma[c] : 1.0f, c12, act ? (beta ? beta[c] : 0.0f) : 0.0f, a);
        if (fs > 0) {  // rolled, as in apply_fin_kernel
#pragma unroll 1
            for (int u = 0; u < V; ++u) dx_vec<NT>(dy, x, dx, jb, jb.v0 + int64_t(u) * blk + tid, k);
        }
        if (fe > fs) {
            int64_t s = fs;
            for (; s + 2 < fe; s += 2) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, BX);
                load_raw_step<NT>(dy, jb.v0 + (s + 1) * stepv, blk, tid, BD);
                dx_full_step<TX, TD, V>(AX, AD, dx, jb.v0 + s * stepv, blk, tid, k);
                load_raw_step<NT>(x, jb.v0 + (s + 2) * stepv, blk, tid, AX);
                load_raw_step<NT>(dy, jb.v0 + (s + 2) * stepv, blk, tid, AD);
                dx_full_step<TX, TD, V>(BX, BD, dx, jb.v0 + (s + 1) * stepv, blk, tid, k);
            }
            if (s + 1 < fe) {
                load_raw_step<NT>(x, jb.v0 + (s + 1) * stepv, blk, tid, BX);
                load_raw_step<NT>(dy, jb.v0 + (s + 1) * stepv, blk, tid, BD);
                dx_full_step<TX, TD, V>(AX, AD, dx, jb.v0 + s * stepv, blk, tid, k);
                dx_full_step<TX, TD, V>(BX, BD, dx, jb.v0 + (s + 1) * stepv, blk, tid, k);
            } else {
                dx_full_step<TX, TD, V>(AX, AD, dx, jb.v0 + s * stepv, blk, tid, k);
            }
        }
        if (fe < nsteps) {
#pragma unroll 1
            for (int u = 0; u < V; ++u) dx_vec<NT>(dy, x, dx, jb, jb.v0 + fe * stepv + int64_t(u) * blk + tid, k);
        }
    }
}

// ------------------------------------------------------------------ resident path
//
// Groups whose rows are whole 8-element vectors and that fit in one workgroup (at most
// kResMaxVecs vectors) are held in registers by one workgroup from the single read to the
// write. The forward reads x once instead of twice, and each direction is one launch
// instead of three; at the 8^3-16^3 sites of a UNet's deep levels the launches, about 5 us
// each on MI355X, and not the bytes, are the cost. Lane t owns vectors t, t + B, t + 2B, ...
// of the workgroup's range (B threads, V vectors each), counted in elements as above, so
// fp32 and bf16 data reduce in the same order. The statistics are an exact two-pass over
// the registers (mean of x - K, then the corrected sum of squared deviations), relative
// to the group's shift K as in the two-pass kernels.

// Forward, one workgroup per group: blockIdx.x = g, blockIdx.y = n. Writes mean, rstd, the
// per-row normalize coefficients (the record fin_fwd_kernel writes, so that
// gn_forward_apply can follow) and y unless y is null, computed exactly as apply_kernel
// computes it from those coefficients.
template <int V, typename TX, typename TY, bool ACT>
__global__ void __launch_bounds__(kResMaxBlock)
res_fwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma,
               const float* __restrict__ beta, float eps, float* __restrict__ mean_out,
               float* __restrict__ rstd_out, KArgs a, float4* __restrict__ coef, TY* __restrict__ y)
{
    __shared__ float s_red[2 * kResMaxWaves];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int vg = int(a.M / kVec);    // vectors per group (<= kResMaxVecs)
    const float fM = float(a.M);       // exact: M <= 8 * kResMaxVecs
    constexpr bool act = ACT;
    const int64_t g = blockIdx.x, n = blockIdx.y, ng = n * a.G + g;
    const int64_t row0 = n * a.C + g * a.Cg;
    const int64_t vb = row0 * (a.S / kVec);  // the group's first vector
    const float K = group_shift(x, a, n, g);
    float e[V * kVec];
    float gms[V], bts[V];  // the vector's gamma_c and beta_c, requested with its loads
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int w = u * blk + tid;
        float v[kVec];
        gms[u] = 1.0f;
        bts[u] = 0.0f;
        if (w < vg) {
            Io<TX>::template load8<kNtApply>(x + (vb + w) * kVec, v);
            const int64_t c = g * a.Cg + fdiv(uint32_t(w), a.div_W);
            if (gamma) gms[u] = gamma[c];
            if (beta) bts[u] = beta[c];
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
    for (int i = tid; i < int(a.Cg); i += blk) {
        const int64_t c = g * a.Cg + i;
        coef[2 * (row0 + i)] = make_float4(hi, lo, (gamma ? gamma[c] : 1.0f) * rstd, beta ? beta[c] : 0.0f);
    }
    if (y) {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int w = u * blk + tid;
            if (w < vg) {
                const float scale = gms[u] * rstd;
                const float shift = bts[u];
                float o[kVec];
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const float v = fmaf((e[u * kVec + i] - hi) - lo, scale, shift);
                    o[i] = act ? relu_f(v) : v;
                }
                Io<TY>::store8(y + (vb + w) * kVec, o);
            }
        }
    }
}

// Backward, one workgroup per g covering the groups (n, g) of all N samples, vector w of
// the workgroup being vector w mod (M/8) of sample w / (M/8), so that row rho = w / (S/8)
// of the workgroup is row (n, c) = (rho / (C/G), g*C/G + rho mod (C/G)). Per vector: sum g
// and sum g*(x - mean) (g = dy, or dy gated by the relu) into LDS; per row, in a fixed
// order: s1 and s2 = rstd * sum g*(x - mean); per sample: c1, c2 and the dx coefficients
// (the record fin_bwd_kernel writes, for gn_backward_apply); per channel: dgamma and dbeta
// over the samples in order; then dx unless dx is null, computed exactly as
// bwd_apply_kernel computes it from those coefficients.
template <int V, typename TX, typename TD, bool ACT>
__global__ void __launch_bounds__(kResMaxBlock)
res_bwd_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ mean,
               const float* __restrict__ rstd, const float* __restrict__ gamma,
               const float* __restrict__ beta, KArgs a, float4* __restrict__ coef,
               float* __restrict__ dgamma, float* __restrict__ dbeta, TX* __restrict__ dx)
{
    __shared__ float s_v1[kResMaxVecs], s_v2[kResMaxVecs];  // per vector; later B, E per sample
    __shared__ float s_r1[kResMaxVecs], s_r2[kResMaxVecs];  // per row, sample-major
    const int tid = threadIdx.x, blk = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = blk >> 6;
    const int W = int(a.S / kVec), Cg = int(a.Cg), N = int(a.N);
    const int nvt = N * int(a.M / kVec);  // vectors of the workgroup (<= kResMaxVecs)
    const int nrows = N * Cg;             // rows of the workgroup
    constexpr bool act = ACT;
    const int64_t g = blockIdx.x;
    // The global vector index of workgroup row rho, and its sample and channel.
    auto row_base = [&](int rho, int& n, int& c) {
        n = int(fdiv(uint32_t(rho), a.div_Cg));
        c = int(g * Cg) + (rho - n * Cg);
        return (int64_t(n) * a.C + c) * W;
    };
    float xs[V * kVec], gs[V * kVec];
    float mus[V], As[V];  // the vector's mean and rstd*gamma_c, kept for the dx
    int rows[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int w = u * blk + tid;
        rows[u] = -1;
        mus[u] = 0.0f;
        As[u] = 0.0f;
        if (w < nvt) {
            const int rho = int(fdiv(uint32_t(w), a.div_W));
            int n, c;
            const int64_t gv = row_base(rho, n, c) + (w - rho * W);
            const int64_t ng = int64_t(n) * a.G + g;
            float e[kVec], f[kVec], d[kVec], q[kVec];
            Io<TX>::template load8<kNtBwdApply>(x + gv * kVec, e);
            Io<TD>::template load8<kNtBwdApply>(dy + gv * kVec, f);
            const float mu = mean[ng];
            const float A = rstd[ng] * (gamma ? gamma[c] : 1.0f);
            const float bt = beta ? beta[c] : 0.0f;
            mus[u] = mu;
            As[u] = A;
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                d[i] = e[i] - mu;
                q[i] = act ? relu_gate(fmaf(d[i], A, bt), f[i]) : f[i];
                xs[u * kVec + i] = e[i];
                gs[u * kVec + i] = q[i];
            }
            s_v1[w] = tree_sum(q);
            s_v2[w] = tree_sumprod(q, d);
            rows[u] = rho;
        }
    }
    __syncthreads();
    for (int rho = wave; rho < nrows; rho += nw) {
        const int n = int(fdiv(uint32_t(rho), a.div_Cg));
        const float rsn = rstd[int64_t(n) * a.G + g];  // requested before the sums
        float p1 = 0.0f, p2 = 0.0f;
        for (int k = lane; k < W; k += 64) {
            p1 = p1 + s_v1[rho * W + k];
            p2 = p2 + s_v2[rho * W + k];
        }
        p1 = wave_sum(p1);
        p2 = wave_sum(p2);
        if (lane == 0) {
            s_r1[rho] = p1;
            s_r2[rho] = p2 * rsn;
        }
    }
    __syncthreads();
    for (int n = wave; n < N; n += nw) {
        const float rs = rstd[int64_t(n) * a.G + g];  // requested before the sums
        float t1 = 0.0f, t2 = 0.0f;
        for (int i = lane; i < Cg; i += 64) {
            const float gm = gamma ? gamma[g * Cg + i] : 1.0f;
            t1 = t1 + gm * s_r1[n * Cg + i];
            t2 = t2 + gm * s_r2[n * Cg + i];
        }
        t1 = wave_sum(t1);
        t2 = wave_sum(t2);
        if (lane == 0) {
            const float c1 = float(double(t1) / double(a.M));
            const float c2 = float(double(t2) / double(a.M));
            s_v1[n] = -(rs * c1);
            s_v2[n] = -((rs * rs) * c2);
        }
    }
    __syncthreads();
    for (int rho = tid; rho < nrows; rho += blk) {
        int n, c;
        (void)row_base(rho, n, c);
        const int64_t ng = int64_t(n) * a.G + g, row = int64_t(n) * a.C + c;
        const float gm = gamma ? gamma[c] : 1.0f;
        coef[2 * row] = make_float4(mean[ng], rstd[ng] * gm, s_v1[n], s_v2[n]);
        coef[2 * row + 1] = make_float4(beta ? beta[c] : 0.0f, a.M == 1 ? 1.0f : 0.0f, 0.0f, 0.0f);
    }
    if (dgamma || dbeta) {
        for (int i = wave; i < Cg; i += nw) {
            float q1 = 0.0f, q2 = 0.0f;
            for (int n = lane; n < N; n += 64) {
                q1 = q1 + s_r2[n * Cg + i];
                q2 = q2 + s_r1[n * Cg + i];
            }
            q1 = wave_sum(q1);
            q2 = wave_sum(q2);
            if (lane == 0) {
                if (dgamma) dgamma[g * Cg + i] = q1;
                if (dbeta) dbeta[g * Cg + i] = q2;
            }
        }
    }
    if (dx) {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int rho = rows[u];
            if (rho >= 0) {
                const int w = u * blk + tid;
                int n, c;
                const int64_t gv = row_base(rho, n, c) + (w - rho * W);
                const float mu = mus[u];
                const float A = As[u];
                const float B = s_v1[n], E = s_v2[n];
                float o[kVec];
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const float d = xs[u * kVec + i] - mu;
                    o[i] = fmaf(A, gs[u * kVec + i], fmaf(E, d, B));
                }
                Io<TX>::store8(dx + gv * kVec, o);
            }
        }
    }
}

// Backward split over samples, one workgroup per (g, n) = (blockIdx.x, blockIdx.y): the
// results of res_bwd_kernel, bit for bit, from N times as many workgroups. The workgroup's
// vectors are its own group (n, g), rows rho = 0 .. C/G - 1 (vector rho*W + k), then the
// "column" rows: for each channel i of the group with i mod N == n (ncol of them) and each
// other sample n' in order, row (n', g*C/G + i), at vector (C/G + crow)*W + k with
// crow = (index of n' among the other samples)*ncol + (i - n)/N. Every row's per-vector
// sums and row sums are computed exactly as res_bwd_kernel computes them, so the rows
// both kernels sum agree bitwise; the workgroup then takes sample n's c1, c2 and dx, and
// dgamma/dbeta of its channels over all samples, in the same order as res_bwd_kernel.
template <int V, typename TX, typename TD, bool ACT>
__global__ void __launch_bounds__(kResMaxBlock)
res_bwd_split_kernel(const TD* __restrict__ dy, const TX* __restrict__ x, const float* __restrict__ mean,
                     const float* __restrict__ rstd, const float* __restrict__ gamma,
                     const float* __restrict__ beta, KArgs a, float4* __restrict__ coef,
                     float* __restrict__ dgamma, float* __restrict__ dbeta, TX* __restrict__ dx)
{
    __shared__ float s_v1[kResMaxVecs], s_v2[kResMaxVecs];  // per vector
    __shared__ float s_r1[kResMaxVecs], s_r2[kResMaxVecs];  // per row: own rows, then column rows
    __shared__ float s_be[2];
    const int tid = threadIdx.x, blk = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = blk >> 6;
    const int W = int(a.S / kVec), Cg = int(a.Cg), N = int(a.N);
    const int64_t g = blockIdx.x;
    const int n = int(blockIdx.y);
    const int ncol = Cg > n ? (Cg - 1 - n) / N + 1 : 0;
    const int vg = Cg * W;
    const int nrows = Cg + (N - 1) * ncol;
    const int nvt = nrows * W;  // <= the plan's bound, within kResMaxVecs
    constexpr bool act = ACT;
    // Sample and channel of workgroup row R.
    auto row_of = [&](int R, int& nr, int& c) {
        if (R < Cg) {
            nr = n;
            c = int(g * Cg) + R;
        } else {
            const int crow = R - Cg, ni = crow / ncol, j = crow - ni * ncol;
            nr = ni < n ? ni : ni + 1;
            c = int(g * Cg) + n + j * N;
        }
    };
    float xs[V * kVec], gs[V * kVec];
    float mus[V], As[V];
    int rows[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int w = u * blk + tid;
        rows[u] = -1;
        mus[u] = 0.0f;
        As[u] = 0.0f;
        if (w < nvt) {
            const int R = int(fdiv(uint32_t(w), a.div_W));
            int nr, c;
            row_of(R, nr, c);
            const int64_t gv = (int64_t(nr) * a.C + c) * W + (w - R * W);
            const int64_t ng = int64_t(nr) * a.G + g;
            float e[kVec], f[kVec], d[kVec], q[kVec];
            Io<TX>::template load8<kNtBwdApply>(x + gv * kVec, e);
            Io<TD>::template load8<kNtBwdApply>(dy + gv * kVec, f);
            const float mu = mean[ng];
            const float A = rstd[ng] * (gamma ? gamma[c] : 1.0f);
            const float bt = beta ? beta[c] : 0.0f;
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                d[i] = e[i] - mu;
                q[i] = act ? relu_gate(fmaf(d[i], A, bt), f[i]) : f[i];
                xs[u * kVec + i] = e[i];
                gs[u * kVec + i] = q[i];
            }
            s_v1[w] = tree_sum(q);
            s_v2[w] = tree_sumprod(q, d);
            if (w < vg) {  // own vectors: kept for the dx
                rows[u] = R;
                mus[u] = mu;
                As[u] = A;
            }
        }
    }
    __syncthreads();
    for (int R = wave; R < nrows; R += nw) {
        int nr, c;
        row_of(R, nr, c);
        const float rsn = rstd[int64_t(nr) * a.G + g];
        float p1 = 0.0f, p2 = 0.0f;
        for (int k = lane; k < W; k += 64) {
            p1 = p1 + s_v1[R * W + k];
            p2 = p2 + s_v2[R * W + k];
        }
        p1 = wave_sum(p1);
        p2 = wave_sum(p2);
        if (lane == 0) {
            s_r1[R] = p1;
            s_r2[R] = p2 * rsn;
        }
    }
    __syncthreads();
    const int64_t ngo = int64_t(n) * a.G + g;
    if (wave == 0) {
        const float rs = rstd[ngo];
        float t1 = 0.0f, t2 = 0.0f;
        for (int i = lane; i < Cg; i += 64) {
            const float gm = gamma ? gamma[g * Cg + i] : 1.0f;
            t1 = t1 + gm * s_r1[i];
            t2 = t2 + gm * s_r2[i];
        }
        t1 = wave_sum(t1);
        t2 = wave_sum(t2);
        if (lane == 0) {
            const float c1 = float(double(t1) / double(a.M));
            const float c2 = float(double(t2) / double(a.M));
            s_be[0] = -(rs * c1);
            s_be[1] = -((rs * rs) * c2);
        }
    }
    __syncthreads();
    const float B = s_be[0], E = s_be[1];
    for (int rho = tid; rho < Cg; rho += blk) {
        const int64_t c = g * Cg + rho, row = int64_t(n) * a.C + c;
        const float gm = gamma ? gamma[c] : 1.0f;
        coef[2 * row] = make_float4(mean[ngo], rstd[ngo] * gm, B, E);
        coef[2 * row + 1] = make_float4(beta ? beta[c] : 0.0f, a.M == 1 ? 1.0f : 0.0f, 0.0f, 0.0f);
    }
    if (dgamma || dbeta) {
        for (int j = wave; j < ncol; j += nw) {
            const int i = n + j * N;
            float q1 = 0.0f, q2 = 0.0f;
            for (int np = lane; np < N; np += 64) {
                const int R = np == n ? i : Cg + (np < n ? np : np - 1) * ncol + j;
                q1 = q1 + s_r2[R];
                q2 = q2 + s_r1[R];
            }
            q1 = wave_sum(q1);
            q2 = wave_sum(q2);
            if (lane == 0) {
                if (dgamma) dgamma[g * Cg + i] = q1;
                if (dbeta) dbeta[g * Cg + i] = q2;
            }
        }
    }
    if (dx) {
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int rho = rows[u];
            if (rho >= 0) {
                const int w = u * blk + tid;
                const int64_t gv = (int64_t(n) * a.C + g * Cg + rho) * W + (w - rho * W);
                float o[kVec];
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const float d = xs[u * kVec + i] - mus[u];
                    o[i] = fmaf(As[u], gs[u * kVec + i], fmaf(E, d, B));
                }
                Io<TX>::store8(dx + gv * kVec, o);
            }
        }
    }
}

}  // namespace

// ------------------------------------------------------------------ launchers

// Calls f with std::bool_constant<NT> for the streamed loads of a reduction or folded
// streaming kernel: plain loads (false) when the host found that x fits the last-level
// cache, so that the step's later kernels find x there, else the kernel's streaming policy
// Stream. The policy moves no bit of any result.
template <bool Stream, typename F>
hipError_t with_policy(const KArgs& a, F&& f)
{
    if (a.cached) return f(std::bool_constant<false>{});
    return f(std::bool_constant<Stream>{});
}

// Calls f with std::bool_constant<ACT>: whether the relu is fused, a template parameter of
// the streaming and backward-sum kernels so that the plain path carries none of its
// arithmetic.
template <typename F>
hipError_t with_act(const KArgs& a, F&& f)
{
    if (a.act) return f(std::bool_constant<true>{});
    return f(std::bool_constant<false>{});
}

hipError_t launch_stats_partials(const void* x, int xdt, const KArgs& a, Workspace ws, hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
        return with_policy<kNtStats>(a, [&](auto nt) {
            using TX = decltype(tx);
            return launch(stats_kernel<TX, decltype(nt)::value>, grid_of(a.jobs), dim3(unsigned(a.block)), st,
                          cp<TX>(x), a, ws.part);
        });
    });
}

hipError_t launch_bwd_partials(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                               const float* rstd, const float* gamma, const float* beta, const KArgs& a,
                               Workspace ws, hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
        return with_type(dydt, [&](auto td) {
            return with_policy<kNtBwdReduce>(a, [&](auto nt) {
                using TX = decltype(tx);
                using TD = decltype(td);
                constexpr bool NT = decltype(nt)::value;
                return with_act(a, [&](auto act) {
                    return launch(bwd_reduce_kernel<TX, TD, NT, decltype(act)::value>, grid_of(a.jobs),
                                  dim3(unsigned(a.block)), st, cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a,
                                  ws.part);
                });
            });
        });
    });
}

hipError_t launch_fwd_stats(const void* x, int xdt, const float* gamma, const float* beta,
                            float eps, float* mean, float* rstd, const KArgs& a, Workspace ws,
                            hipStream_t st)
{
    const hipError_t e = launch_stats_partials(x, xdt, a, ws, st);
    if (e != hipSuccess) return e;
    return launch_fin_fwd(x, xdt, gamma, beta, eps, mean, rstd, a, ws, st);
}

hipError_t launch_fin_fwd(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                          float* mean, float* rstd, const KArgs& a, Workspace ws, hipStream_t st)
{
    return with_type(xdt, [&](auto tx) {
        using TX = decltype(tx);
        return launch(fin_fwd_kernel<TX>, dim3(unsigned(a.N * a.G)), dim3(256), st, cp<TX>(x), gamma, beta,
                      eps, static_cast<const float2*>(ws.part), mean, rstd, a, ws.coef);
    });
}

hipError_t launch_fin_bwd(const float* mean, const float* rstd, const float* gamma, const float* beta,
                          float* dgamma, float* dbeta, const KArgs& a, Workspace ws, hipStream_t st)
{
    const int64_t ngroups = a.N * a.G;
    const int64_t nchan = (dgamma || dbeta) ? a.C : 0;
    return launch(fin_bwd_kernel, dim3(unsigned(ngroups + nchan)), dim3(256), st, mean, rstd, gamma, beta,
                  static_cast<const float2*>(ws.part), a, ngroups, nchan, ws.coef, dgamma, dbeta);
}

hipError_t launch_fwd_apply(const void* x, int xdt, void* y, int ydt, const KArgs& a,
                            Workspace ws, hipStream_t st)
{
    const dim3 grid = grid_of(a.jobs_a), block(unsigned(a.block_a));
    const float4* coef = ws.coef;
    return with_type(xdt, [&](auto tx) {
        return with_policy<kNtApply>(a, [&](auto nt) {
            using TX = decltype(tx);
            constexpr bool NT = decltype(nt)::value;
            return with_act(a, [&](auto act) {
                constexpr bool ACT = decltype(act)::value;
                if (ydt == kF32)
                    return launch(apply_kernel<TX, float, NT, ACT>, grid, block, st, cp<TX>(x), mp<float>(y), a,
                                  coef);
                return launch(apply_kernel<TX, TX, NT, ACT>, grid, block, st, cp<TX>(x), mp<TX>(y), a, coef);
            });
        });
    });
}

hipError_t launch_bwd_reduce(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                             const float* rstd, const float* gamma, const float* beta, float* dgamma,
                             float* dbeta, const KArgs& a, Workspace ws, hipStream_t st)
{
    const hipError_t e = launch_bwd_partials(dy, dydt, x, xdt, mean, rstd, gamma, beta, a, ws, st);
    if (e != hipSuccess) return e;
    return launch_fin_bwd(mean, rstd, gamma, beta, dgamma, dbeta, a, ws, st);
}

hipError_t launch_bwd_apply(const void* dy, int dydt, const void* x, int xdt, void* dx,
                            const KArgs& a, Workspace ws, hipStream_t st)
{
    const dim3 grid = grid_of(a.jobs_a), block(unsigned(a.block_a));
    const float4* coef = ws.coef;
    return with_type(xdt, [&](auto tx) {
        return with_type(dydt, [&](auto td) {
            return with_policy<kNtBwdApply>(a, [&](auto nt) {
                using TX = decltype(tx);
                using TD = decltype(td);
                return with_act(a, [&](auto act) {
                    return launch(bwd_apply_kernel<TX, TD, decltype(nt)::value, decltype(act)::value>, grid, block,
                                  st, cp<TD>(dy), cp<TX>(x), a, coef, mp<TX>(dx));
                });
            });
        });
    });
}

hipError_t launch_fwd_apply_fin(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                                float* mean, float* rstd, void* y, int ydt, const KArgs& a, Workspace ws,
                                hipStream_t st)
{
    const float2* part = static_cast<const float2*>(ws.part);
    return with_type(xdt, [&](auto tx) {
        return with_policy<kNtApply>(a, [&](auto nt) {
            using TX = decltype(tx);
            constexpr bool NT = decltype(nt)::value;
            return with_act(a, [&](auto act) {
                constexpr bool ACT = decltype(act)::value;
                if (ydt == kF32)
                    return launch(apply_fin_kernel<TX, float, NT, ACT>, grid_of(a.jobs_f), dim3(256), st, cp<TX>(x),
                                  gamma, beta, eps, part, mean, rstd, a, ws.coef, mp<float>(y));
                return launch(apply_fin_kernel<TX, TX, NT, ACT>, grid_of(a.jobs_f), dim3(256), st, cp<TX>(x), gamma,
                              beta, eps, part, mean, rstd, a, ws.coef, mp<TX>(y));
            });
        });
    });
}

hipError_t launch_bwd_apply_fin(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                                const float* rstd, const float* gamma, const float* beta, float* dgamma,
                                float* dbeta, void* dx, const KArgs& a, Workspace ws, hipStream_t st)
{
    const float2* part = static_cast<const float2*>(ws.part);
    return with_type(xdt, [&](auto tx) {
        return with_type(dydt, [&](auto td) {
            return with_policy<kNtBwdApply>(a, [&](auto nt) {
                using TX = decltype(tx);
                using TD = decltype(td);
                return with_act(a, [&](auto act) {
                    return launch(bwd_apply_fin_kernel<TX, TD, decltype(nt)::value, decltype(act)::value>,
                                  grid_of(a.jobs_f), dim3(256), st, cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta,
                                  part, a, ws.coef, dgamma, dbeta, mp<TX>(dx));
                });
            });
        });
    });
}

// Calls f with std::integral_constant<int, V> for the resident lane-vector count.
template <typename F>
hipError_t with_vecs(int vecs, F&& f)
{
    if (vecs == 1) return f(std::integral_constant<int, 1>{});
    if (vecs == 2) return f(std::integral_constant<int, 2>{});
    return f(std::integral_constant<int, 4>{});
}

hipError_t launch_res_fwd(const void* x, int xdt, const float* gamma, const float* beta, float eps,
                          float* mean, float* rstd, void* y, int ydt, const KArgs& a, Workspace ws,
                          hipStream_t st, int block, int vecs)
{
    const dim3 grid(unsigned(a.G), unsigned(a.N)), blk{unsigned(block)};
    return with_type(xdt, [&](auto tx) {
        return with_vecs(vecs, [&](auto v) {
            using TX = decltype(tx);
            constexpr int V = decltype(v)::value;
            return with_act(a, [&](auto act) {
                constexpr bool ACT = decltype(act)::value;
                if (y && ydt == kF32)
                    return launch(res_fwd_kernel<V, TX, float, ACT>, grid, blk, st, cp<TX>(x), gamma, beta, eps, mean,
                                  rstd, a, ws.coef, mp<float>(y));
                return launch(res_fwd_kernel<V, TX, TX, ACT>, grid, blk, st, cp<TX>(x), gamma, beta, eps, mean, rstd,
                              a, ws.coef, mp<TX>(y));
            });
        });
    });
}

hipError_t launch_res_bwd(const void* dy, int dydt, const void* x, int xdt, const float* mean,
                          const float* rstd, const float* gamma, const float* beta, float* dgamma,
                          float* dbeta, void* dx, const KArgs& a, Workspace ws, hipStream_t st,
                          int block, int vecs, bool split)
{
    return with_type(xdt, [&](auto tx) {
        return with_type(dydt, [&](auto td) {
            return with_vecs(vecs, [&](auto v) {
                using TX = decltype(tx);
                using TD = decltype(td);
                constexpr int V = decltype(v)::value;
                return with_act(a, [&](auto act) {
                    constexpr bool ACT = decltype(act)::value;
                    if (split)
                        return launch(res_bwd_split_kernel<V, TX, TD, ACT>, dim3(unsigned(a.G), unsigned(a.N)),
                                      dim3(unsigned(block)), st, cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a,
                                      ws.coef, dgamma, dbeta, mp<TX>(dx));
                    return launch(res_bwd_kernel<V, TX, TD, ACT>, dim3(unsigned(a.G)), dim3(unsigned(block)), st,
                                  cp<TD>(dy), cp<TX>(x), mean, rstd, gamma, beta, a, ws.coef, dgamma, dbeta,
                                  mp<TX>(dx));
                });
            });
        });
    });
}

}  // namespace gn
