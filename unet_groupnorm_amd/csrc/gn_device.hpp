// gn_device.hpp -- device-side building blocks shared by the GroupNorm kernel files:
// element access for fp32 / bf16 / fp16 storage, the optional relu, Chan's merge,
// fixed-order reductions and the launch helper. Every function lives in an unnamed
// namespace, so each kernel file has its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

#include "gn_launch.hpp"

namespace gn {

namespace {

// Load policy of the streamed tensors per kernel (true: nontemporal), used where the host
// has not chosen plain loads for a volume that fits the last-level cache.
constexpr bool kNtStats = true, kNtBwdReduce = true;
constexpr bool kNtApply = true, kNtBwdApply = true;
// Store policy: plain stores by default (the channels-last and resident kernels), and
// nontemporal ones in the NCDHW streaming kernels, folded and one-step. Measured on MI355X:
// the folded kernels about 7% faster at 256^3 with nontemporal stores; on a step of one-step
// kernels (the spatial-shard entry points, 1x32x32x256^2 bf16) plain stores left y and dx
// dirty in the last-level cache for the next plain-load reduction to write back (239.8 ->
// 198.7 us a step); the channels-last step went 189 -> 198 us and the resident deep config
// 15.9 -> 16.7 us with nontemporal stores, so they keep plain ones.
constexpr bool kNtStore = false, kNtStoreStream = true;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// The optional activation ("Optimize GroupNorm", paragraphs on the fused ReLU and on the
// NaN-correct ReLU): relu is 0 where v < 0 and v otherwise, so NaN, +Inf and -0.0 pass;
// its gradient is blocked where the relu result is <= 0 and passes otherwise (NaN too).
__device__ __forceinline__ float relu_f(float v) { return v < 0.0f ? 0.0f : v; }
// The backward gate of the relu: closed where relu(pre) <= 0. relu(pre) <= 0 holds exactly
// where pre <= 0 does (negatives and both zeros; a NaN pre gives a NaN relu, and both
// comparisons are false for it, so the gate stays open), so the gate tests pre directly.
__device__ __forceinline__ float relu_gate(float pre, float g) { return pre <= 0.0f ? 0.0f : g; }

// Loads of the streamed tensors are marked nontemporal: each element is read once per
// kernel, and on MI355X this lifts a streaming read from about 6.2 to about 7 TB/s.
template <typename T> struct Io;

template <> struct Io<uint16_t> {  // bf16 storage
    // One 8-element vector as loaded (16 bytes), widened only where it is used.
    struct Raw {
        u32x4 u;
    };
    template <bool NT>
    static __device__ __forceinline__ Raw load_raw(const uint16_t* p)
    {
        const u32x4* q = reinterpret_cast<const u32x4*>(p);
        return Raw{NT ? __builtin_nontemporal_load(q) : *q};
    }
    static __device__ __forceinline__ void widen(const Raw& r, float (&v)[8])
    {
        v[0] = bf16_lo(r.u.x); v[1] = bf16_hi(r.u.x);
        v[2] = bf16_lo(r.u.y); v[3] = bf16_hi(r.u.y);
        v[4] = bf16_lo(r.u.z); v[5] = bf16_hi(r.u.z);
        v[6] = bf16_lo(r.u.w); v[7] = bf16_hi(r.u.w);
    }
    template <bool NT>
    static __device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8])
    {
        widen(load_raw<NT>(p), v);
    }
    static __device__ __forceinline__ float load1(const uint16_t* p)
    {
        return __uint_as_float(uint32_t(*p) << 16);
    }
    template <bool NT = kNtStore>
    static __device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8])
    {
        u32x4 u;
        u.x = pack_bf16(v[0], v[1]);
        u.y = pack_bf16(v[2], v[3]);
        u.z = pack_bf16(v[4], v[5]);
        u.w = pack_bf16(v[6], v[7]);
        if (NT)
            __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
        else
            *reinterpret_cast<u32x4*>(p) = u;
    }
    static __device__ __forceinline__ void store1(uint16_t* p, float v)
    {
        *p = uint16_t(pack_bf16(v, 0.0f) & 0xffffu);
    }
};

template <> struct Io<float> {
    struct Raw {
        f32x4 a, b;
    };
    template <bool NT>
    static __device__ __forceinline__ Raw load_raw(const float* p)
    {
        const f32x4* q = reinterpret_cast<const f32x4*>(p);
        return NT ? Raw{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)} : Raw{q[0], q[1]};
    }
    static __device__ __forceinline__ void widen(const Raw& r, float (&v)[8])
    {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
    template <bool NT>
    static __device__ __forceinline__ void load8(const float* p, float (&v)[8])
    {
        widen(load_raw<NT>(p), v);
    }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
    template <bool NT = kNtStore>
    static __device__ __forceinline__ void store8(float* p, const float (&v)[8])
    {
        const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        if (NT) {
            __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
            __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
        } else {
            *reinterpret_cast<f32x4*>(p) = a;
            *reinterpret_cast<f32x4*>(p + 4) = b;
        }
    }
    static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};

// fp16 storage (IEEE binary16): widening is exact; narrowing converts one value at a time
// with round-to-nearest-even (the default rounding mode), keeping fp16 subnormals and
// overflowing to infinity. The value is first pinned as an fp32 register: otherwise the
// compiler fuses an fma that produced it with the narrowing (v_fma_mixlo_f16), which rounds
// the exact product-sum to fp16 once, and an fp16 output would no longer be the fp32
// output rounded, wherever the fp32 result is an fp16 midpoint.
__device__ __forceinline__ float pin_f32(float v)
{
    asm("" : "+v"(v));
    return v;
}

template <> struct Io<_Float16> {
    struct Raw {
        u32x4 u;
    };
    static __device__ __forceinline__ float lo(uint32_t w)
    {
        return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xffffu)));
    }
    static __device__ __forceinline__ float hi(uint32_t w)
    {
        return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
    }
    // One packed conversion of the pair (gfx950 converts two fp32 values to fp16 in one
    // instruction, rounding each exactly as the scalar conversion does).
    static __device__ __forceinline__ uint32_t pack(float a, float b)
    {
        const f32x2 v = {pin_f32(a), pin_f32(b)};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    template <bool NT>
    static __device__ __forceinline__ Raw load_raw(const _Float16* p)
    {
        const u32x4* q = reinterpret_cast<const u32x4*>(p);
        return Raw{NT ? __builtin_nontemporal_load(q) : *q};
    }
    static __device__ __forceinline__ void widen(const Raw& r, float (&v)[8])
    {
        v[0] = lo(r.u.x); v[1] = hi(r.u.x);
        v[2] = lo(r.u.y); v[3] = hi(r.u.y);
        v[4] = lo(r.u.z); v[5] = hi(r.u.z);
        v[6] = lo(r.u.w); v[7] = hi(r.u.w);
    }
    template <bool NT>
    static __device__ __forceinline__ void load8(const _Float16* p, float (&v)[8])
    {
        widen(load_raw<NT>(p), v);
    }
    static __device__ __forceinline__ float load1(const _Float16* p) { return float(*p); }
    template <bool NT = kNtStore>
    static __device__ __forceinline__ void store8(_Float16* p, const float (&v)[8])
    {
        u32x4 u;
        u.x = pack(v[0], v[1]);
        u.y = pack(v[2], v[3]);
        u.z = pack(v[4], v[5]);
        u.w = pack(v[6], v[7]);
        if (NT)
            __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
        else
            *reinterpret_cast<u32x4*>(p) = u;
    }
    static __device__ __forceinline__ void store1(_Float16* p, float v) { *p = _Float16(pin_f32(v)); }
};

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

// Lane i receives lane i + OFF's value, for the offsets of the fixed trees below (32, 16,
// 8, 4, 2, 1), in registers rather than through LDS: OFF = 32 and 16 exchange halves and
// rows of the wave (gfx950's v_permlane32_swap and v_permlane16_swap), smaller offsets
// shift within each row of 16 lanes (DPP row_shl). Only lanes i < OFF are guaranteed lane
// i + OFF's value, and only those lanes' results reach lane 0 in the trees. Every lane of
// the wave must be active.
template <int OFF>
__device__ __forceinline__ uint32_t lane_down(uint32_t v)
{
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "tree offset");
    if constexpr (OFF == 32) {
        return __builtin_amdgcn_permlane32_swap(v, v, false, false)[1];
    } else if constexpr (OFF == 16) {
        return __builtin_amdgcn_permlane16_swap(v, v, false, false)[1];
    } else {
        return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x100 | OFF, 0xF, 0xF, false));
    }
}

template <int OFF>
__device__ __forceinline__ float lane_down(float v)
{
    return __uint_as_float(lane_down<OFF>(__float_as_uint(v)));
}

template <int OFF>
__device__ __forceinline__ uint64_t lane_down(uint64_t v)
{
    return (uint64_t(lane_down<OFF>(uint32_t(v >> 32))) << 32) | uint64_t(lane_down<OFF>(uint32_t(v)));
}

template <int OFF, typename CT>
__device__ __forceinline__ void wave_merge_level(Moments<CT>& a)
{
    const CT nb = lane_down<OFF>(a.n);
    const float mb = lane_down<OFF>(a.m);
    const float Mb = lane_down<OFF>(a.M2);
    chan_merge(a, nb, mb, Mb);
}

// Lane 0 ends up with the merge of all 64 lanes, combined in a fixed tree: lane i takes
// lane i + off for off = 32, 16, ..., 1 (left operand always the lower lane).
template <typename CT>
__device__ __forceinline__ void wave_merge(Moments<CT>& a)
{
    wave_merge_level<32>(a);
    wave_merge_level<16>(a);
    wave_merge_level<8>(a);
    wave_merge_level<4>(a);
    wave_merge_level<2>(a);
    wave_merge_level<1>(a);
}

// Lane 0 ends up with the sum of all 64 lanes, in the same tree.
__device__ __forceinline__ float wave_sum(float v)
{
    v = v + lane_down<32>(v);
    v = v + lane_down<16>(v);
    v = v + lane_down<8>(v);
    v = v + lane_down<4>(v);
    v = v + lane_down<2>(v);
    v = v + lane_down<1>(v);
    return v;
}

// Balanced pairwise sum of 2^k values (pairs i, i + half at every level), leaving the
// input intact. A constant input is summed exactly: every addition doubles a value.
template <int N>
__device__ __forceinline__ float tree_sum(const float (&t)[N])
{
    float h[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) h[i] = t[i] + t[i + N / 2];
#pragma unroll
    for (int w = N / 4; w >= 1; w >>= 1) {
#pragma unroll
        for (int i = 0; i < w; ++i) h[i] = h[i] + h[i + w];
    }
    return h[0];
}

// Sum of squares in the same tree shape, first level fused: d_i^2 + d_{i+half}^2.
template <int N>
__device__ __forceinline__ float tree_sumsq(const float (&d)[N])
{
    float h[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) h[i] = fmaf(d[i], d[i], d[i + N / 2] * d[i + N / 2]);
#pragma unroll
    for (int w = N / 4; w >= 1; w >>= 1) {
#pragma unroll
        for (int i = 0; i < w; ++i) h[i] = h[i] + h[i + w];
    }
    return h[0];
}

// Sum of products in the same tree shape, first level fused: a_i b_i + a_{i+half} b_{i+half}.
template <int N>
__device__ __forceinline__ float tree_sumprod(const float (&a)[N], const float (&b)[N])
{
    float h[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) h[i] = fmaf(a[i], b[i], a[i + N / 2] * b[i + N / 2]);
#pragma unroll
    for (int w = N / 4; w >= 1; w >>= 1) {
#pragma unroll
        for (int i = 0; i < w; ++i) h[i] = h[i] + h[i + w];
    }
    return h[0];
}

// Waves of the largest workgroup a fixed-order block reduction serves (512 threads).
constexpr int kMaxWaves = 8;

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

// ------------------------------------------------------------------ resident workgroups

constexpr int kResMaxWaves = kResMaxBlock / 64;

// floor(x / d) for x < 2^16 with the launch's precomputed multiplier for d.
__device__ __forceinline__ uint32_t fdiv(uint32_t x, FastDiv f)
{
    return uint32_t((uint64_t(x) * f.m) >> 32);
}

// The streaming job that workgroup slot w (0 <= w < jobs) of a streaming kernel takes,
// with the order's parameters from set_job_order. With F > 1 (every reduction job is
// exactly F streaming jobs, and the inputs stay in the last-level cache) the slots take
// the last streaming job of every reduction job first, then the second-to-last, and so
// on, so that each pass over x (and dy) runs against the direction of the reduction pass
// before it, whose most recently read lines are the ones the cache still holds, and the
// next reduction pass finds the lines this one read last. The map c*F + (F - 1 - p), over
// c < R = jobs / F and p < F with w = p*R + c, is a permutation of [0, jobs), so the
// results do not depend on it.
__device__ __forceinline__ int64_t permuted_job(int64_t w, int32_t F, int32_t R, int32_t shift, FastDiv divR)
{
    if (F <= 1) return w;
    uint32_t p, c;
    if (shift >= 0) {
        p = uint32_t(w) >> shift;
        c = uint32_t(w) & ((1u << shift) - 1u);
    } else {
        p = fdiv(uint32_t(w), divR);
        c = uint32_t(w) - p * uint32_t(R);
    }
    return int64_t(c) * F + (F - 1 - int64_t(p));
}

// The folded (NCDHW) or streaming (channels-last) jobs' order.
template <typename A>
__device__ __forceinline__ int64_t job_in_order(int64_t w, const A& a)
{
    return permuted_job(w, a.fold_nest, a.fold_R, a.fold_shift, a.div_fold_R);
}

// The one-step streaming jobs' order (NCDHW split-phase and spatial-shard calls).
__device__ __forceinline__ int64_t step_job_in_order(int64_t w, const KArgs& a)
{
    return permuted_job(w, a.step_nest, a.step_R, a.step_shift, a.div_step_R);
}

// Block-wide sums of a and b; waves are added in wave order and every thread returns
// the result. s holds 2 * kResMaxWaves floats and may be reused on return.
__device__ __forceinline__ float2 block_allsum2(float a, float b, float* s)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) { s[wave] = a; s[kResMaxWaves + wave] = b; }
    __syncthreads();
    float ra = s[0], rb = s[kResMaxWaves];
    for (int w = 1; w < nw; ++w) { ra = ra + s[w]; rb = rb + s[kResMaxWaves + w]; }
    __syncthreads();
    return make_float2(ra, rb);
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

inline dim3 grid_of(int64_t jobs) { return dim3(unsigned(jobs < kMaxGrid ? jobs : kMaxGrid)); }

// Calls f with a value of the storage type of dtype dt: float, bf16 (as uint16_t) or fp16.
template <typename F>
hipError_t with_type(int dt, F&& f)
{
    if (dt == kBF16) return f(uint16_t{});
    if (dt == kF16) return f(_Float16{});
    return f(float{});
}

}  // namespace

}  // namespace gn
