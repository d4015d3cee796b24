// probe_kernels.hip -- measurement kernels built into libgn_probe.so, beside libgn.so and
// not part of it. Two kinds:
//
//  - Streaming probes: a read stream, a write fill and a copy over a device buffer, with
//    plain or nontemporal loads and stores. They move bytes and do nothing else, so their
//    rates are the HBM rates the device delivers for pure reads, pure writes and a 1:1 mix;
//    the GroupNorm kernels' times are compared with the bound those rates give for each
//    kernel's own mix of reads and writes.
//  - A negative control for the determinism tests: per-group sums of a bf16 volume in which
//    each workgroup reduces its job in a fixed order and then adds its partial to the
//    group's total with a global atomic add, so the partials are combined in the order the
//    workgroups happen to finish. Run twice on the same input it can give different bits,
//    which is what a bitwise-reproducibility check has to be able to detect ("Make loss
//    calculation deterministic and sync-free", first paragraph: atomically ordered sums
//    drift between identical calls). libgn.so itself has no atomics.
//
// C ABI (all pointers are device pointers; `stream` is a hipStream_t, NULL for the null
// stream; every function returns 0 on success, 1 for arguments it rejects before launching
// anything, 2 when the runtime refuses the launch):
//   int gnp_read (const void* src, size_t bytes, int nontemporal, int vecs, uint32_t magic,
//                 uint32_t* sink, int64_t grid, void* stream);
//       reads `bytes` (a multiple of 16 * 256 * vecs) once; sink[0..63] is written only by
//       a lane whose xor of everything it read equals `magic` (so the loads cannot be
//       dropped; pass a value the data cannot produce and sink stays untouched).
//   int gnp_write(void* dst, size_t bytes, int nontemporal, int vecs, uint32_t value,
//                 int64_t grid, void* stream);
//       fills `bytes` with the 32-bit `value`.
//   int gnp_copy (const void* src, void* dst, size_t bytes, int nontemporal_loads,
//                 int nontemporal_stores, int vecs, int64_t grid, void* stream);
//   `vecs` (2, 4, 8 or 16) is the number of 16-byte vectors each lane has in flight per
//   tile; workgroups (256 threads) stride over the tiles, `grid` of them.
//   int gnp_atomic_group_sums(const uint16_t* x_bf16, int64_t groups, int64_t group_elems,
//                             int64_t chunk, float* sums, void* stream);
//       sums[g] = sum of the group's bf16 values, g < groups, each group `group_elems`
//       contiguous elements split into jobs of `chunk` elements (chunk a multiple of 2048
//       dividing group_elems); zeroes sums first, then accumulates with atomic adds.
//   int gnp_barrier(int64_t grid, int group, int rounds, int kind, uint32_t* counters,
//                   int* failed, void* stream);
//       the cost of cross-workgroup synchronization: `grid` workgroups (256 threads),
//       launched cooperatively so that all are resident at once, pass `rounds` barriers.
//       kind 0: no barrier (the launch alone); 1: the grid-wide barrier of cooperative
//       groups; 2: a barrier among each `group` consecutive workgroups on a counter per
//       group (device-scope atomic add, then polling with device-scope atomic loads between
//       a release and an acquire fence); 3: the same without the fences. counters holds
//       grid / group zeroed words (the call zeroes them); a wait that polls more than 2^22
//       times gives up, sets *failed and leaves, so every wave ends.
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeBlock = 256;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p)
{
    return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v)
{
    if (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Tile t covers vectors [t * 256 * V, (t + 1) * 256 * V); lane `tid` takes vectors
// tid, tid + 256, ... of it, so every load and store instruction of a wave is one contiguous
// 1 KiB. Workgroups stride over the tiles.
template <int V, bool NT>
__global__ void __launch_bounds__(kProbeBlock)
read_kernel(const u32x4* __restrict__ src, int64_t tiles, uint32_t magic, uint32_t* __restrict__ sink)
{
    const int tid = threadIdx.x;
    uint32_t acc = 0;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const u32x4* p = src + t * (kProbeBlock * V) + tid;
        u32x4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) v[u] = ld<NT>(p + u * kProbeBlock);
#pragma unroll
        for (int u = 0; u < V; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == magic) sink[tid & 63] = acc;
}

template <int V, bool NT>
__global__ void __launch_bounds__(kProbeBlock)
write_kernel(u32x4* __restrict__ dst, int64_t tiles, uint32_t value)
{
    const int tid = threadIdx.x;
    const u32x4 v = {value, value, value, value};
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        u32x4* p = dst + t * (kProbeBlock * V) + tid;
#pragma unroll
        for (int u = 0; u < V; ++u) st<NT>(p + u * kProbeBlock, v);
    }
}

template <int V, bool NTL, bool NTS>
__global__ void __launch_bounds__(kProbeBlock)
copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t tiles)
{
    const int tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t o = t * (kProbeBlock * V) + tid;
        u32x4 v[V];
#pragma unroll
        for (int u = 0; u < V; ++u) v[u] = ld<NTL>(src + o + u * kProbeBlock);
#pragma unroll
        for (int u = 0; u < V; ++u) st<NTS>(dst + o + u * kProbeBlock, v[u]);
    }
}

// Calls f with std::integral_constant<int, V> for V in {2, 4, 8, 16}; -1 for other values.
template <typename F>
int with_vecs(int vecs, F&& f)
{
    switch (vecs) {
        case 2: return f(std::integral_constant<int, 2>{});
        case 4: return f(std::integral_constant<int, 4>{});
        case 8: return f(std::integral_constant<int, 8>{});
        case 16: return f(std::integral_constant<int, 16>{});
        default: return -1;
    }
}

int64_t tile_bytes(int vecs) { return int64_t(16) * kProbeBlock * vecs; }

// ------------------------------------------------------------------ negative control

__global__ void zero_kernel(float* __restrict__ p, int64_t n)
{
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// One workgroup per job of `chunk` elements of one group: lane t sums its 8-element vectors
// t, t + 256, ... in order, the wave in a fixed shuffle tree, the waves in order through
// LDS; then thread 0 adds the job's partial to sums[group] atomically.
__global__ void __launch_bounds__(kProbeBlock)
atomic_sums_kernel(const uint16_t* __restrict__ x, int64_t group_elems, int64_t chunk, int64_t jobs_per_group,
                   float* __restrict__ sums)
{
    __shared__ float s_w[kProbeBlock / 64];
    const int tid = threadIdx.x;
    const int64_t j = blockIdx.x;
    const int64_t g = j / jobs_per_group, k = j - g * jobs_per_group;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + g * group_elems + k * chunk);
    const int64_t nvec = chunk / 8;
    float s = 0.0f;
    for (int64_t v = tid; v < nvec; v += kProbeBlock) {
        const u32x4 w = p[v];
        const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) s = (s + __uint_as_float(e[i] << 16)) + __uint_as_float(e[i] & 0xffff0000u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_down(s, off);
    if ((tid & 63) == 0) s_w[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        float r = s_w[0];
        for (int w = 1; w < kProbeBlock / 64; ++w) r = r + s_w[w];
        atomicAdd(sums + g, r);
    }
}

// ------------------------------------------------------------------ barrier cost

constexpr int kSpinLimit = 1 << 22;

template <int KIND>
__global__ void __launch_bounds__(kProbeBlock)
barrier_kernel(int group, int rounds, uint32_t* __restrict__ counters, int* __restrict__ failed)
{
    const int g = blockIdx.x / group;
    for (int r = 0; r < rounds; ++r) {
        if (KIND == 1) {
            cooperative_groups::this_grid().sync();
        } else if (KIND >= 2) {
            __syncthreads();
            if (threadIdx.x == 0) {
                if (KIND == 2) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_fetch_add(counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t target = uint32_t(group) * uint32_t(r + 1);
                int spins = 0;
                while (__hip_atomic_load(counters + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                    if (++spins > kSpinLimit) {
                        __hip_atomic_store(failed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (KIND == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
        }
    }
}

int status(hipError_t e) { return e == hipSuccess ? 0 : 2; }

unsigned grid_for(int64_t grid, int64_t tiles)
{
    const int64_t g = grid < tiles ? grid : tiles;
    return unsigned(g < 1 ? 1 : g);
}

}  // namespace

extern "C" {

int gnp_read(const void* src, size_t bytes, int nontemporal, int vecs, uint32_t magic, uint32_t* sink,
             int64_t grid, void* stream)
{
    if (!src || !sink || bytes == 0 || grid < 1 || vecs < 1 || bytes % tile_bytes(vecs) != 0) return 1;
    const int64_t tiles = int64_t(bytes / tile_bytes(vecs));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* s = static_cast<const u32x4*>(src);
    const int rc = with_vecs(vecs, [&](auto v) {
        constexpr int V = decltype(v)::value;
        if (nontemporal)
            read_kernel<V, true><<<grid_for(grid, tiles), kProbeBlock, 0, st>>>(s, tiles, magic, sink);
        else
            read_kernel<V, false><<<grid_for(grid, tiles), kProbeBlock, 0, st>>>(s, tiles, magic, sink);
        return status(hipGetLastError());
    });
    return rc < 0 ? 1 : rc;
}

int gnp_write(void* dst, size_t bytes, int nontemporal, int vecs, uint32_t value, int64_t grid, void* stream)
{
    if (!dst || bytes == 0 || grid < 1 || vecs < 1 || bytes % tile_bytes(vecs) != 0) return 1;
    const int64_t tiles = int64_t(bytes / tile_bytes(vecs));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    u32x4* d = static_cast<u32x4*>(dst);
    const int rc = with_vecs(vecs, [&](auto v) {
        constexpr int V = decltype(v)::value;
        if (nontemporal)
            write_kernel<V, true><<<grid_for(grid, tiles), kProbeBlock, 0, st>>>(d, tiles, value);
        else
            write_kernel<V, false><<<grid_for(grid, tiles), kProbeBlock, 0, st>>>(d, tiles, value);
        return status(hipGetLastError());
    });
    return rc < 0 ? 1 : rc;
}

int gnp_copy(const void* src, void* dst, size_t bytes, int nontemporal_loads, int nontemporal_stores, int vecs,
             int64_t grid, void* stream)
{
    if (!src || !dst || bytes == 0 || grid < 1 || vecs < 1 || bytes % tile_bytes(vecs) != 0) return 1;
    const int64_t tiles = int64_t(bytes / tile_bytes(vecs));
    const unsigned g = grid_for(grid, tiles);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    const int rc = with_vecs(vecs, [&](auto v) {
        constexpr int V = decltype(v)::value;
        if (nontemporal_loads && nontemporal_stores)
            copy_kernel<V, true, true><<<g, kProbeBlock, 0, st>>>(s, d, tiles);
        else if (nontemporal_loads)
            copy_kernel<V, true, false><<<g, kProbeBlock, 0, st>>>(s, d, tiles);
        else if (nontemporal_stores)
            copy_kernel<V, false, true><<<g, kProbeBlock, 0, st>>>(s, d, tiles);
        else
            copy_kernel<V, false, false><<<g, kProbeBlock, 0, st>>>(s, d, tiles);
        return status(hipGetLastError());
    });
    return rc < 0 ? 1 : rc;
}

int gnp_atomic_group_sums(const uint16_t* x_bf16, int64_t groups, int64_t group_elems, int64_t chunk,
                          float* sums, void* stream)
{
    if (!x_bf16 || !sums || groups < 1 || chunk < 2048 || chunk % 2048 != 0 || group_elems < chunk ||
        group_elems % chunk != 0 || reinterpret_cast<uintptr_t>(x_bf16) % 16 != 0)
        return 1;
    const int64_t jobs_per_group = group_elems / chunk;
    const int64_t jobs = groups * jobs_per_group;
    if (jobs > (int64_t(1) << 31) - 1) return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    zero_kernel<<<unsigned((groups + 255) / 256), 256, 0, st>>>(sums, groups);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return 2;
    atomic_sums_kernel<<<unsigned(jobs), kProbeBlock, 0, st>>>(x_bf16, group_elems, chunk, jobs_per_group, sums);
    return status(hipGetLastError());
}

int gnp_barrier(int64_t grid, int group, int rounds, int kind, uint32_t* counters, int* failed, void* stream)
{
    if (grid < 1 || grid > 65536 || group < 1 || grid % group != 0 || rounds < 0 || kind < 0 || kind > 3 ||
        !counters || !failed)
        return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemsetAsync(counters, 0, size_t(grid / group) * sizeof(uint32_t), st) != hipSuccess) return 2;
    void* args[] = {&group, &rounds, &counters, &failed};
    const void* k = kind == 0 ? reinterpret_cast<const void*>(barrier_kernel<0>)
                  : kind == 1 ? reinterpret_cast<const void*>(barrier_kernel<1>)
                  : kind == 2 ? reinterpret_cast<const void*>(barrier_kernel<2>)
                              : reinterpret_cast<const void*>(barrier_kernel<3>);
    return status(hipLaunchCooperativeKernel(k, dim3(unsigned(grid)), dim3(kProbeBlock), args, 0, st));
}

}  // extern "C"
