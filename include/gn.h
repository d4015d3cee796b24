/*
 * gn.h -- C ABI of libgn.so: 3D GroupNorm forward and backward on MI355X (gfx950).
 *
 * What is computed (cited from the pages the library is built from):
 *   - "Optimize GroupNorm" (LBANN/ScaFFold pull 93), paragraph on ATen's per-(batch,
 *     group) statistics: GroupNorm statistics are taken per (sample n, group g) over
 *     the group's C/G channels and every voxel; y = gamma_c * (x - mu) * rstd + beta_c.
 *   - Same page, paragraph on the independent review: rstd = 1/sqrt(var + eps) with
 *     the biased variance (a single-element group has rstd = 316 at eps = 1e-5, and
 *     its input gradient is exactly zero); mean/rstd are outputs, not differentiable.
 *   - Same page, paragraph introducing the NDHWC Triton kernel: the statistics are fp32;
 *     each tile's mean and squared deviations come from a two-pass form with a correction
 *     term, tiles are combined with Chan's merge of (count, mean, M2), and every sum runs in
 *     registers in one fixed order without floating-point atomics, so repeated calls give
 *     the same bits.
 *   - Same page, paragraph folding seven launches into four: how the work is split (the
 *     launch shapes, the number of partial results per group, the tiles and the order in
 *     which partials are combined) depends on the shape alone. That page also moves the
 *     finalize into the elementwise kernels; gn_forward and gn_backward do the same,
 *     while the split-phase entry points (which must leave the statistics in between)
 *     and the channels-last entry points run it as a small kernel of its own.
 *   - "Preserve GroupNorm dtype" (LBANN/ScaFFold pull 105), first paragraph: everything
 *     up to the output is fp32 arithmetic and the narrowing happens once, in the final
 *     store, so a bf16 output equals the fp32 result rounded a single time; fp32 output
 *     stays available. Second paragraph: the plan takes no dtype, so the backward on the
 *     same values in fp32 and in bf16 gives bitwise identical dx/dgamma/dbeta.
 *
 * Layout. Every tensor argument is contiguous NCDHW: element (n, c, s) of a volume
 * with S = D*H*W voxels lives at flat index (n*C + c)*S + s. Group (n, g) is the
 * contiguous run of M = (C/G)*S elements starting at (n*C + g*C/G)*S. mean and rstd
 * are [N*G] fp32, indexed n*G + g. gamma, beta, dgamma, dbeta are [C] fp32.
 *
 * Ownership and ordering. The caller owns and allocates every buffer, including the
 * workspace (gn_workspace_bytes). The library never allocates device memory (the static
 * scratch array of gn_forward_noalloc is part of its code object), never synchronizes the
 * device or the stream, and never copies device-to-host. All work is
 * enqueued on `stream` (a hipStream_t; NULL means the null stream of the current
 * device) in stream order, and the call returns as soon as it is enqueued. Outputs are
 * fully overwritten (dgamma/dbeta are written, not accumulated). The workspace holds
 * partial results and per-row coefficients from the first half of a direction to its
 * second half (gn_forward_stats -> gn_forward_apply, gn_backward_reduce ->
 * gn_backward_apply); nothing else carries from one call to the next, and it needs no
 * initialization.
 *
 * Pointers. x, y, dy, dx and the workspace must be 16-byte aligned device pointers;
 * mean, rstd, gamma, beta, dgamma, dbeta 4-byte aligned device pointers. All of them
 * must live on one device, the device that owns x: every pointer argument is checked
 * (GN_ERR_DEVICE for host memory, pinned host memory or another device's memory). The
 * kernels are launched on x's device whatever device is current, and a stream that belongs
 * to another device is rejected. Buffer sizes cannot be checked through plain pointers: each
 * must hold the elements stated for it.
 *
 * Errors. Every entry point returns an int status (gn_status). All validation runs
 * before anything is enqueued; on any error other than GN_ERR_LAUNCH nothing has been
 * enqueued and no output is touched. After GN_ERR_LAUNCH outputs are undefined.
 * Nothing is thrown across the ABI and no state is kept between calls, apart from the
 * contents of gn_forward_noalloc's scratch.
 */
#ifndef GN_H
#define GN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of x, y, dy, dx. gamma, beta, mean, rstd, dgamma, dbeta are always fp32. */
typedef enum gn_dtype {
    GN_F32 = 0,  /* IEEE binary32 */
    GN_BF16 = 1, /* bfloat16: the upper 16 bits of a binary32 */
    GN_F16 = 2   /* IEEE binary16 ("Optimize GroupNorm", NDHWC-kernel paragraph: fp32, bf16
                    and fp16 inputs with fp32 statistics) */
} gn_dtype;

typedef enum gn_status {
    GN_OK = 0,
    GN_ERR_NULL = 1,      /* a required pointer is NULL */
    GN_ERR_SHAPE = 2,     /* N, C, S or G <= 0, N*(C/G)*S == 1, or N*C*S too large */
    GN_ERR_GROUPS = 3,    /* C is not a multiple of G */
    GN_ERR_DTYPE = 4,     /* unsupported dtype or dtype combination */
    GN_ERR_EPS = 5,       /* eps is negative or not finite */
    GN_ERR_WORKSPACE = 6, /* workspace smaller than gn_workspace_bytes(N, C, S, G) */
    GN_ERR_ALIGN = 7,     /* a pointer is not aligned as stated above */
    GN_ERR_DEVICE = 8,    /* a pointer argument is not device memory of x's device, or the
                             stream belongs to another device */
    GN_ERR_LAUNCH = 9,    /* the HIP runtime refused a launch; outputs are undefined */
    GN_ERR_ACTIVATION = 10, /* unknown activation code */
    GN_ERR_LAYOUT = 11,     /* channels-last: C not a multiple of 8, C/8 not dividing 256, or
                               C/G neither dividing 8 nor a multiple of 8 */
    GN_ERR_SCRATCH = 12     /* gn_forward_noalloc: gn_workspace_bytes(N, C, S, G) exceeds
                               GN_NOALLOC_SCRATCH_BYTES */
} gn_status;

/*
 * Activation applied after the affine, inside the normalize store ("Optimize GroupNorm",
 * paragraphs on the rung ladder with the fused ReLU and on the NaN-correct ReLU):
 * relu(v) = 0 where v < 0, else v (NaN, +Inf and -0.0 pass unchanged, -Inf becomes 0), as
 * torch's F.relu; in the backward the gradient is blocked where relu(pre) <= 0 and passes
 * otherwise (NaN too), pre being the affine output recomputed in fp32 from x.
 */
typedef enum gn_activation {
    GN_ACT_NONE = 0,
    GN_ACT_RELU = 1
} gn_activation;

/*
 * Workspace size in bytes for a volume of N samples, C channels, S = D*H*W voxels and
 * G groups. A pure function of the shape (no dtype, no device). Returns 0 for a shape
 * that gn_forward would reject. One workspace of this size serves gn_forward and
 * gn_backward alike (they may share it when they are stream-ordered).
 */
size_t gn_workspace_bytes(int64_t N, int64_t C, int64_t S, int64_t G);

/*
 * Forward. Statistics per (n, g) in fp32 (written to mean and rstd), then
 * y = act(gamma_c * (x - mean) * rstd + beta_c) computed in fp32 and stored once in
 * y_dtype. x_dtype is GN_F32, GN_BF16 or GN_F16; y_dtype is x_dtype or GN_F32 (the fp32-output
 * mode). gamma == NULL means all ones, beta == NULL all zeros. eps must be finite and
 * >= 0. activation is a gn_activation. Two kernels: the partial statistics, then the
 * normalize with the finalize folded into each of its workgroups ("Optimize GroupNorm",
 * paragraph folding seven launches into four); mean, rstd and y are bitwise those of
 * gn_forward_stats followed by gn_forward_apply (three kernels), which compute the same
 * merge in the same order.
 */
int gn_forward(const void* x, int x_dtype, const float* gamma, const float* beta,
               int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
               void* y, int y_dtype, float* mean, float* rstd,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * First half of gn_forward: fp32 partial statistics of x, merged in a fixed order into
 * mean and rstd, plus per-row normalize coefficients left in the workspace for
 * gn_forward_apply. Two kernels.
 */
int gn_forward_stats(const void* x, int x_dtype, const float* gamma, const float* beta,
                     int64_t N, int64_t C, int64_t S, int64_t G, float eps,
                     float* mean, float* rstd,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second half of gn_forward: writes y from x and the coefficients that gn_forward_stats
 * left in the workspace (same x, same shape, stream-ordered after it). One kernel.
 */
int gn_forward_apply(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                     int activation, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward. Recomputes xhat = (x - mean) * rstd from the mean/rstd gn_forward wrote,
 * reduces sum(dy) and sum(dy * xhat) per (n, c) in a fixed order, then writes
 *   dx = rstd * (gamma_c * dy - c1 - xhat * c2),  c1 = (1/M) sum_{c in g} gamma_c sum(dy),
 *                                                 c2 = (1/M) sum_{c in g} gamma_c sum(dy*xhat)
 * in x_dtype, and dgamma_c = sum_n sum(dy * xhat), dbeta_c = sum_n sum(dy).
 * dy_dtype is GN_F32, GN_BF16 or GN_F16 independently of x_dtype; the same dy values in any
 * dtype give bitwise identical results. gamma == NULL means all ones. dx, dgamma and
 * dbeta may each be NULL (not computed). A group with M == 1 has dx == +0 exactly for
 * finite inputs (NaN/Inf still propagate). With activation GN_ACT_RELU, dy is the gradient
 * of the relu's output and is gated as stated above before all of this (beta, NULL for
 * zeros, is then needed to recompute the pre-activation; it is ignored otherwise).
 * With dx, two kernels: the per-job sums, then dx with the finalize (c1, c2, and dgamma,
 * dbeta) folded in; without dx, gn_backward_reduce alone. The results are bitwise those
 * of gn_backward_reduce followed by gn_backward_apply (three kernels).
 */
int gn_backward(const void* dy, int dy_dtype, const void* x, int x_dtype,
                const float* mean, const float* rstd, const float* gamma,
                const float* beta, int activation,
                int64_t N, int64_t C, int64_t S, int64_t G,
                void* dx, float* dgamma, float* dbeta,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * First half of gn_backward: per-job fp32 sums of dy and dy*xhat, merged in a fixed
 * order into dgamma/dbeta (either may be NULL) and per-row dx coefficients left in the
 * workspace for gn_backward_apply. Two kernels.
 */
int gn_backward_reduce(const void* dy, int dy_dtype, const void* x, int x_dtype,
                       const float* mean, const float* rstd, const float* gamma,
                       const float* beta, int activation,
                       int64_t N, int64_t C, int64_t S, int64_t G,
                       float* dgamma, float* dbeta,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second half of gn_backward: writes dx from x, dy and the coefficients that
 * gn_backward_reduce left in the workspace (same inputs, stream-ordered after it).
 * One kernel.
 */
int gn_backward_apply(const void* dy, int dy_dtype, const void* x, int x_dtype,
                      int64_t N, int64_t C, int64_t S, int64_t G, int activation, void* dx,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gn_forward for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. Same arguments,
 * semantics, results (bitwise those of gn_forward) and errors, without the workspace: the
 * library's own static scratch array of GN_NOALLOC_SCRATCH_BYTES per device serves as the
 * workspace. Shapes whose gn_workspace_bytes exceeds that size return GN_ERR_SCRATCH before
 * anything is enqueued. The call allocates nothing. Every call on one device shares that
 * device's scratch, which keeps the last call's contents: calls that overlap on one device
 * (two streams at once, or a graph replayed beside another call) race, and must be ordered
 * by the caller. Nothing in the scratch needs to start at zero.
 */
#define GN_NOALLOC_SCRATCH_BYTES (1u << 20)

int gn_forward_noalloc(const void* x, int x_dtype, const float* gamma, const float* beta,
                       int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                       void* y, int y_dtype, float* mean, float* rstd, void* stream);

/*
 * The two launches of gn_forward as two calls, stream-ordered on one workspace, so that
 * each can be timed or overlapped on its own; together they are bitwise gn_forward.
 * gn_forward_partials leaves the partial statistics of x in the workspace (one kernel);
 * gn_forward_finish takes gn_forward's arguments, merges them and writes mean, rstd and y
 * (one kernel). On shapes that gn_plan_query reports resident_forward for, the first call
 * enqueues nothing and the second runs the whole forward. Errors as gn_forward.
 */
int gn_forward_partials(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                        void* workspace, size_t workspace_bytes, void* stream);

int gn_forward_finish(const void* x, int x_dtype, const float* gamma, const float* beta,
                      int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                      void* y, int y_dtype, float* mean, float* rstd,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two launches of gn_backward, likewise: gn_backward_partials leaves the per-job sums
 * of dy and dy*xhat in the workspace; gn_backward_finish takes gn_backward's arguments and
 * writes dx, dgamma and dbeta (each may be NULL; with dx NULL it runs the finalize alone).
 * Together they are bitwise gn_backward; resident_backward shapes as above.
 */
int gn_backward_partials(const void* dy, int dy_dtype, const void* x, int x_dtype,
                         const float* mean, const float* rstd, const float* gamma,
                         const float* beta, int activation,
                         int64_t N, int64_t C, int64_t S, int64_t G,
                         void* workspace, size_t workspace_bytes, void* stream);

int gn_backward_finish(const void* dy, int dy_dtype, const void* x, int x_dtype,
                       const float* mean, const float* rstd, const float* gamma,
                       const float* beta, int activation,
                       int64_t N, int64_t C, int64_t S, int64_t G,
                       void* dx, float* dgamma, float* dbeta,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Static English description of a status code (never NULL). */
const char* gn_status_string(int status);

/*
 * The launch plan for a shape: a pure function of (N, C, S, G) with no dtype and no
 * device input, exposed so that tests and benchmarks can see the decomposition. The
 * reductions work on jobs: reduction job j covers elements
 * [k*chunk, min((k+1)*chunk, S)) of row r = j / chunks_per_row (row r = n*C + c),
 * k = j % chunks_per_row, and leaves one fp32 partial; their number and length fix the
 * reduction order. The streaming kernels of the split-phase entry points (normalize, dx)
 * cover the rows the same way with apply_chunk and apply_chunks_per_row, and those of
 * gn_forward / gn_backward, which merge their group's partials first, with fold_chunk
 * and fold_chunks_per_row (256 threads each); neither reduces anything that is stored.
 */
typedef struct gn_plan_info {
    int64_t rows;                 /* N*C */
    int64_t chunk;                /* elements per reduction job (a row's last may be shorter) */
    int64_t chunks_per_row;       /* reduction jobs per row */
    int64_t jobs;                 /* rows * chunks_per_row: workgroups of a reduction launch */
    int64_t partials_per_group;   /* (C/G) * chunks_per_row */
    int32_t block;                /* threads per reduction workgroup (64, 128 or 256) */
    int32_t vectors_per_step;     /* 8-element vectors each reduction thread loads per step */
    int64_t apply_chunk;          /* elements per streaming job */
    int64_t apply_chunks_per_row; /* streaming jobs per row */
    int64_t apply_jobs;           /* rows * apply_chunks_per_row: workgroups of a streaming launch */
    int32_t apply_block;          /* threads per streaming workgroup */
    int32_t apply_vectors;        /* 8-element vectors each streaming thread moves */
    size_t workspace_bytes;       /* == gn_workspace_bytes */
    /* Resident path (S a multiple of 8 and a small enough group): the forward runs one
     * workgroup per group (n, g), the backward one per g covering all N samples; each
     * holds its elements in registers from the single read to the write. */
    int32_t resident_forward;     /* 1 if the forward takes the resident path */
    int32_t resident_backward;    /* 1 if the backward takes the resident path */
    int32_t resident_block_forward, resident_vectors_forward;    /* threads, vectors per thread */
    int32_t resident_block_backward, resident_vectors_backward;
    int64_t fold_chunk;           /* elements per streaming job with the finalize folded in */
    int64_t fold_chunks_per_row;
    int64_t fold_jobs;            /* rows * fold_chunks_per_row */
    /* Resident backward over N > 1 samples split into one workgroup per (n, g): each also
     * sums the other samples' rows of its channels i (i mod N == n), so that dgamma and
     * dbeta keep the bits of the one-workgroup-per-g form. */
    int32_t resident_backward_split;
} gn_plan_info;

/* Fills *out for a valid shape and returns GN_OK; otherwise returns the shape error. */
int gn_plan_query(int64_t N, int64_t C, int64_t S, int64_t G, gn_plan_info* out);

/*
 * Channels-last (NDHWC) activations ("Optimize GroupNorm", paragraph introducing the NDHWC
 * kernel): x, y, dy and dx hold element (n, s, c) at flat index (n*S + s)*C + c; mean,
 * rstd, gamma, beta, dgamma and dbeta are laid out as above. Same arguments, dtypes,
 * semantics, ownership and errors as gn_forward / gn_backward, with the workspace of
 * gn_workspace_bytes_cl. Supported when C is a multiple of 8, C/8 divides 256 (C <= 2048)
 * and C/G divides 8 or is a multiple of 8 (every UNet shape); other shapes return
 * GN_ERR_LAYOUT before anything is enqueued. Three kernels per direction, or one on the
 * resident path that gn_plan_query_cl reports.
 */
size_t gn_workspace_bytes_cl(int64_t N, int64_t C, int64_t S, int64_t G);

int gn_forward_cl(const void* x, int x_dtype, const float* gamma, const float* beta,
                  int64_t N, int64_t C, int64_t S, int64_t G, float eps, int activation,
                  void* y, int y_dtype, float* mean, float* rstd,
                  void* workspace, size_t workspace_bytes, void* stream);

int gn_backward_cl(const void* dy, int dy_dtype, const void* x, int x_dtype,
                   const float* mean, const float* rstd, const float* gamma,
                   const float* beta, int activation,
                   int64_t N, int64_t C, int64_t S, int64_t G,
                   void* dx, float* dgamma, float* dbeta,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * The channels-last plan. A reduction job is chunk voxels of one sample (jobs_per_sample
 * per sample; the last may be shorter); lane t of a workgroup of `block` threads owns the
 * channel vector t mod (C/8) and voxel t / (C/8) + r * voxels_per_round of round r
 * (rounds_per_step rounds per reduction step, apply_rounds per streaming job).
 */
typedef struct gn_plan_info_cl {
    int64_t chunk;                /* voxels per reduction job */
    int64_t jobs_per_sample;
    int64_t jobs;                 /* N * jobs_per_sample */
    int64_t voxels_per_round;     /* block / (C/8) */
    int64_t apply_chunk;          /* voxels per streaming job */
    int64_t apply_jobs_per_sample;
    int64_t apply_jobs;
    int32_t block;                /* threads per workgroup */
    int32_t rounds_per_step;
    int32_t apply_rounds;
    int32_t groups_per_vector;    /* max(1, 8 / (C/G)) */
    size_t workspace_bytes;       /* == gn_workspace_bytes_cl */
    /* Resident path (C/G a multiple of 8 with C/(8G) a power of two up to 8, and a small
     * enough group): one workgroup per group (n, g) forward and per g over all N samples
     * backward, holding its elements in registers; one kernel per direction. */
    int32_t resident_forward, resident_backward;
    int32_t resident_block_forward, resident_vectors_forward;
    int32_t resident_block_backward, resident_vectors_backward;
} gn_plan_info_cl;

int gn_plan_query_cl(int64_t N, int64_t C, int64_t S, int64_t G, gn_plan_info_cl* out);

/*
 * Spatial shards ("Optimize GroupNorm", DistConv paragraphs: activations split over GPUs
 * along D/H/W, each shard normalized with its own statistics, global statistics left
 * open). With these calls a rank holding a shard (a contiguous NCDHW tensor of S voxels
 * per row, the same N, C, G on every rank) normalizes with the statistics of the whole
 * volume:
 *   forward:  gn_forward_shard_stats (this shard's record per group)
 *             -> the caller gathers all P shards' records, [P][N*G], in shard order
 *             -> gn_forward_shard_merge (mean, rstd; coefficients into the workspace)
 *             -> gn_forward_apply on this shard;
 *   backward: gn_backward_shard_sums (this shard's (s1, s2) per row, with the global mean
 *             and rstd) -> the caller gathers [P][N*C] -> gn_backward_shard_merge (dgamma,
 *             dbeta over the whole volume; dx coefficients into the workspace)
 *             -> gn_backward_apply on this shard.
 * The merges run the same fixed-order computation on every rank, so all ranks obtain
 * bitwise identical mean, rstd, dgamma and dbeta. The workspace is this shard's
 * (gn_workspace_bytes(N, C, S, G)). A record holds a group's element count in 32 bits, so
 * (C/G) * S must be below 2^32. A shard is a volume in its own right for validation (so
 * N * (C/G) * S == 1 is rejected), but its piece of a group may be a single element: the
 * backward merge records whether the whole group is one, and gn_backward_apply answers
 * dx = 0 only then. Device pointers; moments and sums 16- and 8-byte aligned.
 */
typedef struct gn_moments {
    float mean_hi;   /* the shard's group mean as mean_hi + mean_lo */
    float mean_lo;
    float m2;        /* sum of squared deviations from that mean */
    uint32_t count;  /* elements of the group in the shard */
} gn_moments;

int gn_forward_shard_stats(const void* x, int x_dtype, int64_t N, int64_t C, int64_t S, int64_t G,
                           gn_moments* moments /* [N*G] */,
                           void* workspace, size_t workspace_bytes, void* stream);

int gn_forward_shard_merge(const gn_moments* moments /* [P][N*G] */, int64_t P,
                           const float* gamma, const float* beta,
                           int64_t N, int64_t C, int64_t S, int64_t G, float eps,
                           float* mean, float* rstd,
                           void* workspace, size_t workspace_bytes, void* stream);

int gn_backward_shard_sums(const void* dy, int dy_dtype, const void* x, int x_dtype,
                           const float* mean, const float* rstd, const float* gamma,
                           const float* beta, int activation,
                           int64_t N, int64_t C, int64_t S, int64_t G,
                           float* sums /* [N*C][2] */,
                           void* workspace, size_t workspace_bytes, void* stream);

int gn_backward_shard_merge(const float* sums /* [P][N*C][2] */, int64_t P,
                            const float* mean, const float* rstd, const float* gamma,
                            const float* beta,
                            int64_t N, int64_t C, int64_t S, int64_t S_total, int64_t G,
                            float* dgamma, float* dbeta,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ABI version of this header (incremented on any incompatible change); gn_abi_version()
 * returns the version the library was built with, so a caller can check that the two
 * agree before the first call. */
#define GN_ABI_VERSION 11
int gn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GN_H */
