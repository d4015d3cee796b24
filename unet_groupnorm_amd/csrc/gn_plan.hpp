// gn_plan.hpp -- launch plan for the GroupNorm kernels: a pure function of the shape.
//
// "Optimize GroupNorm" (LBANN/ScaFFold pull 93), paragraph folding seven launches into
// four: the way the work is split -- launch shapes, partials per group, tiles and the
// order partials are combined in -- is decided by the shape and nothing else; "Preserve
// GroupNorm dtype" (pull 105), second paragraph: the plan takes no dtype, which is what
// makes the fp32 and bf16 backward bitwise identical.
//
// Two decompositions of the volume, both into "jobs" that are contiguous runs of one
// row (row = n*C + c):
//   - reduction jobs (statistics, backward sums): few and long, one fp32 partial each;
//     their count and length fix the reduction order;
//   - streaming jobs (normalize, dx): one short step each, so that the grid is large
//     and every workgroup moves a few KiB and retires. They reduce nothing, so their
//     shape can change without moving a bit.
// Small groups whose rows are whole 8-element vectors take the resident path instead: one
// workgroup holds a group (forward) or a group across all samples (backward) in registers
// from the single read to the write, one launch per direction.
//
// This unit is plain C++ (no HIP), so it is exercised on a host without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

namespace gn {

// Elements per lane vector: one 16-byte load of bf16, two of fp32. The element -> lane
// assignment is defined in these units, so it is the same for both dtypes.
constexpr int kVec = 8;
// Largest reduction workgroup (threads); the plan sizes smaller ones to short rows.
constexpr int kRedBlock = 256;
// Vectors each lane holds per step of a reduction job (register tile = kVec * kStepVecs).
constexpr int kStepVecs = 4;
// Reduction workgroups a launch aims for (512: 2 per CU on the 256 CUs of an MI355X), and
// the job length (elements) for which it settles for half as many, but at least 256 (one
// per CU). Measured on MI355X, bf16, fwd+bwd steps: against 2048 jobs, 512 is 1-2% faster
// at 128^3-256^3 and 10% at 96^3 (C=32), and fewer, longer jobs also shorten the folded
// kernels' partials merge; 256 jobs of 256K elements are another 1.5% at 128^3 (C=32), while
// 256 jobs are 1-11% slower at 256^3, at 2x128^3 and at the 32^3 UNet site.
constexpr int64_t kTargetJobs = 512;
constexpr int64_t kLongChunk = 262144;
constexpr int64_t kMinJobs = 256;
// Vectors each lane moves in a one-step streaming job (split-phase and spatial-shard calls).
// Measured on one rank's share of the 256^3 site split in 8: 1 vector 187.3 us a step,
// 2 vectors 176.0, 4 vectors 181.2.
constexpr int kApplyVecs = 2;
// Resident path: one workgroup holds a whole group in registers (at most kResMaxBlock
// threads with kResMaxLaneVecs vectors each).
constexpr int kResMaxBlock = 1024;
constexpr int kResMaxLaneVecs = 4;
constexpr int64_t kResMaxVecs = int64_t(kResMaxBlock) * kResMaxLaneVecs;  // 32768 elements
// Elements per job of the streaming kernels that run the finalize themselves (gn_forward,
// gn_backward with dx): each such workgroup first merges its group's partials, so its job
// is long enough to amortize that and short enough that the grid stays large (measured on
// MI355X, bf16, 128^3 and 256^3 with C=32 and the 32^3-64^3 UNet sites: 8192-12288 best;
// 4096 about 20% slower, 32768 and more up to 9% slower at 256^3).
constexpr int64_t kFoldChunk = 8192;
// Upper bound on a reduction job's element count (in-job counts stay within 32 bits).
constexpr int64_t kMaxChunk = int64_t(1) << 30;
// Upper bound on N*C*S accepted (indices stay far from int64 overflow).
constexpr int64_t kMaxNumel = int64_t(1) << 48;

struct Plan {
    int64_t N = 0, C = 0, S = 0, G = 0;
    int64_t Cg = 0;      // channels per group
    int64_t M = 0;       // elements per group
    int64_t rows = 0;    // N * C
    // reduction jobs
    int64_t chunk = 0;   // elements per job
    int64_t K = 0;       // jobs per row
    int64_t jobs = 0;    // rows * K
    int64_t P = 0;       // partials per group = Cg * K
    int block = 0;       // threads per workgroup
    // streaming jobs
    int64_t chunk_a = 0;
    int64_t K_a = 0;
    int64_t jobs_a = 0;
    int block_a = 0;
    // streaming jobs of the kernels with the finalize folded in (256 threads each)
    int64_t chunk_f = 0;
    int64_t K_f = 0;
    int64_t jobs_f = 0;
    // resident path (one workgroup per group; every row a whole number of vectors):
    // forward per group (n, g), backward per g across all samples
    bool res_fwd = false, res_bwd = false;
    int res_block_f = 0, res_vecs_f = 0;   // threads, vectors per lane (1, 2 or 4)
    int res_block_b = 0, res_vecs_b = 0;
    // backward split over samples (N > 1): one workgroup per (n, g) instead of per g, which
    // also sums the rows of the other samples for its share of the group's channels
    // (channels i with i mod N == n), so that dgamma/dbeta still come from one workgroup
    bool res_bwd_split = false;
    // workspace: [partials: float2 * jobs][row coefficients: 2 float4 * rows], 256-byte aligned
    size_t ws_coef_offset = 0;
    size_t ws_bytes = 0;
};

// Returns 0 and fills *p for a valid shape, else a gn_status shape error code
// (2 = GN_ERR_SHAPE, 3 = GN_ERR_GROUPS).
int make_plan(int64_t N, int64_t C, int64_t S, int64_t G, Plan* p);

// Channels-last (NDHWC: x[n][s][c] at (n*S + s)*C + c). Every voxel is C/8 whole vectors
// (C a multiple of 8). A workgroup of kClBlock threads gives lane t the channel vector
// t mod (C/8) for a whole job and the voxels t / (C/8) + r * vps, vps = kClBlock / (C/8);
// so C/8 must divide kClBlock. The lane's 8 channels lie in ngl = max(1, 8 / (C/G))
// groups, which needs C/G to divide 8 or to be a multiple of 8.
constexpr int kClBlock = 256;
// Reduction workgroups a channels-last launch aims for: one per CU. Each job ends in
// per-channel shuffle trees and three workgroup barriers, and its K partials per group feed
// the finalize. Measured on MI355X (bf16, fwd+bwd, plain loads and nontemporal stores):
// 256 jobs against 512, 128^3 x 32 channels 175.7 -> 172.3 us, 256^3 1357 -> 1354, 64^3 x 64
// 61.7 -> 61.4, 32^3 x 128 31.8 -> 31.2; 1024 slower at 128^3 and 256^3; 128 too few.
constexpr int64_t kClTargetJobs = 256;
constexpr int kClRounds = 4;        // voxel rounds a reduction lane holds per step
// Channels-last resident path: at most this many vectors of a group per voxel, at most this
// many (sample, channel) rows in a backward workgroup, and at most this many vectors per
// workgroup. A group's channels are 16-64 bytes of every voxel, C*2 bytes apart, so its
// loads are narrow; measured on MI355X (bf16, fwd+bwd): 8^3 x 512 channels, G=32 (1024
// vectors a group) 28 -> 18 us a step against the three-kernel path, while 16^3 x 256
// channels (4096 vectors) went 28 -> 72 us and a backward over 4 samples of 1024 vectors
// 29 -> 37 us.
constexpr int kClResMaxGroupVecs = 8;
constexpr int kClResMaxRows = 512;
constexpr int64_t kClResMaxVecs = 1024;
constexpr int kClApplyRounds = 2;   // voxel rounds of a streaming job (measured: 1, 4, 8 and 16 slower)

struct PlanCL {
    int64_t N = 0, C = 0, S = 0, G = 0;
    int64_t Cg = 0, M = 0;
    int64_t Cv = 0;      // vectors per voxel (C / 8)
    int64_t vps = 0;     // voxels per round of a workgroup (kClBlock / Cv)
    int ngl = 0;         // groups per lane vector: 1, 2, 4 or 8
    // reduction jobs: chunk voxels of one sample, K jobs per sample
    int64_t chunk = 0, K = 0, jobs = 0;
    // streaming jobs
    int64_t chunk_a = 0, K_a = 0, jobs_a = 0;
    // resident path (C/G a multiple of 8 with cvg = C/(8G) a power of two up to
    // kClResMaxGroupVecs): forward per group (n, g), backward per g across all samples
    bool res_fwd = false, res_bwd = false;
    int res_block_f = 0, res_vecs_f = 0;
    int res_block_b = 0, res_vecs_b = 0;
    int lcvg = 0;        // log2 of the group's vectors per voxel
    // workspace: [partials: float2 * jobs * C][group partials: float2 * jobs * G]
    // [per-channel: float2 * N*C][per-group: float4 * N*G]
    size_t ws_partg_offset = 0, ws_coefc_offset = 0, ws_coefg_offset = 0, ws_bytes = 0;
};

// Returns 0 and fills *p, else 2 (shape), 3 (groups) or 4 (shape not supported channels-last).
int make_plan_cl(int64_t N, int64_t C, int64_t S, int64_t G, PlanCL* p);

}  // namespace gn
